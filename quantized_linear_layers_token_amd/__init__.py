"""Python binding of libqlin.so (quantized decoder projections on MI355X).

Argument marshalling only: every function below forwards device pointers,
sizes and the current HIP stream to the C ABI declared in include/qlin.h and
raises QlinError on a non-OK status.  torch supplies memory and streams; no
computation happens here.  If the library is not built, importing this package
fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqlin.so")

(QLIN_OK, QLIN_ERR_NULL, QLIN_ERR_SHAPE, QLIN_ERR_ALIGN, QLIN_ERR_UNSUPPORTED, QLIN_ERR_HIP, QLIN_ERR_ALIAS,
 QLIN_ERR_TOO_LARGE) = range(8)
OUT_BF16, OUT_I32, OUT_F32 = 0, 1, 2
SCHEME_W8A8, SCHEME_FP8_ROWWISE, SCHEME_FP8_BLOCK = 0, 1, 2
MAX_SEGMENTS = 4
PATH_AUTO, PATH_GEMV, PATH_SMALL, PATH_LARGE = 0, 1, 2, 3
# the tiled GEMM with a fixed output tile (weight rows x tokens)
PATH_LARGE_256X128, PATH_LARGE_128X128, PATH_LARGE_128X64, PATH_LARGE_128X256 = 4, 5, 6, 7
PATH_LARGE_128X128_K2, PATH_LARGE_128X64_K2 = 8, 9
PATH_LARGE_256X256_W8 = 10   # int8 and FP8 rowwise only
PATH_LARGE_256X256 = 11      # int8 and FP8 rowwise only
ABI_VERSION = 3
NOALLOC_MAX_CODE_BYTES = 16 << 20    # staging capacity of qlin_linear_noalloc
NOALLOC_MAX_SCALES = 1 << 20
MAX_K = 131072

# Exported symbols and their C signatures (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_S = ctypes.c_int
SIGNATURES = {
    "qlin_quant_act_int8": (_S, [_P, _I64, _I64, _P, _P, _P]),
    "qlin_quant_act_fp8": (_S, [_P, _I64, _I64, _I32, _P, _P, _P]),
    "qlin_gemv_w8a8": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _S, _P]),
    "qlin_gemm_w8a8": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _P]),
    "qlin_gemm_w8a8_ex": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _S, _P]),
    "qlin_gemm_fp8_rowwise": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _P]),
    "qlin_gemm_fp8_rowwise_ex": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _S, _P]),
    "qlin_gemm_fp8_block": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _P]),
    "qlin_gemm_fp8_block_ex": (_S, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _S, _S, _P]),
    "qlin_linear": (_S, [_S, _P, _I64, _I64, _P, _I32, _S, _P, _P, _P]),
    "qlin_linear_weight_only": (_S, [_S, _P, _I64, _I64, _P, _I32, _S, _P]),
    "qlin_linear_swiglu": (_S, [_S, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P, _P, _P, _P]),
    "qlin_linear_noalloc": (_S, [_S, _P, _I64, _I64, _P, _I32, _S, _P]),
    "qlin_pack_weights": (_S, [_S, _P, _I64, _I64, _P, _P]),
    "qlin_linear_packed": (_S, [_S, _P, _I64, _I64, _P, _I32, _S, _P, _P, _P]),
    "qlin_linear_swiglu_packed": (_S, [_S, _P, _I64, _I64, _P, _P, _P, _P, _I64, _P, _P, _P, _P]),
    "qlin_status_string": (ctypes.c_char_p, [_S]),
    "qlin_abi_version": (_S, []),
    "qlin_last_hip_error": (_S, []),
}


class QlinSegment(ctypes.Structure):
    """struct qlin_segment: one weight matrix reading the call's activations."""
    _fields_ = [("q_w", ctypes.c_void_p), ("s_w", ctypes.c_void_p), ("y", ctypes.c_void_p), ("n", ctypes.c_int64)]


class QlinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.qlin_status_string(status).decode() if _lib is not None else str(status)
        if status == QLIN_ERR_HIP:
            msg += f" (hip error {_lib.qlin_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def _load():
    # torch is imported first so that libqlin.so binds (by soname) to the HIP
    # runtime torch already loaded: one runtime per process, shared streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python quantized_linear_layers_token_amd/build.py` "
            "(the HIP library is the only implementation; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.qlin_abi_version() != ABI_VERSION:
        raise ImportError(f"libqlin ABI {lib.qlin_abi_version()} != binding ABI {ABI_VERSION}")
    return lib


_lib = _load()


def lib():
    """The raw ctypes handle of libqlin.so."""
    return _lib


def _check(status: int, where: str):
    if status != QLIN_OK:
        raise QlinError(status, where)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dims2(t, name, elem=None):
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 2-D tensor")
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name} must have {elem}-byte elements, not {t.element_size()}")
    return t.shape[0], t.shape[1]


def _out_bytes(out):
    return 2 if out == OUT_BF16 else 4


def _args(*items):
    """Checks every tensor argument before its address reaches the library,
    which sees only pointers: (name, tensor, bytes the call reads or writes,
    required element size or None).  A tensor must be contiguous and hold at
    least that many bytes, and all of them must be device tensors.  Optional
    arguments (None) are left to the library, which returns QLIN_ERR_NULL
    where one is required."""
    given = [(n, t, b, e) for n, t, b, e in items if t is not None]
    for name, t, nbytes, elem in given:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if elem is not None and t.element_size() != elem:
            raise ValueError(f"{name} must have {elem}-byte elements, not {t.element_size()}")
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{name} holds {have} bytes; the call accesses {nbytes}")
    for name, t, _, _ in given:
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def _sx_count(scheme_block, M, K):
    return M * (K // 128) if scheme_block else M


def _sw_count(scheme_block, N, K):
    return (N // 128) * (K // 128) if scheme_block else N


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def qlin_quant_act_int8(x, q, s, stream=None):
    """x: bf16 (or int16 bit patterns) [M, K]; q: int8 [M, K]; s: f32 [M]."""
    M, K = _dims2(x, "x", 2)
    _args(("q", q, M * K, 1), ("s", s, 4 * M, 4), ("x", x, 0, None))
    _check(_lib.qlin_quant_act_int8(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(stream)), "qlin_quant_act_int8")


def qlin_quant_act_fp8(x, q, s, group=0, stream=None):
    """x: bf16 [M, K]; q: uint8 E4M3 codes [M, K]; s: f32 [M] (group 0) or [M, K/128] (group 128)."""
    M, K = _dims2(x, "x", 2)
    _args(("q", q, M * K, 1), ("s", s, 4 * _sx_count(group == 128, M, K), 4), ("x", x, 0, None))
    _check(_lib.qlin_quant_act_fp8(_ptr(x), M, K, group, _ptr(q), _ptr(s), _stream(stream)), "qlin_quant_act_fp8")


# --------------------------------------------------------------------------
# Products
# --------------------------------------------------------------------------

def qlin_gemv_w8a8(q_x, s_x, q_w, s_w, y, out=OUT_BF16, stream=None):
    """q_x int8 [K] or [1, K]; s_x f32 [1]; q_w int8 [N, K]; s_w bf16 [N]; y [N] or [1, N]."""
    N, K = _dims2(q_w, "q_w", 1)
    _args(("q_x", q_x, K, 1), ("s_x", s_x, 4, 4), ("s_w", s_w, 2 * N, 2), ("y", y, N * _out_bytes(out), None),
          ("q_w", q_w, 0, None))
    _check(_lib.qlin_gemv_w8a8(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), _ptr(y), N, K, out, _stream(stream)),
           "qlin_gemv_w8a8")


def _mnk(q_x, q_w, s_x, s_w, y, out, block=False):
    M, K = _dims2(q_x, "q_x", 1)
    N, K2 = _dims2(q_w, "q_w", 1)
    if K != K2:
        raise ValueError(f"K mismatch: q_x has {K}, q_w has {K2}")
    _args(("s_x", s_x, 4 * _sx_count(block, M, K), 4), ("s_w", s_w, 2 * _sw_count(block, N, K), 2),
          ("y", y, M * N * _out_bytes(out), None), ("q_x", q_x, 0, None), ("q_w", q_w, 0, None))
    return M, N, K


def qlin_gemm_w8a8(q_x, s_x, q_w, s_w, y, out=OUT_BF16, path=PATH_AUTO, stream=None):
    """q_x int8 [M, K]; s_x f32 [M]; q_w int8 [N, K]; s_w bf16 [N]; y [M, N] (bf16 / i32 / f32)."""
    M, N, K = _mnk(q_x, q_w, s_x, s_w, y, out)
    _check(_lib.qlin_gemm_w8a8_ex(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), _ptr(y), M, N, K, out, path,
                                  _stream(stream)), "qlin_gemm_w8a8")


def qlin_gemm_fp8_rowwise(q_x, s_x, q_w, s_w, y, out=OUT_BF16, path=PATH_AUTO, stream=None):
    """q_x uint8 E4M3 [M, K]; s_x f32 [M]; q_w uint8 E4M3 [N, K]; s_w bf16 [N]; y [M, N]."""
    M, N, K = _mnk(q_x, q_w, s_x, s_w, y, out)
    _check(_lib.qlin_gemm_fp8_rowwise_ex(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), _ptr(y), M, N, K, out, path,
                                         _stream(stream)), "qlin_gemm_fp8_rowwise")


def qlin_gemm_fp8_block(q_x, s_x, q_w, s_w, y, out=OUT_BF16, path=PATH_AUTO, stream=None):
    """q_x uint8 E4M3 [M, K]; s_x f32 [M, K/128]; q_w uint8 E4M3 [N, K]; s_w bf16 [N/128, K/128]; y [M, N]."""
    M, N, K = _mnk(q_x, q_w, s_x, s_w, y, out, block=True)
    _check(_lib.qlin_gemm_fp8_block_ex(_ptr(q_x), _ptr(s_x), _ptr(q_w), _ptr(s_w), _ptr(y), M, N, K, out, path,
                                       _stream(stream)), "qlin_gemm_fp8_block")


def status_string(status: int) -> str:
    return _lib.qlin_status_string(status).decode()


# --------------------------------------------------------------------------
# Fused projection (bf16 activations in)
# --------------------------------------------------------------------------

def _segment_args(scheme, M, K, segments, out):
    """The _args items of the segments' tensors (shapes checked here)."""
    block = scheme == SCHEME_FP8_BLOCK
    items = []
    for i, (qw, sw, y) in enumerate(segments):
        n, k2 = _dims2(qw, f"segment {i} q_w", 1)
        if k2 != K:
            raise ValueError("every q_w must be [n, K]")
        items += [(f"segment {i} s_w", sw, 2 * _sw_count(block, n, K), 2),
                  (f"segment {i} y", y, M * n * _out_bytes(out), None), (f"segment {i} q_w", qw, 0, None)]
    return items


def segments_array(segments):
    """[(q_w [n, K], s_w, y), ...] -> ctypes array of QlinSegment."""
    arr = (QlinSegment * len(segments))()
    for i, (qw, sw, y) in enumerate(segments):
        arr[i] = QlinSegment(_ptr(qw), _ptr(sw), _ptr(y), qw.shape[0])
    return arr


def qlin_linear(scheme, x, segments, out=OUT_BF16, q_x=None, s_x=None, stream=None):
    """x bf16 [M, K]; segments: list of (q_w [n, K], s_w, y [M, n]) sharing x.
    q_x / s_x: staging for the quantized activations (optional where one launch
    does the whole call: M == 1, the two-token form, or M <= 4 with K <= 4096)."""
    M, K = _dims2(x, "x", 2)
    block = scheme == SCHEME_FP8_BLOCK
    _args(*_segment_args(scheme, M, K, segments, out), ("q_x", q_x, M * K, 1),
          ("s_x", s_x, 4 * _sx_count(block, M, K), 4), ("x", x, 0, None))
    arr = segments_array(segments)
    _check(_lib.qlin_linear(scheme, _ptr(x), M, K, arr, len(segments), out, _ptr(q_x), _ptr(s_x),
                            _stream(stream)), "qlin_linear")


def qlin_pack_weights(scheme, q_w, q_w_packed, stream=None):
    """Reorders q_w [N, K] (1-byte codes, row-major) into the matrix-core
    operand order of qlin_linear_packed, written to q_w_packed (N * K bytes,
    e.g. a tensor like q_w).  Any scheme; N and K multiples of 128."""
    N, K = _dims2(q_w, "q_w", 1)
    _args(("q_w_packed", q_w_packed, N * K, 1), ("q_w", q_w, 0, None))
    _check(_lib.qlin_pack_weights(scheme, _ptr(q_w), N, K, _ptr(q_w_packed), _stream(stream)), "qlin_pack_weights")


def qlin_linear_packed(scheme, x, segments, out=OUT_BF16, q_x=None, s_x=None, stream=None):
    """qlin_linear for M >= 33 with every segment's q_w [n, K] in the packed
    order that qlin_pack_weights writes (s_w and y as for qlin_linear);
    q_x / s_x staging required (s_x [M, K/128] for the block scheme)."""
    M, K = _dims2(x, "x", 2)
    _args(*_segment_args(scheme, M, K, segments, out), ("q_x", q_x, M * K, 1),
          ("s_x", s_x, 4 * _sx_count(scheme == SCHEME_FP8_BLOCK, M, K), 4), ("x", x, 0, None))
    arr = segments_array(segments)
    _check(_lib.qlin_linear_packed(scheme, _ptr(x), M, K, arr, len(segments), out, _ptr(q_x), _ptr(s_x),
                                   _stream(stream)), "qlin_linear_packed")


def qlin_linear_swiglu_packed(scheme, x, gate, up, h, q_x=None, s_x=None, stream=None):
    """qlin_linear_swiglu for M >= 33 with gate and up as (packed q_w [I, K],
    s_w) pairs from qlin_pack_weights; q_x / s_x staging required."""
    M, K = _dims2(x, "x", 2)
    (gq, gs), (uq, us) = gate, up
    if gq.dim() != 2 or gq.shape[1] != K or tuple(uq.shape) != tuple(gq.shape):
        raise ValueError("gate and up q_w must both be [I, K]")
    I = gq.shape[0]
    block = scheme == SCHEME_FP8_BLOCK
    _args(("gate q_w", gq, I * K, 1), ("up q_w", uq, I * K, 1), ("gate s_w", gs, 2 * _sw_count(block, I, K), 2),
          ("up s_w", us, 2 * _sw_count(block, I, K), 2), ("h", h, 2 * M * I, None), ("q_x", q_x, M * K, 1),
          ("s_x", s_x, 4 * _sx_count(block, M, K), 4), ("x", x, 0, None))
    _check(_lib.qlin_linear_swiglu_packed(scheme, _ptr(x), M, K, _ptr(gq), _ptr(gs), _ptr(uq), _ptr(us), I, _ptr(h),
                                          _ptr(q_x), _ptr(s_x), _stream(stream)), "qlin_linear_swiglu_packed")


def qlin_linear_noalloc(scheme, x, segments, out=OUT_BF16, stream=None):
    """qlin_linear with the library's fixed scratch as staging (no q_x / s_x):
    for callers that cannot allocate.  Calls that may overlap on one GPU race
    on the scratch."""
    M, K = _dims2(x, "x", 2)
    _args(*_segment_args(scheme, M, K, segments, out), ("x", x, 0, None))
    arr = segments_array(segments)
    _check(_lib.qlin_linear_noalloc(scheme, _ptr(x), M, K, arr, len(segments), out, _stream(stream)),
           "qlin_linear_noalloc")


def qlin_linear_weight_only(scheme, x, segments, out=OUT_BF16, stream=None):
    """Weight-only numerics: x bf16 [M, K] (M <= 32) times the dequantized
    weights of each segment (q_w [n, K], s_w, y [M, n]); the input is not rounded."""
    M, K = _dims2(x, "x", 2)
    _args(*_segment_args(scheme, M, K, segments, out), ("x", x, 0, None))
    arr = segments_array(segments)
    _check(_lib.qlin_linear_weight_only(scheme, _ptr(x), M, K, arr, len(segments), out, _stream(stream)),
           "qlin_linear_weight_only")


def qlin_linear_swiglu(scheme, x, gate, up, h, q_x=None, s_x=None, stream=None):
    """x bf16 [M, K]; gate, up: (q_w [I, K], s_w) of one gated MLP; h bf16
    [M, I] receives silu(gate projection) * (up projection), each rounded as
    the header states.  q_x / s_x: staging for the quantized activations
    (optional at M == 1)."""
    M, K = _dims2(x, "x", 2)
    (gq, gs), (uq, us) = gate, up
    if gq.dim() != 2 or gq.shape[1] != K or tuple(uq.shape) != tuple(gq.shape):
        raise ValueError("gate and up q_w must both be [I, K]")
    I = gq.shape[0]
    block = scheme == SCHEME_FP8_BLOCK
    _args(("gate q_w", gq, I * K, 1), ("up q_w", uq, I * K, 1), ("gate s_w", gs, 2 * _sw_count(block, I, K), 2),
          ("up s_w", us, 2 * _sw_count(block, I, K), 2), ("h", h, 2 * M * I, None), ("q_x", q_x, M * K, 1),
          ("s_x", s_x, 4 * _sx_count(block, M, K), 4), ("x", x, 0, None))
    _check(_lib.qlin_linear_swiglu(scheme, _ptr(x), M, K, _ptr(gq), _ptr(gs), _ptr(uq), _ptr(us), gq.shape[0],
                                   _ptr(h), _ptr(q_x), _ptr(s_x), _stream(stream)), "qlin_linear_swiglu")
