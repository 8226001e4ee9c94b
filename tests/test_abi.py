"""C-ABI boundary checks that run without a GPU: the library loads, exports
every symbol include/qlin.h declares, and rejects bad arguments from the host
before any launch (the calls below never reach a kernel: validation returns
first, so fake device addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlin.h")

Q = pytest.importorskip("quantized_linear_layers_token_amd")
L = Q.lib()

A = 0x10000000          # a fake, 256-byte aligned "device" address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlin_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) == 19, names
    for n in names:
        assert hasattr(L, n), f"{n} not exported by libqlin.so"
        assert n in Q.SIGNATURES, f"{n} has no binding signature"
    assert set(Q.SIGNATURES) == set(names)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define QLIN_ABI_VERSION (\d+)", text).group(1)) == Q.ABI_VERSION == L.qlin_abi_version()
    assert int(re.search(r"#define QLIN_MAX_K\s+(\d+)", text).group(1)) == Q.MAX_K
    enums = dict((k, int(v)) for k, v in re.findall(r"(QLIN_[A-Z0-9_]+) = (\d+)", text))
    assert enums["QLIN_OK"] == Q.QLIN_OK and enums["QLIN_ERR_ALIAS"] == Q.QLIN_ERR_ALIAS
    assert enums["QLIN_OUT_I32"] == Q.OUT_I32 and enums["QLIN_PATH_LARGE"] == Q.PATH_LARGE
    assert 127 * 128 * Q.MAX_K < 2 ** 31


def test_status_strings():
    for s in range(8):
        assert Q.status_string(s).startswith("QLIN_")
    assert Q.status_string(99) == "QLIN_ERR_UNKNOWN"
    assert L.qlin_last_hip_error() == 0


def quant_int8(x, M, K, q, s):
    return L.qlin_quant_act_int8(x, M, K, q, s, None)


def gemm(fn, qx, sx, qw, sw, y, M, N, K, out=0, path=0):
    return getattr(L, fn + "_ex")(qx, sx, qw, sw, y, M, N, K, out, path, None)


B = {"qx": A, "sx": A + 0x1000000, "qw": A + 0x2000000, "sw": A + 0x3000000, "y": A + 0x4000000}


def test_quant_validation():
    assert quant_int8(None, 0, 16, None, None) == Q.QLIN_OK                      # M == 0: no-op
    assert quant_int8(None, 4, 16, None, None) == Q.QLIN_ERR_NULL
    assert quant_int8(A, 4, 0, A + 4096, A + 8192) == Q.QLIN_ERR_SHAPE
    assert quant_int8(A, 4, 24, A + 4096, A + 8192) == Q.QLIN_ERR_SHAPE           # K % 16
    assert quant_int8(A, 4, Q.MAX_K + 16, A + 2 ** 22, A + 2 ** 23) == Q.QLIN_ERR_SHAPE
    assert quant_int8(A, -1, 16, A + 4096, A + 8192) == Q.QLIN_ERR_SHAPE
    assert quant_int8(A + 8, 4, 16, A + 4096, A + 8192) == Q.QLIN_ERR_ALIGN
    assert quant_int8(A, 4, 16, A + 4096 + 4, A + 8192) == Q.QLIN_ERR_ALIGN
    assert quant_int8(A, 4, 16, A + 4096, A + 8192 + 2) == Q.QLIN_ERR_ALIGN
    assert quant_int8(A, 4, 16, A + 64, A + 8192) == Q.QLIN_ERR_ALIAS            # q inside x (128 bytes)
    assert quant_int8(A, 4, 16, A + 4096, A + 4096 + 32) == Q.QLIN_ERR_ALIAS     # s inside q
    f8 = L.qlin_quant_act_fp8
    assert f8(A, 4, 16, 64, A + 4096, A + 8192, None) == Q.QLIN_ERR_SHAPE          # group must be 0 / 128
    assert f8(A, 4, 144, 128, A + 4096, A + 8192, None) == Q.QLIN_ERR_SHAPE        # K % 128 for groups
    assert f8(None, 0, 128, 128, None, None, None) == Q.QLIN_OK


@pytest.mark.parametrize("fn", ["qlin_gemm_w8a8", "qlin_gemm_fp8_rowwise", "qlin_gemm_fp8_block"])
def test_product_validation(fn):
    b = B
    args = (b["qx"], b["sx"], b["qw"], b["sw"], b["y"])
    assert gemm(fn, *args, 0, 256, 256) == Q.QLIN_OK                     # M == 0
    assert gemm(fn, *args, 4, 0, 256) == Q.QLIN_OK                       # N == 0
    assert gemm(fn, None, *args[1:], 4, 256, 256) == Q.QLIN_ERR_NULL
    assert gemm(fn, *args[:4], None, 4, 256, 256) == Q.QLIN_ERR_NULL
    assert gemm(fn, *args, 4, 256, 0) == Q.QLIN_ERR_SHAPE
    assert gemm(fn, *args, 4, 256, 40) == Q.QLIN_ERR_SHAPE
    assert gemm(fn, *args, 4, -256, 256) == Q.QLIN_ERR_SHAPE
    assert gemm(fn, b["qx"] + 8, *args[1:], 4, 256, 256) == Q.QLIN_ERR_ALIGN
    assert gemm(fn, *args[:2], b["qw"] + 4, *args[3:], 4, 256, 256) == Q.QLIN_ERR_ALIGN
    assert gemm(fn, *args[:4], b["y"] + 2, 4, 256, 256) == Q.QLIN_ERR_ALIGN
    assert gemm(fn, *args[:3], b["sw"] + 1, b["y"], 4, 256, 256) == Q.QLIN_ERR_ALIGN
    assert gemm(fn, *args, 4, 256, 256, out=7) == Q.QLIN_ERR_UNSUPPORTED
    assert gemm(fn, *args, 4, 256, 256, path=12) == Q.QLIN_ERR_UNSUPPORTED
    if fn == "qlin_gemm_fp8_block":
        assert gemm(fn, *args, 4, 256, 256, path=Q.PATH_LARGE_256X256_W8) == Q.QLIN_ERR_UNSUPPORTED
        assert gemm(fn, *args, 4, 256, 256, path=Q.PATH_LARGE_256X256) == Q.QLIN_ERR_UNSUPPORTED
    assert gemm(fn, *args, 4, 256, 256, path=-1) == Q.QLIN_ERR_UNSUPPORTED
    assert gemm(fn, *args, 2, 256, 256, path=Q.PATH_GEMV) == Q.QLIN_ERR_UNSUPPORTED
    assert gemm(fn, *args, 33, 256, 256, path=Q.PATH_SMALL) == Q.QLIN_ERR_UNSUPPORTED
    assert gemm(fn, *args[:4], b["qw"] + 256, 4, 256, 256) == Q.QLIN_ERR_ALIAS    # y overlaps q_w
    if fn == "qlin_gemm_w8a8":
        pass
    else:
        assert gemm(fn, *args, 4, 256, 256, out=Q.OUT_I32) == Q.QLIN_ERR_UNSUPPORTED
    if fn == "qlin_gemm_fp8_block":
        assert gemm(fn, *args, 4, 200, 256) == Q.QLIN_ERR_SHAPE           # N % 128
        assert gemm(fn, *args, 4, 256, 272) == Q.QLIN_ERR_SHAPE           # K % 128


def test_gemv_validation():
    b = B
    g = L.qlin_gemv_w8a8
    assert g(b["qx"], b["sx"], b["qw"], b["sw"], b["y"], 0, 256, 0, None) == Q.QLIN_OK
    assert g(None, b["sx"], b["qw"], b["sw"], b["y"], 16, 256, 0, None) == Q.QLIN_ERR_NULL
    assert g(b["qx"], b["sx"], b["qw"], b["sw"], b["y"], 16, 100, 0, None) == Q.QLIN_ERR_SHAPE
    assert g(b["qx"], b["sx"], b["qw"], b["sw"], b["y"], 16, 256, 5, None) == Q.QLIN_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    # The package's loader raises when the shared library is absent (no fallback).
    import importlib.util
    src = os.path.join(ROOT, "quantized_linear_layers_token_amd", "__init__.py")
    pkg = tmp_path / "qlin_copy"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("qlin_copy", str(pkg / "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="no fallback"):
        spec.loader.exec_module(mod)


def test_ctypes_handle_is_shared():
    assert isinstance(L, ctypes.CDLL)


def test_linear_validation():
    Seg = Q.QlinSegment
    x = A
    segs = (Seg * 3)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 64),
                     Seg(A + 0x4000000, A + 0x5000000, A + 0x6000000, 64),
                     Seg(A + 0x7000000, A + 0x8000000, A + 0x9000000, 128))
    lin = L.qlin_linear
    assert lin(0, x, 1, 256, None, 1, 0, None, None, None) == Q.QLIN_ERR_NULL
    assert lin(0, x, 1, 256, segs, 0, 0, None, None, None) == Q.QLIN_ERR_SHAPE
    assert lin(0, x, 1, 256, segs, 5, 0, None, None, None) == Q.QLIN_ERR_SHAPE
    assert lin(9, x, 1, 256, segs, 3, 0, None, None, None) == Q.QLIN_ERR_UNSUPPORTED
    assert lin(1, x, 1, 256, segs, 3, Q.OUT_I32, None, None, None) == Q.QLIN_ERR_UNSUPPORTED
    assert lin(2, x, 1, 256, segs, 3, 0, None, None, None) == Q.QLIN_ERR_SHAPE       # block: n % 128
    assert lin(0, x, 0, 256, segs, 3, 0, None, None, None) == Q.QLIN_OK              # M == 0
    assert lin(0, x, 1, 250, segs, 3, 0, None, None, None) == Q.QLIN_ERR_SHAPE
    assert lin(0, None, 1, 256, segs, 3, 0, None, None, None) == Q.QLIN_ERR_NULL
    assert lin(0, x, 5, 256, segs, 3, 0, None, None, None) == Q.QLIN_ERR_NULL         # M > 4 needs staging
    assert lin(0, x, 2, 16400, segs, 3, 0, None, None, None) == Q.QLIN_ERR_NULL       # so do 2 long tokens
    assert lin(0, x, 4, 256, segs, 3, 0, A + 0xA000000, None, None) == Q.QLIN_ERR_NULL
    assert lin(0, x + 8, 1, 256, segs, 3, 0, None, None, None) == Q.QLIN_ERR_ALIGN
    bad = (Seg * 2)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 64),
                    Seg(A + 0x4000000, A + 0x5000000, A + 0x3000000 + 64, 64))    # outputs overlap
    assert lin(0, x, 1, 256, bad, 2, 0, None, None, None) == Q.QLIN_ERR_ALIAS
    bad2 = (Seg * 1)(Seg(A + 0x1000000, A + 0x2000000, A + 0x1000000 + 512, 64))  # y inside q_w
    assert lin(0, x, 1, 256, bad2, 1, 0, None, None, None) == Q.QLIN_ERR_ALIAS
    nul = (Seg * 1)(Seg(None, A + 0x2000000, A + 0x3000000, 64))
    assert lin(0, x, 1, 256, nul, 1, 0, None, None, None) == Q.QLIN_ERR_NULL
    empty = (Seg * 1)(Seg(None, None, None, 0))
    assert lin(0, x, 1, 256, empty, 1, 0, None, None, None) == Q.QLIN_OK             # no rows: no-op
    # staging buffers overlapping a segment's weights or weight scales
    one = (Seg * 1)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 64))
    sx_ok, qx_ok = A + 0xB000000, A + 0xA000000
    assert lin(0, x, 8, 256, one, 1, 0, A + 0x1000000 + 4096, sx_ok, None) == Q.QLIN_ERR_ALIAS   # q_x in q_w
    assert lin(0, x, 8, 256, one, 1, 0, A + 0x2000000 - 1024, sx_ok, None) == Q.QLIN_ERR_ALIAS   # q_x over s_w
    assert lin(0, x, 8, 256, one, 1, 0, qx_ok, A + 0x1000000 + 64, None) == Q.QLIN_ERR_ALIAS     # s_x in q_w
    assert lin(0, x, 8, 256, one, 1, 0, qx_ok, A + 0x2000000 + 4, None) == Q.QLIN_ERR_ALIAS      # s_x in s_w


def test_linear_weight_only_validation():
    Seg = Q.QlinSegment
    x = A
    segs = (Seg * 2)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 128),
                     Seg(A + 0x4000000, A + 0x5000000, A + 0x6000000, 128))
    wo = L.qlin_linear_weight_only
    assert wo(0, x, 1, 256, None, 1, 0, None) == Q.QLIN_ERR_NULL
    assert wo(0, x, 1, 256, segs, 0, 0, None) == Q.QLIN_ERR_SHAPE
    assert wo(9, x, 1, 256, segs, 2, 0, None) == Q.QLIN_ERR_UNSUPPORTED
    assert wo(0, x, 1, 256, segs, 2, Q.OUT_I32, None) == Q.QLIN_ERR_UNSUPPORTED   # no integer accumulator here
    assert wo(0, x, 33, 256, segs, 2, 0, None) == Q.QLIN_ERR_UNSUPPORTED          # at most 32 tokens
    assert wo(2, x, 1, 200, segs, 2, 0, None) == Q.QLIN_ERR_SHAPE                 # block: K % 128
    assert wo(0, x, 0, 256, segs, 2, 0, None) == Q.QLIN_OK                        # M == 0
    assert wo(0, None, 1, 256, segs, 2, 0, None) == Q.QLIN_ERR_NULL
    assert wo(0, x + 8, 1, 256, segs, 2, 0, None) == Q.QLIN_ERR_ALIGN
    bad = (Seg * 1)(Seg(A + 0x1000000, A + 0x2000000, x + 64, 128))             # y overlaps x
    assert wo(0, x, 4, 256, bad, 1, 0, None) == Q.QLIN_ERR_ALIAS


def test_linear_swiglu_validation():
    sg = L.qlin_linear_swiglu
    x, gq, gs, uq, us, h = A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000
    qx, sx = A + 0x6000000, A + 0x7000000
    assert sg(9, x, 1, 256, gq, gs, uq, us, 128, h, None, None, None) == Q.QLIN_ERR_UNSUPPORTED
    assert sg(0, x, 0, 256, gq, gs, uq, us, 128, h, None, None, None) == Q.QLIN_OK       # M == 0
    assert sg(0, x, 1, 256, gq, gs, uq, us, 0, h, None, None, None) == Q.QLIN_OK         # I == 0
    assert sg(0, x, 1, 250, gq, gs, uq, us, 128, h, None, None, None) == Q.QLIN_ERR_SHAPE
    assert sg(2, x, 1, 256, gq, gs, uq, us, 64, h, None, None, None) == Q.QLIN_ERR_SHAPE  # block: I % 128
    assert sg(0, x, 1, 256, None, gs, uq, us, 128, h, None, None, None) == Q.QLIN_ERR_NULL
    assert sg(0, x, 1, 256, gq, gs, None, us, 128, h, None, None, None) == Q.QLIN_ERR_NULL
    assert sg(0, x, 1, 256, gq, gs, uq, us, 128, None, None, None, None) == Q.QLIN_ERR_NULL
    assert sg(0, x, 5, 256, gq, gs, uq, us, 128, h, None, None, None) == Q.QLIN_ERR_NULL  # M > 4 needs staging
    assert sg(0, x, 1, 256, gq, gs, uq, us, 128, h + 8, None, None, None) == Q.QLIN_ERR_ALIGN
    assert sg(0, x, 1, 256, gq, gs, uq + 8, us, 128, h, None, None, None) == Q.QLIN_ERR_ALIGN
    assert sg(0, x, 1, 256, gq, gs, uq, us, 128, uq + 256, None, None, None) == Q.QLIN_ERR_ALIAS  # h in up
    assert sg(0, x, 1, 256, gq, gs, uq, us, 128, gs, None, None, None) == Q.QLIN_ERR_ALIAS        # h on gate scales
    assert sg(0, x, 4, 256, gq, gs, uq, us, 128, qx, qx, sx, None) == Q.QLIN_ERR_ALIAS            # h on staging


def test_pack_weights_validation():
    pk = L.qlin_pack_weights
    w, p = A, A + 0x1000000
    assert pk(9, w, 256, 384, p, None) == Q.QLIN_ERR_UNSUPPORTED
    assert pk(0, w, 200, 384, p, None) == Q.QLIN_ERR_SHAPE            # N % 128
    assert pk(1, w, 256, 400, p, None) == Q.QLIN_ERR_SHAPE            # K % 128
    assert pk(0, w, -128, 384, p, None) == Q.QLIN_ERR_SHAPE
    assert pk(0, w, 0, 384, p, None) == Q.QLIN_OK                     # no rows: no-op
    assert pk(0, None, 256, 384, p, None) == Q.QLIN_ERR_NULL
    assert pk(0, w, 256, 384, None, None) == Q.QLIN_ERR_NULL
    assert pk(0, w + 8, 256, 384, p, None) == Q.QLIN_ERR_ALIGN
    assert pk(0, w, 256, 384, w + 256 * 384 - 16, None) == Q.QLIN_ERR_ALIAS


def test_linear_packed_validation():
    Seg = Q.QlinSegment
    x, qx, sx = A, A + 0xA000000, A + 0xB000000
    segs = (Seg * 2)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 128),
                     Seg(A + 0x4000000, A + 0x5000000, A + 0x6000000, 256))
    odd = (Seg * 1)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 64))
    lp = L.qlin_linear_packed
    assert lp(9, x, 64, 256, segs, 2, 0, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED   # unknown scheme
    assert lp(2, x, 64, 256, segs, 2, Q.OUT_I32, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED
    assert lp(0, x, 32, 256, segs, 2, 0, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED   # M <= 32: row-major kernels
    assert lp(0, x, 64, 256, odd, 1, 0, qx, sx, None) == Q.QLIN_ERR_SHAPE          # n % 128
    assert lp(0, x, 64, 272, segs, 2, 0, qx, sx, None) == Q.QLIN_ERR_SHAPE         # K % 128
    assert lp(0, x, 64, 256, segs, 2, 0, None, None, None) == Q.QLIN_ERR_NULL      # staging required
    assert lp(1, x, 64, 256, segs, 2, Q.OUT_I32, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED
    assert lp(0, x, 0, 256, segs, 2, 0, qx, sx, None) == Q.QLIN_OK                 # M == 0
    assert lp(0, x, 64, 256, segs, 2, 0, A + 0x1000000 + 64, sx, None) == Q.QLIN_ERR_ALIAS   # q_x in q_w


def test_linear_swiglu_packed_validation():
    sg = L.qlin_linear_swiglu_packed
    x, gq, gs, uq, us, h = A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, A + 0x5000000
    qx, sx = A + 0x6000000, A + 0x7000000
    assert sg(9, x, 64, 256, gq, gs, uq, us, 128, h, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED
    assert sg(0, x, 0, 256, gq, gs, uq, us, 128, h, qx, sx, None) == Q.QLIN_OK         # M == 0
    assert sg(0, x, 64, 256, gq, gs, uq, us, 0, h, qx, sx, None) == Q.QLIN_OK          # I == 0
    assert sg(0, x, 32, 256, gq, gs, uq, us, 128, h, qx, sx, None) == Q.QLIN_ERR_UNSUPPORTED   # M <= 32
    assert sg(0, x, 64, 256, gq, gs, uq, us, 64, h, qx, sx, None) == Q.QLIN_ERR_SHAPE   # I % 128
    assert sg(1, x, 64, 272, gq, gs, uq, us, 128, h, qx, sx, None) == Q.QLIN_ERR_SHAPE  # K % 128
    assert sg(0, x, 64, 256, gq, gs, uq, us, 128, h, None, None, None) == Q.QLIN_ERR_NULL   # staging required
    assert sg(0, x, 64, 256, None, gs, uq, us, 128, h, qx, sx, None) == Q.QLIN_ERR_NULL
    assert sg(0, x, 64, 256, gq, gs, uq, us, 128, uq + 256, qx, sx, None) == Q.QLIN_ERR_ALIAS   # h in up


def test_library_has_no_unresolved_internal_symbols():
    # a kernel whose device code failed to emit leaves its host launch stub
    # undefined; the loader only notices at the first call
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", Q.LIB_PATH], capture_output=True, text=True).stdout
    bad = [ln for ln in out.splitlines() if "qlin" in ln]
    assert not bad, bad


def test_linear_noalloc_refuses_calls_past_its_scratch():
    # refused before any launch (fake addresses, never dereferenced)
    Seg = Q.QlinSegment
    segs = (Seg * 1)(Seg(A + 0x1000000, A + 0x2000000, A + 0x3000000, 128))
    na = L.qlin_linear_noalloc
    K = 4096
    M = Q.NOALLOC_MAX_CODE_BYTES // K + 1                        # one token too many
    assert na(0, A, M, K, segs, 1, 0, None) == Q.QLIN_ERR_TOO_LARGE
    assert na(2, A, 1 << 20 + 1, 128, segs, 1, 0, None) == Q.QLIN_ERR_TOO_LARGE   # too many scales
    assert na(0, A, 0, K, segs, 1, 0, None) == Q.QLIN_OK                           # M == 0
    assert na(0, None, 8, K, segs, 1, 0, None) == Q.QLIN_ERR_NULL                  # qlin_linear's validation
    assert na(0, A, 8, 250, segs, 1, 0, None) == Q.QLIN_ERR_SHAPE
    assert na(0, A, 1, 256, None, 1, 0, None) == Q.QLIN_ERR_NULL
    assert "scratch" in Q.status_string(Q.QLIN_ERR_TOO_LARGE)
