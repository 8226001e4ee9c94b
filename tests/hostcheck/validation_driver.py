"""Drives the C-ABI validation layer built for the host with AddressSanitizer
and UndefinedBehaviorSanitizer (qlin_api.hip + the stub launchers beside this
file), without a GPU and without torch.  Run in a child process whose
LD_PRELOAD starts with the ASan runtime; any sanitizer report ends it with a
non-zero status.  Argument: the path of the sanitized library.

Checks: boundary cases with known statuses, then a seeded random sweep of
every entry point (sizes from 0 to past the limits, odd alignments, null and
overlapping pointers, 0..5 segments).  For every call: the status is a
defined one, and a call that returns an error has launched nothing."""
import ctypes
import random
import sys

lib = ctypes.CDLL(sys.argv[1])
P, I64, I32, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int


class Seg(ctypes.Structure):
    _fields_ = [("q_w", P), ("s_w", P), ("y", P), ("n", I64)]


SIG = {
    "qlin_quant_act_int8": [P, I64, I64, P, P, P],
    "qlin_quant_act_fp8": [P, I64, I64, I32, P, P, P],
    "qlin_gemv_w8a8": [P, P, P, P, P, I64, I64, S, P],
    "qlin_gemm_w8a8_ex": [P, P, P, P, P, I64, I64, I64, S, S, P],
    "qlin_gemm_fp8_rowwise_ex": [P, P, P, P, P, I64, I64, I64, S, S, P],
    "qlin_gemm_fp8_block_ex": [P, P, P, P, P, I64, I64, I64, S, S, P],
    "qlin_linear": [S, P, I64, I64, P, I32, S, P, P, P],
    "qlin_linear_packed": [S, P, I64, I64, P, I32, S, P, P, P],
    "qlin_pack_weights": [S, P, I64, I64, P, P],
    "qlin_linear_swiglu_packed": [S, P, I64, I64, P, P, P, P, I64, P, P, P, P],
    "qlin_linear_weight_only": [S, P, I64, I64, P, I32, S, P],
    "qlin_linear_swiglu": [S, P, I64, I64, P, P, P, P, I64, P, P, P, P],
}
for name, args in SIG.items():
    getattr(lib, name).restype = S
    getattr(lib, name).argtypes = args
lib.qlin_hostcheck_launches.restype = S
lib.qlin_status_string.restype = ctypes.c_char_p
lib.qlin_status_string.argtypes = [S]

OK, NULL, SHAPE, ALIGN, UNSUP, HIP, ALIAS = range(7)
STATUSES = set(range(8))
A = 0x10000000
calls = 0


def call(name, *args):
    """One call; checks the status is defined and that errors launch nothing."""
    global calls
    before = lib.qlin_hostcheck_launches()
    st = getattr(lib, name)(*args)
    after = lib.qlin_hostcheck_launches()
    assert st in STATUSES, (name, st)
    assert lib.qlin_status_string(st).startswith(b"QLIN_")
    if st != OK:
        assert after == before, f"{name} returned {st} after launching"
    calls += 1
    return st


libc = ctypes.CDLL(None)
libc.malloc.restype = P
libc.malloc.argtypes = [ctypes.c_size_t]


def segs(*items):
    """The segments array in malloc'd memory of exactly len(items) entries, so
    that AddressSanitizer sees a read past its end (never freed: the process is
    short)."""
    n = max(1, len(items))
    p = libc.malloc(n * ctypes.sizeof(Seg))
    arr = (Seg * n).from_address(p)
    for i, (w, s, y, nn) in enumerate(items):
        arr[i] = Seg(w, s, y, nn)
    return p


if len(sys.argv) > 2 and sys.argv[2] == "--planted-overflow":
    # positive control: one segment in memory, two announced -- the sanitizer
    # must stop the process at the read of the second
    one = segs((A + 0x1000000, A + 0x2000000, A + 0x3000000, 64))
    lib.qlin_linear(0, A, 1, 256, one, 2, 0, None, None, None)
    print("planted overflow not detected")
    sys.exit(0)


# ---- boundary cases with known statuses -----------------------------------
gemm = "qlin_gemm_w8a8_ex"
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 64, 256, 0, 0, None) == OK
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 64, 250, 0, 0, None) == SHAPE
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 1 << 24, 1 << 24, 131072, 0, 0,
            None) == ALIAS                                   # the huge output range overlaps everything
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, (1 << 24) + 1, 4, 256, 0, 0,
            None) == SHAPE
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, -1, 4, 256, 0, 0, None) == SHAPE
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 131088, 0, 0, None) == SHAPE
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 256, 7, 0, None) == UNSUP
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 256, 0, 12, None) == UNSUP
assert call(gemm, A, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 256, 0, -1, None) == UNSUP
assert call(gemm, A + 1, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 256, 0, 0, None) == ALIGN
assert call(gemm, None, A + 0x1000000, A + 0x2000000, A + 0x3000000, A + 0x4000000, 4, 4, 256, 0, 0, None) == NULL
x = A
three = segs((A + 0x1000000, A + 0x2000000, A + 0x3000000, 64), (A + 0x4000000, A + 0x5000000, A + 0x6000000, 64),
             (A + 0x7000000, A + 0x8000000, A + 0x9000000, 128))
assert call("qlin_linear", 0, x, 1, 256, three, 3, 0, None, None, None) == OK
assert call("qlin_linear", 0, x, 1, 256, three, 0, 0, None, None, None) == SHAPE
assert call("qlin_linear", 0, x, 1, 256, three, 5, 0, None, None, None) == SHAPE      # reads no fourth segment
assert call("qlin_linear", 0, x, 8, 256, three, 3, 0, None, None, None) == NULL       # staging required
assert call("qlin_linear", 0, x, 8, 256, three, 3, 0, A + 0x1000000 + 64, A + 0xB000000, None) == ALIAS
huge = segs((A + 0x1000000, A + 0x2000000, A + 0x3000000, 1 << 24), (A + 0x4000000, A + 0x5000000, A + 0x6000000, 1))
assert call("qlin_linear", 0, x, 1, 256, huge, 2, 0, None, None, None) == SHAPE       # rows past the maximum
assert call("qlin_linear_swiglu", 0, x, 1, 256, A + 0x1000000, A + 0x2000000, A + 0x4000000, A + 0x5000000, 128,
            A + 0x6000000, None, None, None) == OK
assert call("qlin_linear_swiglu", 2, x, 1, 256, A + 0x1000000, A + 0x2000000, A + 0x4000000, A + 0x5000000, 100,
            A + 0x6000000, None, None, None) == SHAPE
wide = segs((A + 0x1000000, A + 0x2000000, A + 0x3000000, 128), (A + 0x4000000, A + 0x5000000, A + 0x6000000, 256))
assert call("qlin_linear_packed", 0, x, 64, 256, wide, 2, 0, A + 0xA000000, A + 0xB000000, None) == OK
assert call("qlin_linear_packed", 0, x, 32, 256, wide, 2, 0, A + 0xA000000, A + 0xB000000, None) == UNSUP
assert call("qlin_linear_packed", 0, x, 64, 256, three, 3, 0, A + 0xA000000, A + 0xB000000, None) == SHAPE
assert call("qlin_linear_packed", 2, x, 64, 256, wide, 2, 0, A + 0xA000000, A + 0xB000000, None) == OK
assert call("qlin_linear_packed", 9, x, 64, 256, wide, 2, 0, A + 0xA000000, A + 0xB000000, None) == UNSUP
assert call("qlin_pack_weights", 1, A, 256, 384, A + 0x1000000, None) == OK
assert call("qlin_linear_swiglu_packed", 2, x, 64, 256, A + 0x1000000, A + 0x2000000, A + 0x4000000, A + 0x5000000, 128,
            A + 0x6000000, A + 0xA000000, A + 0xB000000, None) == OK
assert call("qlin_linear_swiglu_packed", 0, x, 16, 256, A + 0x1000000, A + 0x2000000, A + 0x4000000, A + 0x5000000,
            128, A + 0x6000000, A + 0xA000000, A + 0xB000000, None) == UNSUP
assert call("qlin_pack_weights", 1, A, 256, 384, A + 0x100, None) == ALIAS
assert call("qlin_pack_weights", 0, A, 200, 384, A + 0x1000000, None) == SHAPE
assert call("qlin_quant_act_fp8", x, 4, 256, 64, A + 0x1000000, A + 0x2000000, None) == SHAPE
assert call("qlin_quant_act_fp8", x, 4, 200, 128, A + 0x1000000, A + 0x2000000, None) == SHAPE
assert call("qlin_quant_act_int8", x, 4, 256, x + 256, A + 0x2000000, None) == ALIAS

# ---- seeded random sweep --------------------------------------------------
rng = random.Random(20261203)
SIZES = [0, 1, 2, 3, 4, 5, 16, 17, 31, 32, 33, 128, 129, 512, 1000, 4096, 14336, 16384, 16400, 131072, 131088,
         (1 << 24), (1 << 24) + 1, -1, -(1 << 40), 1 << 40]


def ptr():
    r = rng.random()
    if r < 0.05:
        return None
    base = A + rng.randrange(0, 64) * 0x1000000
    if r < 0.15:
        base += rng.choice([1, 2, 4, 8])                     # misaligned
    if r < 0.25:
        base = A + rng.randrange(0, 0x2000000)               # anywhere: overlaps likely
    return base


def size():
    return rng.choice(SIZES) if rng.random() < 0.7 else rng.randrange(0, 5000)


for it in range(20000):
    fn = rng.randrange(8)
    M, N, K = size(), size(), rng.choice([16, 128, 256, 4096, 14336, 250, 0, -16, 131072, 131200])
    out, path = rng.choice([0, 1, 2, 3, -1]), rng.choice(list(range(0, 12)) + [-1, 12, 99])
    scheme = rng.choice([0, 1, 2, 3, -1])
    if fn == 0:
        call("qlin_quant_act_int8", ptr(), M, K, ptr(), ptr(), None)
    elif fn == 1:
        call("qlin_quant_act_fp8", ptr(), M, K, rng.choice([0, 128, 64, -1]), ptr(), ptr(), None)
    elif fn == 2:
        call("qlin_gemv_w8a8", ptr(), ptr(), ptr(), ptr(), ptr(), N, K, out, None)
    elif fn == 3:
        call(rng.choice(["qlin_gemm_w8a8_ex", "qlin_gemm_fp8_rowwise_ex", "qlin_gemm_fp8_block_ex"]),
             ptr(), ptr(), ptr(), ptr(), ptr(), M, N, K, out, path, None)
    elif fn in (4, 5):
        nseg = rng.randrange(0, 6)
        items = [(ptr(), ptr(), ptr(), rng.choice([0, 1, 64, 128, 256, 1000, 1 << 24, -1])) for _ in range(nseg)]
        arr = segs(*items) if rng.random() > 0.05 else None
        # the count passed is the array's, or one the library must refuse before reading (0, 5, -1)
        cnt = rng.choice([nseg, nseg, 0, 5, -1]) if nseg else rng.choice([0, 5, -1])
        if fn == 4:
            call(rng.choice(["qlin_linear", "qlin_linear_packed"]), scheme, ptr(), M, K, arr, cnt, out, ptr(), ptr(),
                 None)
        else:
            call("qlin_linear_weight_only", scheme, ptr(), M, K, arr, cnt, out, None)
    elif fn == 7:
        call("qlin_pack_weights", scheme, ptr(), N, K, ptr(), None)
    else:
        call(rng.choice(["qlin_linear_swiglu", "qlin_linear_swiglu_packed"]), scheme, ptr(), M, K, ptr(), ptr(), ptr(),
             ptr(), size(), ptr(), ptr(), ptr(), None)

print(f"hostcheck: {calls} calls, {lib.qlin_hostcheck_launches()} reached a launcher, no sanitizer report")
