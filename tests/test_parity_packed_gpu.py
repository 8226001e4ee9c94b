"""GPU parity of the packed-weight path: qlin_pack_weights against the layout
definition (packed_layout.packed_reference, pinned to the formula in
include/qlin.h by test_packed_layout.py), and qlin_linear_packed against the CPU
oracle -- W8A8 bit for bit (same int32 sums, same f32 epilogue order; the
int32 accumulator output exactly), FP8 rowwise and block FP8 within the FP8
tolerance -- on 64- and 128-token tiles, one and two K groups, ragged token
tails, several segments, and the q/k/v, o and down shapes of an 8B model at
512 tokens (Qwen3 8B's for the block scheme)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, dev, empty, host, torch_mod
from packed_layout import packed_reference

pytestmark = pytest.mark.gpu
BF16, I32, F32 = 0, 1, 2
W8A8, FP8R, FP8B = 0, 1, 2


def Q():
    import quantized_linear_layers_token_amd as q
    return q


@pytest.mark.parametrize("scheme,S", [(W8A8, 32), (FP8R, 64), (FP8B, 64)])
@pytest.mark.parametrize("N,K", [(128, 128), (384, 1024), (256, 14336)])
def test_pack_weights_layout(scheme, S, N, K):
    torch = torch_mod()
    w = W.w_int8(8000 + N, N, K).view(np.uint8) if scheme == W8A8 else W.w_e4m3(8000 + N, N, K)
    p = empty(torch, (N * K + 64,), torch.uint8, fill=0xA5)
    Q().qlin_pack_weights(scheme, dev(w), p[:N * K])
    got = host(p)
    assert (got[N * K:] == 0xA5).all(), "guard band overwritten"
    assert np.array_equal(got[:N * K], packed_reference(np.ascontiguousarray(w), S))


def packed_segments(scheme, seed, ns, K):
    """[(row-major codes, scales, packed device codes)] for each width."""
    torch = torch_mod()
    out = []
    for i, n in enumerate(ns):
        qw = W.w_int8(seed + 10 * i, n, K) if scheme == W8A8 else W.w_e4m3(seed + 10 * i, n, K)
        sw = W.scale_bf16(seed + 10 * i + 1, (n // 128, K // 128) if scheme == FP8B else (n,))
        pw = empty(torch, (n, K), torch.uint8)
        Q().qlin_pack_weights(scheme, dev(qw), pw)
        out.append((qw, sw, pw))
    return out


def run_packed(scheme, x, segs, out):
    torch = torch_mod()
    M, K = x.shape
    esz = 2 if out == BF16 else 4
    ys = [empty(torch, (M * qw.shape[0] * esz + 64,), torch.uint8, fill=0xFF) for qw, _, _ in segs]
    qx = empty(torch, (M, K), torch.uint8, fill=0x55)
    sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
    Q().qlin_linear_packed(scheme, dev(x), [(pw, dev(sw), y) for (_, sw, pw), y in zip(segs, ys)], out=out,
                           q_x=qx, s_x=sx)
    res = []
    for (qw, _, _), y in zip(segs, ys):
        raw = host(y)
        n = qw.shape[0]
        assert (raw[M * n * esz:] == 0xFF).all(), "guard band overwritten"
        res.append(raw[:M * n * esz].view({BF16: np.uint16, I32: np.int32, F32: np.float32}[out]).reshape(M, n))
    return res


CASES = [
    # (M, K, segment widths): 128 x 64 tiles with two K groups below 192 tiles of
    # 128 x 128, 128 x 128 with two K groups up to 256, with one K group past it
    (33, 128, [128]),                       # smallest M, one tile, 31 rows past M
    (64, 256, [128, 256]),                  # exactly one tile, two segments
    (200, 1024, [384, 128]),                # ragged last tile (8 tokens)
    (130, 512, [1024, 256, 256]),           # q/k/v-shaped segments, 2 tokens in the last tile
    (300, 256, [4096, 4096]),               # 128-token tiles (3 x 64 panels), ragged 44
    (97, 4096, [640, 128, 512, 256]),       # four segments, long K
    (1100, 256, [2048, 2048]),              # past 256 tiles of 128 x 128 (9 x 32): one K group, ragged 76
    (2000, 128, [2304]),                    # one K group (16 x 18 tiles), one K stage only
    (600, 256, [8192, 8192]),               # one K group, 5 x 128 tiles, ragged 88
]


def oracle_quant(scheme, x):
    if scheme == W8A8:
        return O.quant_act_int8(x)
    return O.quant_act_fp8(x, 128 if scheme == FP8B else 0)


def exact(scheme, qx, sx, qw, sw):
    if scheme == W8A8:
        return O.rescale_rowwise(O.contract_int8(qx, qw), sx, sw)
    if scheme == FP8R:
        return O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    return O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,ns", CASES)
def test_linear_packed_matches_oracle(scheme, M, K, ns):
    x = W.x_bf16(8100 + M + K + len(ns), M, K)
    segs = packed_segments(scheme, 8200 + K, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys = run_packed(scheme, x, segs, BF16)
    for (qw, sw, _), y in zip(segs, ys):
        if scheme == W8A8:
            acc = O.contract_int8(qx_ref, qw)
            assert np.array_equal(y, O.epilogue_f32_order(acc, sx_ref, sw))
        assert_within_tol(y, exact(scheme, qx_ref, sx_ref, qw, sw), f"packed scheme {scheme}")


@pytest.mark.parametrize("M", [100, 300])
def test_linear_packed_int8_accumulator_and_f32_exact(M):
    K, ns = 512, [4096, 4096] if M == 300 else [256, 384]
    x = W.x_bf16(8300 + M, M, K)
    segs = packed_segments(W8A8, 8301, ns, K)
    qx_ref, sx_ref = O.quant_act_int8(x)
    acc_ys = run_packed(W8A8, x, segs, I32)
    f32_ys = run_packed(W8A8, x, segs, F32)
    for (qw, sw, _), ya, yf in zip(segs, acc_ys, f32_ys):
        acc = O.contract_int8(qx_ref, qw)
        assert np.array_equal(ya, acc)
        assert_within_tol(yf, O.rescale_rowwise(acc, sx_ref, sw), "packed W8A8 f32", f32=True)


@pytest.mark.parametrize("scheme", [FP8R, FP8B])
def test_linear_packed_fp8_f32_output(scheme):
    M, K = 150, 1024
    x = W.x_bf16(8400, M, K)
    segs = packed_segments(scheme, 8401, [256, 512], K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    for (qw, sw, _), y in zip(segs, run_packed(scheme, x, segs, F32)):
        assert_within_tol(y, exact(scheme, qx_ref, sx_ref, qw, sw), "packed FP8 f32", f32=True)


def test_linear_packed_block_long_k():
    # 112 and 129 K blocks (an odd count: the last bf16 block scale ends two
    # bytes before a 4-byte boundary of the scale row)
    for K in (14336, 16512):
        M = 40
        x = W.x_bf16(8450 + K, M, K)
        segs = packed_segments(FP8B, 8451, [256], K)
        qx_ref, sx_ref = oracle_quant(FP8B, x)
        (qw, sw, _), = segs
        y, = run_packed(FP8B, x, segs, BF16)
        assert_within_tol(y, exact(FP8B, qx_ref, sx_ref, qw, sw), f"packed block K={K}")


@pytest.mark.parametrize("scheme", [W8A8, FP8B])
def test_linear_packed_max_k(scheme):
    # K = QLIN_MAX_K: 1024 stages, 4 MB per 32-row block descriptor, 1024 block scales per row
    K = Q().MAX_K
    M = 40
    x = W.x_bf16(8470, M, K)
    segs = packed_segments(scheme, 8471, [128], K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    (qw, sw, _), = segs
    y, = run_packed(scheme, x, segs, BF16)
    if scheme == W8A8:
        assert np.array_equal(y, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw))
    assert_within_tol(y, exact(scheme, qx_ref, sx_ref, qw, sw), f"packed K={K}")


def test_linear_packed_empty_segment_in_the_list():
    # a zero-width segment between two others is skipped; the others' panels follow on
    torch = torch_mod()
    M, K = 70, 256
    x = W.x_bf16(8480, M, K)
    a = packed_segments(W8A8, 8481, [256], K)[0]
    c = packed_segments(W8A8, 8482, [128], K)[0]
    ya = empty(torch, (M, 256), torch.int16, fill=0x11)
    yc = empty(torch, (M, 128), torch.int16, fill=0x11)
    qx, sx = empty(torch, (M, K), torch.uint8), empty(torch, (M,), torch.float32)
    none = torch.empty((0, K), dtype=torch.uint8, device="cuda")
    Q().qlin_linear_packed(W8A8, dev(x), [(a[2], dev(a[1]), ya), (none, None, None), (c[2], dev(c[1]), yc)],
                           q_x=qx, s_x=sx)
    qx_ref, sx_ref = O.quant_act_int8(x)
    for (qw, sw, _), y in ((a, ya), (c, yc)):
        got = host(y).view(np.uint16)
        assert np.array_equal(got, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw))


LLAMA = [("qkv", 4096, [4096, 1024, 1024]), ("o", 4096, [4096]), ("down", 14336, [4096])]
QWEN3 = [("qkv", 4096, [4096, 1024, 1024]), ("o", 4096, [4096]), ("down", 12288, [4096]),
         ("gateup", 4096, [12288, 12288])]


@pytest.mark.parametrize("scheme,name,K,ns", [(s, *c) for s in (W8A8, FP8R) for c in LLAMA] +
                         [(FP8B, *c) for c in QWEN3])
def test_linear_packed_8b_512_tokens(scheme, name, K, ns):
    # the projections the packed path serves, at the prefill size it is timed on
    M = 512
    x = W.x_bf16(8500 + K, M, K)
    segs = packed_segments(scheme, 8600 + K, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys = run_packed(scheme, x, segs, BF16)
    for (qw, sw, _), y in zip(segs, ys):
        if scheme == W8A8:
            assert np.array_equal(y, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw)), name
        else:
            assert_within_tol(y, exact(scheme, qx_ref, sx_ref, qw, sw), name)


def test_linear_packed_matches_row_major_path():
    # same int8 call through qlin_linear (row-major tiled GEMM) and qlin_linear_packed
    torch = torch_mod()
    M, K, n = 257, 2048, 768
    x = dev(W.x_bf16(8700, M, K))
    qw = dev(W.w_int8(8701, n, K))
    sw = dev(W.scale_bf16(8702, (n,)))
    pw = torch.empty_like(qw)
    Q().qlin_pack_weights(W8A8, qw, pw)
    qx, sx = empty(torch, (M, K), torch.uint8), empty(torch, (M,), torch.float32)
    y1, y2 = empty(torch, (M, n), torch.int16), empty(torch, (M, n), torch.int16)
    Q().qlin_linear(W8A8, x, [(qw, sw, y1)], q_x=qx, s_x=sx)
    Q().qlin_linear_packed(W8A8, x, [(pw, sw, y2)], q_x=qx, s_x=sx)
    assert torch.equal(y1, y2)


def test_linear_packed_refuses_small_m():
    torch = torch_mod()
    K, n = 256, 128
    x = dev(W.x_bf16(8800, 32, K))
    pw = dev(W.w_int8(8801, n, K))
    sw = dev(W.scale_bf16(8802, (n,)))
    y = empty(torch, (32, n), torch.int16, fill=0x3C)
    qx, sx = empty(torch, (32, K), torch.uint8), empty(torch, (32,), torch.float32)
    with pytest.raises(Q().QlinError):
        Q().qlin_linear_packed(W8A8, x, [(pw, sw, y)], q_x=qx, s_x=sx)
    with pytest.raises(Q().QlinError):
        Q().qlin_pack_weights(9, pw, torch.empty_like(pw))
    assert (host(y).view(np.uint8) == 0x3C).all()      # nothing launched


# ---- SwiGLU on packed weights ---------------------------------------------

SG_CASES = [
    # (M, K, I): 128 x 64 tiles (two K groups), ragged tails, 128 x 128 with two
    # K groups (192 tiles), with one K group (past 256 tiles)
    (33, 128, 128),
    (200, 1024, 384),
    (150, 512, 4096),
    (256, 128, 6144),
    (300, 256, 8192),
]


def run_swiglu_packed(scheme, x, pair):
    torch = torch_mod()
    M, K = x.shape
    I = pair[0][0].shape[0]
    h = empty(torch, (M * I * 2 + 64,), torch.uint8, fill=0xFF)
    qx = empty(torch, (M, K), torch.uint8, fill=0x55)
    sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
    packed = []
    for qw, sw in pair:
        pw = empty(torch, (I, K), torch.uint8)
        Q().qlin_pack_weights(scheme, dev(qw), pw)
        packed.append((pw, dev(sw)))
    Q().qlin_linear_swiglu_packed(scheme, dev(x), packed[0], packed[1], h, q_x=qx, s_x=sx)
    raw = host(h)
    assert (raw[M * I * 2:] == 0xFF).all(), "guard band overwritten"
    return raw[:M * I * 2].view(np.uint16).reshape(M, I)


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,I", SG_CASES)
def test_swiglu_packed_matches_oracle(scheme, M, K, I):
    from test_parity_swiglu_gpu import check, make_pair, run
    x = W.x_bf16(8900 + M + K, M, K)
    gate, up = make_pair(scheme, 8910 + I, I, K)
    h = run_swiglu_packed(scheme, x, (gate, up))
    check(scheme, x, gate, up, h, f"swiglu packed scheme {scheme} M={M} K={K} I={I}")
    if scheme == W8A8:
        # the row-major launch: same int32 sums and epilogue, so the same h
        h_rm, _, _ = run(scheme, x, gate, up, True)
        assert np.array_equal(h, h_rm)


@pytest.mark.parametrize("scheme,K,I", [(W8A8, 4096, 14336), (FP8R, 4096, 14336), (FP8B, 4096, 12288)])
def test_swiglu_packed_8b_gate_up_512_tokens(scheme, K, I):
    from test_parity_swiglu_gpu import check, make_pair
    M = 512
    x = W.x_bf16(8950 + I, M, K)
    gate, up = make_pair(scheme, 8960 + I, I, K)
    check(scheme, x, gate, up, run_swiglu_packed(scheme, x, (gate, up)), f"8B gate/up scheme {scheme}")


def test_swiglu_packed_block_odd_block_count():
    # K / 128 = 33 blocks (odd): each stage's bf16 scale at an odd 2-byte offset of its row
    from test_parity_swiglu_gpu import check, make_pair
    M, K, I = 50, 33 * 128, 256
    x = W.x_bf16(8980, M, K)
    gate, up = make_pair(FP8B, 8981, I, K)
    check(FP8B, x, gate, up, run_swiglu_packed(FP8B, x, (gate, up)), "swiglu packed block, 33 K blocks")


def test_swiglu_packed_refuses_small_m():
    torch = torch_mod()
    K, I = 256, 128
    x = dev(W.x_bf16(8990, 32, K))
    pw = dev(W.w_int8(8991, I, K))
    sw = dev(W.scale_bf16(8992, (I,)))
    h = empty(torch, (32, I), torch.int16, fill=0x3C)
    qx, sx = empty(torch, (32, K), torch.uint8), empty(torch, (32,), torch.float32)
    with pytest.raises(Q().QlinError):
        Q().qlin_linear_swiglu_packed(W8A8, x, (pw, sw), (pw, sw), h, q_x=qx, s_x=sx)
    assert (host(h).view(np.uint8) == 0x3C).all()      # nothing launched

