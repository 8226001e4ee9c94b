"""GPU parity of the products against the CPU oracle, for every kernel
(one-row, small-M, large-M), including each kernel forced outside its default
regime, ragged shapes, fused projections, and guard / poison checks.

int8: the int32 accumulator (out = I32) is bit-exact; bf16 output equals the
oracle's f32-order epilogue bit for bit and is within 4e-3 * max|y_ref| of the
exact fp64 rescale.  FP8: within 4e-3 * max|y_ref| (f32 accumulation in any
order)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, dev, empty, host, torch_mod

pytestmark = pytest.mark.gpu

AUTO, GEMV, SMALL, LARGE = 0, 1, 2, 3
BF16, I32, F32 = 0, 1, 2


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def paths_for(M):
    p = [AUTO, LARGE]
    if M <= 32:
        p.append(SMALL)
    if M == 1:
        p.append(GEMV)
    return p


def run_product(fn, qx, sx, qw, sw, M, N, out, path, guard=64):
    """Run one product with a poisoned output and a guard band after it."""
    torch = torch_mod()
    esz = 2 if out == BF16 else 4
    y = empty(torch, (M * N * esz + guard,), torch.uint8, fill=0xFF)
    getattr(Q(), fn)(dev(qx).view(qx.shape), dev(sx), dev(qw).view(qw.shape), dev(sw), y, out=out, path=path)
    raw = host(y)
    assert (raw[M * N * esz:] == 0xFF).all(), "guard band overwritten"
    body = raw[:M * N * esz]
    if out == BF16:
        return body.view(np.uint16).reshape(M, N)
    if out == I32:
        return body.view(np.int32).reshape(M, N)
    return body.view(np.float32).reshape(M, N)


def int8_case(seed, M, N, K):
    x = W.x_bf16(seed, M, K)
    qw = W.w_int8(seed + 1, N, K)
    sw = W.scale_bf16(seed + 2, N)
    qx, sx = O.quant_act_int8(x)
    return qx, sx, qw, sw


def check_int8(qx, sx, qw, sw, path):
    M, N = qx.shape[0], qw.shape[0]
    acc = O.contract_int8(qx, qw)
    got = run_product("qlin_gemm_w8a8", qx, sx, qw, sw, M, N, I32, path)
    assert np.array_equal(got, acc), f"int32 accumulator mismatch (path {path})"
    ybf = run_product("qlin_gemm_w8a8", qx, sx, qw, sw, M, N, BF16, path)
    assert np.array_equal(ybf, O.epilogue_f32_order(acc, sx, sw)), f"bf16 epilogue mismatch (path {path})"
    assert_within_tol(ybf, O.rescale_rowwise(acc, sx, sw), f"int8 path {path}")
    yf = run_product("qlin_gemm_w8a8", qx, sx, qw, sw, M, N, F32, path)
    f = (sx[:, None] * O.bf16_bits_to_f32(sw)[None, :]).astype(np.float32)
    assert np.array_equal(yf, (acc.astype(np.float32) * f).astype(np.float32))


INT8_SHAPES = [
    (1, 1, 16), (1, 7, 48), (1, 100, 1040), (1, 1024, 4096), (1, 33, 20000), (1, 17, 16400),
    (2, 16, 128), (5, 50, 400), (16, 256, 4096), (17, 130, 272), (32, 1024, 4096), (31, 48, 14336),
    (33, 128, 128), (100, 200, 528), (128, 384, 1024), (65, 77, 4112),
]


@pytest.mark.parametrize("M,N,K", INT8_SHAPES)
def test_int8_all_paths(M, N, K):
    case = int8_case(10 * M + N + K, M, N, K)
    for p in paths_for(M):
        check_int8(*case, p)


def test_gemv_entry_point():
    qx, sx, qw, sw = int8_case(77, 1, 300, 2048)
    torch = torch_mod()
    y = empty(torch, (300,), torch.int32, fill=0xFF)
    Q().qlin_gemv_w8a8(dev(qx), dev(sx), dev(qw), dev(sw), y, out=I32)
    assert np.array_equal(host(y), O.contract_int8(qx, qw)[0])


def test_int8_extreme_codes_fit_int32():
    # all codes at +-127 / -128 over K = 14336: the largest accumulator magnitude
    K = 14336
    qx = np.full((3, K), -127, np.int8)
    qx[1] = 127
    qx[2, ::2] = 127
    qw = np.full((40, K), -128, np.int8)
    qw[1::2] = 127
    sx = np.ones(3, np.float32)
    sw = np.full(40, 0x3F80, np.uint16)
    for M in (1, 3):
        for p in paths_for(M):
            got = run_product("qlin_gemm_w8a8", qx[:M], sx[:M], qw, sw, M, 40, I32, p)
            assert np.array_equal(got, O.contract_int8(qx[:M], qw))


U32 = 2.0 ** -24   # f32 unit roundoff


def f32_sum_bound_rowwise(qx, qw, sx, sw):
    """Rigorous bound on |y_f32 - y_exact| for an f32 accumulation of exact E4M3
    products in any order: (K + 4) u * sum_k |x_k w_k| * |s_x s_w| (the products
    of two E4M3 values are exact in f32; the +4 covers the scale products)."""
    K = qx.shape[1]
    absum = np.abs(O.e4m3_decode(qx)) @ np.abs(O.e4m3_decode(qw)).T
    return (K + 4) * U32 * absum * np.abs(O.rescale_rowwise(np.ones_like(absum), sx, sw))


def f32_sum_bound_block(qx, qw, sx, sw):
    """Same bound for the block form: every product is weighted by its block's
    factor |s_x s_w|; block partials and their promotion add K/128 + 4 roundings."""
    M, K = qx.shape
    N = qw.shape[0]
    ax, aw = np.abs(O.e4m3_decode(qx)), np.abs(O.e4m3_decode(qw))
    tot = np.zeros((M, N))
    for kb in range(K // 128):
        sl = slice(kb * 128, kb * 128 + 128)
        f = np.abs(sx[:, kb].astype(np.float64))[:, None] * np.repeat(O.bf16_bits_to_f64(sw[:, kb]), 128)[None, :N]
        tot += f * (ax[:, sl] @ aw[:, sl].T)
    return (K + K // 128 + 4) * U32 * tot


def mfma_group_bound(qx, qw, fac):
    """Extra error of the E4M3 matrix-core paths.  Measured on gfx950: one
    v_mfma_*_f8f6f4 instruction sums its products on a grid 2^-13 relative to
    its largest product (smaller contributions are dropped), while the f32
    accumulator carried between instructions is exact-rounded.  Every
    instruction covers K inside one aligned 128-wide block, so per block
    |error| <= 128 * 2^-12 * max|x| * max|w| (2x margin on the grid), times the
    block's |scale|.  fac[kb] -> [M, N] factor of block kb."""
    M, K = qx.shape
    ax, aw = np.abs(O.e4m3_decode(qx)), np.abs(O.e4m3_decode(qw))
    tot = np.zeros((M, qw.shape[0]))
    for kb in range((K + 127) // 128):
        sl = slice(kb * 128, min(K, kb * 128 + 128))
        tot += 128 * 2.0 ** -12 * np.outer(ax[:, sl].max(1), aw[:, sl].max(1)) * fac(kb)
    return tot


def rowwise_bound(qx, qw, sx, sw, path):
    f32 = f32_sum_bound_rowwise(qx, qw, sx, sw)
    if path == GEMV or (path == AUTO and qx.shape[0] == 1):
        return f32                                         # VALU path: exact products, f32 sums
    sc = np.abs(O.rescale_rowwise(np.ones((qx.shape[0], qw.shape[0])), sx, sw))
    return f32 + mfma_group_bound(qx, qw, lambda kb: sc)


def block_bound(qx, qw, sx, sw, path):
    f32 = f32_sum_bound_block(qx, qw, sx, sw)
    if path == GEMV or (path == AUTO and qx.shape[0] == 1):
        return f32
    N = qw.shape[0]
    fac = lambda kb: np.abs(sx[:, kb].astype(np.float64))[:, None] * np.repeat(O.bf16_bits_to_f64(sw[:, kb]), 128)[None, :N]
    return f32 + mfma_group_bound(qx, qw, fac)


def fp8_row_case(seed, M, N, K):
    x = W.x_bf16(seed, M, K)
    qw = W.w_e4m3(seed + 1, N, K)
    sw = W.scale_bf16(seed + 2, N)
    qx, sx = O.quant_act_fp8(x, 0)
    return qx, sx, qw, sw


FP8_SHAPES = [(1, 1, 16), (1, 100, 1040), (1, 1024, 4096), (1, 33, 20000), (3, 50, 400), (16, 256, 4096),
              (32, 130, 14336), (33, 128, 128), (100, 200, 528), (64, 512, 4096)]


@pytest.mark.parametrize("M,N,K", FP8_SHAPES)
def test_fp8_rowwise_all_paths(M, N, K):
    qx, sx, qw, sw = fp8_row_case(20 * M + N + K, M, N, K)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    for p in paths_for(M):
        bound = rowwise_bound(qx, qw, sx, sw, p)
        y = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, BF16, p)
        assert_within_tol(y, y_exact, f"fp8 rowwise path {p}")
        yf = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, F32, p)
        assert np.all(np.abs(yf - y_exact) <= bound), f"f32 result outside the summation bound (path {p})"


def fp8_block_case(seed, M, N, K):
    x = W.x_bf16(seed, M, K)
    qw = W.w_e4m3(seed + 1, N, K)
    sw = W.scale_bf16(seed + 2, (N // 128, K // 128))
    qx, sx = O.quant_act_fp8(x, 128)
    return qx, sx, qw, sw


BLOCK_SHAPES = [(1, 128, 128), (1, 1024, 4096), (1, 256, 12288), (2, 128, 256), (16, 384, 1024),
                (32, 256, 4096), (33, 128, 128), (100, 256, 640), (64, 512, 4096)]


@pytest.mark.parametrize("M,N,K", BLOCK_SHAPES)
def test_fp8_block_all_paths(M, N, K):
    qx, sx, qw, sw = fp8_block_case(30 * M + N + K, M, N, K)
    y_exact = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)
    for p in paths_for(M):
        bound = block_bound(qx, qw, sx, sw, p)
        y = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, BF16, p)
        assert_within_tol(y, y_exact, f"fp8 block path {p}")
        yf = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, F32, p)
        assert np.all(np.abs(yf - y_exact) <= bound), f"f32 result outside the summation bound (path {p})"


def test_fp8_block_scale_indexing():
    # A single block scale changed: only its 128-row output block may move, and by
    # the amount the oracle predicts (catches transposed or shifted scale grids).
    M, N, K = 16, 384, 512
    qx, sx, qw, sw = fp8_block_case(4242, M, N, K)
    sw2 = sw.copy()
    sw2[1, 2] = 0x4000
    for p in (AUTO, LARGE, SMALL):
        y0 = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, F32, p)
        y1 = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw2, M, N, F32, p)
        e1 = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw2)
        assert np.array_equal(y0[:, :128], y1[:, :128]) and np.array_equal(y0[:, 256:], y1[:, 256:])
        assert np.all(np.abs(y1 - e1) <= block_bound(qx, qw, sx, sw2, p))
        assert not np.array_equal(y0[:, 128:256], y1[:, 128:256])


def test_fp8_extreme_codes():
    # +-448 everywhere and all-subnormal rows
    K = 4096
    qx = np.full((2, K), 0x7E, np.uint8)
    qx[1] = 0x01
    qw = np.full((64, K), 0xFE, np.uint8)
    qw[::2] = 0x07
    sx = np.array([1.0, 2.0], np.float32)
    sw = np.full(64, 0x3F80, np.uint16)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    for M in (1, 2):
        for p in paths_for(M):
            y = run_product("qlin_gemm_fp8_rowwise", qx[:M], sx[:M], qw, sw, M, 64, F32, p)
            assert np.all(np.abs(y - y_exact[:M]) <= rowwise_bound(qx[:M], qw, sx[:M], sw, p))


def test_end_to_end_w8a8_quant_then_gemm():
    torch = torch_mod()
    M, N, K = 16, 4096, 4096          # the single-projection workload (K = N = 4096, 16 tokens)
    x = W.x_bf16(1, M, K)
    qw = W.w_int8(2, N, K)
    sw = W.scale_bf16(3, N)
    yb_ref, y_exact, qx_ref, sx_ref, acc = O.linear_w8a8(x, qw, sw)
    xd = dev(x)
    q = empty(torch, (M, K), torch.int8)
    s = empty(torch, (M,), torch.float32)
    y = empty(torch, (M, N), torch.int16)
    Q().qlin_quant_act_int8(xd, q, s)
    Q().qlin_gemm_w8a8(q, s, dev(qw), dev(sw), y)
    assert np.array_equal(host(q), qx_ref) and np.array_equal(host(s), sx_ref)
    yb = host(y, np.uint16)
    assert np.array_equal(yb, O.epilogue_f32_order(acc, sx_ref, sw))
    assert_within_tol(yb, y_exact, "end to end")
    assert_within_tol(yb_ref, y_exact, "oracle bf16")


def test_output_stream_order_and_m0():
    torch = torch_mod()
    qx, sx, qw, sw = int8_case(9, 4, 64, 256)
    y = empty(torch, (4, 64), torch.int32, fill=0x33)
    Q().lib().qlin_gemm_w8a8(dev(qx).data_ptr(), dev(sx).data_ptr(), dev(qw).data_ptr(), dev(sw).data_ptr(),
                             y.data_ptr(), 0, 64, 256, I32, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (host(y).view(np.uint8) == 0x33).all()
    # on a side stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        yy = empty(torch, (4, 64), torch.int32)
        Q().qlin_gemm_w8a8(dev(qx), dev(sx), dev(qw), dev(sw), yy, out=I32)
    s.synchronize()
    assert np.array_equal(host(yy), O.contract_int8(qx, qw))


def test_fp8_mfma_accumulation_model():
    # Pins the E4M3 matrix-core arithmetic the error bounds above rely on
    # (rowwise product, out = F32, unit scales, K = 256):
    #  - across instructions the f32 accumulator is exact-rounded;
    #  - inside one instruction, products >= 2^-13 of the largest are kept exactly.
    K = 256
    one = 0x38
    cases = [
        ([(0, one, one), (1, 0x18, 0x01)], 1 + 2.0 ** -13),                      # same instruction
        ([(0, one, one), (1, 0x18, 0x03)], 1 + 3 * 2.0 ** -13),
        ([(0, 0xB8, one), (1, 0xA0, 0x03)], -(1 + 1.5 * 2.0 ** -11)),
        ([(0, one, one), (128, 0x01, 0x02)], 1 + 2.0 ** -17),                     # across instructions
        ([(0, 0x7E, 0x7E), (128, one, one)], 448.0 ** 2 + 1),
        ([(0, 0x7E, 0x7E), (128, 0xFE, 0x7E), (200, one, one)], 1.0),
        ([(1, 0x18, 0x01), (2, 0x01, 0x01), (3, 0x01, 0x01)], 2.0 ** -13 + 2.0 ** -17),
    ]
    n = len(cases)
    X = np.zeros((n, K), np.uint8)
    Wt = np.zeros((n, K), np.uint8)
    for i, (terms, _) in enumerate(cases):
        for k, a, b in terms:
            X[i, k], Wt[i, k] = a, b
    sx = np.ones(n, np.float32)
    sw = np.full(n, 0x3F80, np.uint16)
    exact = np.diag(O.contract_e4m3(X, Wt))
    assert list(exact) == [c[1] for c in cases]
    for p in (SMALL, LARGE):
        y = run_product("qlin_gemm_fp8_rowwise", X, sx, Wt, sw, n, n, F32, p)
        assert np.array_equal(np.diag(y).astype(np.float64), exact), p


# Every fixed output tile of the tiled GEMM, on shapes spanning several tiles
# with ragged M, N and K edges, one- to three-stage K (pipeline prologue and the
# odd last stage) and tile counts that do and do not divide by the 8 XCDs.
TILE_PATHS = [4, 5, 6, 7, 8, 9]   # 256x128, 128x128, 128x64, 128x256 (weight rows x tokens), then
                                # 128x128 and 128x64 with two K groups (odd stage counts: K = 1040, 384)
ROWWISE_TILE_PATHS = TILE_PATHS + [10, 11]   # 256x256 with 8 or 4 wavefronts (rowwise schemes only)
TILE_SHAPES = [(300, 600, 1040), (129, 257, 16), (40, 130, 384), (512, 1024, 128), (260, 384, 256)]
TILE_BLOCK_SHAPES = [(300, 640, 1152), (129, 256, 128), (40, 128, 384), (512, 1024, 256)]


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_int8_every_tile(M, N, K):
    case = int8_case(11 * M + N + K, M, N, K)
    for p in ROWWISE_TILE_PATHS:
        check_int8(*case, p)


@pytest.mark.parametrize("M,N,K", TILE_SHAPES)
def test_fp8_rowwise_every_tile(M, N, K):
    qx, sx, qw, sw = fp8_row_case(21 * M + N + K, M, N, K)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    bound = rowwise_bound(qx, qw, sx, sw, LARGE)
    for p in ROWWISE_TILE_PATHS:
        y = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, BF16, p)
        assert_within_tol(y, y_exact, f"fp8 rowwise tile path {p}")
        yf = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, F32, p)
        assert np.all(np.abs(yf - y_exact) <= bound), f"f32 result outside the summation bound (path {p})"


@pytest.mark.parametrize("M,N,K", TILE_BLOCK_SHAPES)
def test_fp8_block_every_tile(M, N, K):
    qx, sx, qw, sw = fp8_block_case(31 * M + N + K, M, N, K)
    y_exact = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)
    bound = block_bound(qx, qw, sx, sw, LARGE)
    for p in TILE_PATHS:
        y = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, BF16, p)
        assert_within_tol(y, y_exact, f"fp8 block tile path {p}")
        yf = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, F32, p)
        assert np.all(np.abs(yf - y_exact) <= bound), f"f32 result outside the summation bound (path {p})"


# The wide small-M tile (64 weight rows: four MFMA row tiles share each token
# load) runs for calls with at least 256 such tiles, as the fused gate/up
# projection of Llama-3.1-8B (N = 2 x 14336, K = 4096) at 2..32 tokens: one
# token tile up to 16 tokens, two from 17.  Every output is compared.
WIDE_N, WIDE_K = 28672, 4096
WIDE_M = [5, 16, 17, 32]


@pytest.mark.parametrize("M", WIDE_M)
def test_int8_small_m_wide_tiles(M):
    print(f"int8 wide small-M M={M}", flush=True)
    check_int8(*int8_case(5000 + M, M, WIDE_N, WIDE_K), SMALL)


@pytest.mark.parametrize("M", WIDE_M)
def test_fp8_rowwise_small_m_wide_tiles(M):
    print(f"fp8 rowwise wide small-M M={M}", flush=True)
    qx, sx, qw, sw = fp8_row_case(5100 + M, M, WIDE_N, WIDE_K)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, WIDE_N, BF16, SMALL)
    assert_within_tol(y, y_exact, f"fp8 rowwise wide small-M M={M}")
    yf = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, WIDE_N, F32, SMALL)
    assert np.all(np.abs(yf - y_exact) <= rowwise_bound(qx, qw, sx, sw, SMALL))


@pytest.mark.parametrize("M", WIDE_M)
def test_fp8_block_small_m_wide_tiles(M):
    print(f"fp8 block wide small-M M={M}", flush=True)
    qx, sx, qw, sw = fp8_block_case(5200 + M, M, WIDE_N, WIDE_K)
    y_exact = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, WIDE_N, BF16, SMALL)
    assert_within_tol(y, y_exact, f"fp8 block wide small-M M={M}")
    yf = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, WIDE_N, F32, SMALL)
    assert np.all(np.abs(yf - y_exact) <= block_bound(qx, qw, sx, sw, SMALL))


# The 32-row small-M tile (two MFMA row tiles share each token load) runs for
# calls with at least 192 such tiles and K <= 4096 that have too few 64-row
# tiles, as the fused q/k/v projection of Llama-3.1-8B (N = 6144, K = 4096).
# A ragged last tile (N = 6160) and ragged K for the rowwise schemes.
MID_M = [5, 16, 17, 32]


@pytest.mark.parametrize("M", MID_M)
def test_int8_small_m_mid_tiles(M):
    print(f"int8 32-row small-M M={M}", flush=True)
    check_int8(*int8_case(5300 + M, M, 6160, 4000), SMALL)


@pytest.mark.parametrize("M", MID_M)
def test_fp8_rowwise_small_m_mid_tiles(M):
    print(f"fp8 rowwise 32-row small-M M={M}", flush=True)
    qx, sx, qw, sw = fp8_row_case(5400 + M, M, 6160, 4000)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, 6160, BF16, SMALL)
    assert_within_tol(y, y_exact, f"fp8 rowwise 32-row small-M M={M}")
    yf = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, 6160, F32, SMALL)
    assert np.all(np.abs(yf - y_exact) <= rowwise_bound(qx, qw, sx, sw, SMALL))


@pytest.mark.parametrize("M", MID_M)
def test_fp8_block_small_m_mid_tiles(M):
    print(f"fp8 block 32-row small-M M={M}", flush=True)
    qx, sx, qw, sw = fp8_block_case(5500 + M, M, 6144, 4096)
    y_exact = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, 6144, BF16, SMALL)
    assert_within_tol(y, y_exact, f"fp8 block 32-row small-M M={M}")
    yf = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, 6144, F32, SMALL)
    assert np.all(np.abs(yf - y_exact) <= block_bound(qx, qw, sx, sw, SMALL))
