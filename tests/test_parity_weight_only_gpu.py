"""GPU parity of the weight-only ("equivalent") numerics against the CPU
oracle: bf16 inputs times dequantized int8 / E4M3 weights, one to four
segments per call, the one-token kernel (M = 1, K <= 16384) and the
matrix-core kernel (2..32 tokens, or longer K).

bf16 outputs: within 4e-3 * max|y_ref| of the exact value.  F32 outputs:
inside the f32 summation bound of exact products (every bf16 x int8/E4M3
product is exact in f32), plus the in-instruction summation allowance used for
the FP8 matrix-core products (every kernel here sums on the matrix cores)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, bf16_to_f64, dev, empty, host, torch_mod

pytestmark = pytest.mark.gpu
BF16, I32, F32 = 0, 1, 2
W8A8, FP8R, FP8B = 0, 1, 2
NAME = {W8A8: "int8", FP8R: "fp8_rowwise", FP8B: "fp8_block"}
U32 = 2.0 ** -24


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def make_segments(scheme, seed, ns, K):
    segs = []
    for i, n in enumerate(ns):
        qw = W.w_int8(seed + 10 * i, n, K) if scheme == W8A8 else W.w_e4m3(seed + 10 * i, n, K)
        sw = W.scale_bf16(seed + 10 * i + 1, (n // 128, K // 128) if scheme == FP8B else (n,))
        segs.append((qw, sw))
    return segs


def run(scheme, x, segs, out):
    torch = torch_mod()
    M, K = x.shape
    esz = 2 if out == BF16 else 4
    ys = [empty(torch, (M * qw.shape[0] * esz + 64,), torch.uint8, fill=0xFF) for qw, _ in segs]
    Q().qlin_linear_weight_only(scheme, dev(x), [(dev(qw), dev(sw), y) for (qw, sw), y in zip(segs, ys)], out=out)
    res = []
    for (qw, _), y in zip(segs, ys):
        raw = host(y)
        n = qw.shape[0]
        assert (raw[M * n * esz:] == 0xFF).all(), "guard band overwritten"
        res.append(raw[:M * n * esz].view(np.uint16 if out == BF16 else np.float32).reshape(M, n))
    return res


def f32_bound(scheme, x, qw, sw, mfma):
    """|y_f32 - y_exact| bound: f32 sums of exact products in any order,
    (K + K/128 + 4) u * sum_k |x w|; the matrix-core path adds, per 128-wide
    block, 128 * 2^-12 * max|x| * max|w| (the in-instruction allowance)."""
    K = x.shape[1]
    ax = np.abs(bf16_to_f64(x))
    aw = np.abs(O.dequantize_weights(qw, sw, NAME[scheme]))
    bound = (K + K // 128 + 4) * U32 * (ax @ aw.T)
    if mfma:
        for kb in range((K + 127) // 128):
            sl = slice(kb * 128, min(K, kb * 128 + 128))
            bound = bound + 128 * 2.0 ** -12 * np.outer(ax[:, sl].max(1), aw[:, sl].max(1))
    return bound


CASES = [
    # (M, K, segment widths)
    (1, 128, [128]),
    (1, 4096, [384, 128, 256]),        # one-token kernel, three segments
    (1, 14336, [256]),                 # one-token kernel, long rows (one row per wave)
    (1, 16512, [128]),                 # K above the one-token limit: matrix-core kernel
    (2, 1024, [256, 128]),
    (5, 4096, [384]),
    (16, 512, [128, 256, 128, 384]),   # four segments
    (17, 1152, [256]),                 # two token tiles
    (32, 4096, [512, 128]),
]


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,ns", CASES)
def test_weight_only_matches_oracle(scheme, M, K, ns):
    x = W.x_bf16(8000 + M + K, M, K)
    segs = make_segments(scheme, 8100 + K + M, ns, K)
    mfma = True                         # every kernel sums on the matrix cores
    ys_bf = run(scheme, x, segs, BF16)
    ys_f = run(scheme, x, segs, F32)
    for (qw, sw), yb, yf in zip(segs, ys_bf, ys_f):
        _, y_exact = O.linear_weight_only(x, qw, sw, NAME[scheme])
        assert_within_tol(yb, y_exact, f"weight-only {NAME[scheme]} M={M} K={K}")
        bound = f32_bound(scheme, x, qw, sw, mfma)
        assert np.all(np.abs(yf.astype(np.float64) - y_exact) <= bound), \
            f"f32 result outside the summation bound ({NAME[scheme]} M={M} K={K})"


def test_weight_only_ragged_rows_and_k():
    # widths and K that are not multiples of any tile edge (rowwise schemes)
    M, K = 3, 1040
    x = W.x_bf16(8200, M, K)
    for scheme in (W8A8, FP8R):
        segs = make_segments(scheme, 8210, [200, 72, 1], K)
        for (qw, sw), yf in zip(segs, run(scheme, x, segs, F32)):
            _, y_exact = O.linear_weight_only(x, qw, sw, NAME[scheme])
            assert np.all(np.abs(yf.astype(np.float64) - y_exact) <= f32_bound(scheme, x, qw, sw, True))
    x1 = W.x_bf16(8201, 1, K)
    segs = make_segments(W8A8, 8220, [200, 72, 1], K)
    for (qw, sw), yf in zip(segs, run(W8A8, x1, segs, F32)):
        _, y_exact = O.linear_weight_only(x1, qw, sw, "int8")
        assert np.all(np.abs(yf.astype(np.float64) - y_exact) <= f32_bound(W8A8, x1, qw, sw, True))


def test_weight_only_equals_quantized_path_when_rounding_is_exact():
    # the input is s * q with power-of-two s and max|q| = 127: the W8A8 path's
    # rounding is exact, so both numerics give the same f32 value up to summation order
    rng = np.random.default_rng(8300)
    M, K, N = 1, 4096, 256
    q = rng.integers(-127, 128, (M, K))
    q[:, 0] = 127
    x = O.round_to_bf16_bits(q.astype(np.float64) * 2.0 ** -4)
    qw = W.w_int8(8301, N, K)
    sw = W.scale_bf16(8302, N)
    yf = run(W8A8, x, [(qw, sw)], F32)[0]
    _, y_exact, _, _, _ = O.linear_w8a8(x, qw, sw)
    assert np.all(np.abs(yf.astype(np.float64) - y_exact) <= f32_bound(W8A8, x, qw, sw, True))
