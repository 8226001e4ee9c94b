"""Seeded random sweeps against the CPU oracle, with the same bars as the fixed
cases (int8 accumulators, codes, scales and bf16 epilogue bit-exact; FP8
within 4e-3 * max|y_ref| and inside the f32 summation bound):

  * the products: shapes drawn across all three regimes (one row, up to 32
    rows, the tiled GEMM) with ragged M, N and K, each run on a kernel path
    drawn from those that accept it (automatic choice, a forced regime, or
    one fixed GEMM tile);
  * qlin_linear: token counts drawn around every launch-form boundary, one to
    four ragged segments, with and without the staging buffers;
  * qlin_linear_swiglu: the same token counts, ragged gate widths (the SwiGLU
    tests' bound on h);
  * qlin_linear_weight_only: 1..32 tokens, one to four ragged segments, K on
    both sides of the one-token kernel's limit (bf16 within the tolerance,
    f32 inside the summation bound);
  * the activation quantizers: token counts and row lengths across every
    per-thread chunk count and the two-pass long-row kernel, inputs scaled by
    powers of two from the subnormal to the large end of bf16 (codes and
    scales bit-exact, including tokens and groups whose absmax lies below
    2^-118, where Q/a overflows f32 and the rounding pre-scales by 2^64)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, e4m3_equal_mod_zero
from test_parity_quant_gpu import run_fp8 as quant_fp8
from test_parity_quant_gpu import run_int8 as quant_int8
from test_parity_linear_gpu import exact as linear_exact
from test_parity_linear_gpu import make_segments, oracle_quant, run_linear
from test_parity_swiglu_gpu import check as swiglu_check
from test_parity_swiglu_gpu import make_pair
from test_parity_swiglu_gpu import run as run_swiglu
from test_parity_weight_only_gpu import NAME as WO_NAME
from test_parity_weight_only_gpu import f32_bound as wo_f32_bound
from test_parity_weight_only_gpu import make_segments as wo_segments
from test_parity_weight_only_gpu import run as run_weight_only
from test_parity_gemm_gpu import (AUTO, BF16, F32, GEMV, LARGE, SMALL, block_bound, check_int8, fp8_block_case,
                                  fp8_row_case, int8_case, rowwise_bound, run_product)

pytestmark = pytest.mark.gpu

FIXED_TILES = [4, 5, 6, 7, 8, 9]
W8_TILE = 10            # 256 x 256 with 8 wavefronts: int8 and FP8 rowwise only
N_CASES = 30


def draw(scheme, i):
    """Case i of a scheme: (seed, M, N, K, path), from a generator seeded by both."""
    rng = np.random.default_rng(20261203 + 1000 * scheme + i)
    regime = i % 3
    M = 1 if regime == 0 else int(rng.integers(2, 33)) if regime == 1 else int(rng.integers(33, 600))
    if scheme == 2:
        N = 128 * int(rng.integers(1, 6))
        K = 128 * int(rng.integers(1, 24))
    else:
        N = int(rng.integers(1, 700))
        K = 16 * int(rng.integers(1, 190))
    paths = [AUTO, LARGE] + FIXED_TILES + ([] if scheme == 2 else [W8_TILE])
    if M <= 32:
        paths.append(SMALL)
    if M == 1:
        paths.append(GEMV)
    return 7000 + 100 * scheme + i, M, N, K, int(rng.choice(paths))


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_int8(i):
    seed, M, N, K, path = draw(0, i)
    check_int8(*int8_case(seed, M, N, K), path)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_fp8_rowwise(i):
    seed, M, N, K, path = draw(1, i)
    qx, sx, qw, sw = fp8_row_case(seed, M, N, K)
    y_exact = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, BF16, path)
    assert_within_tol(y, y_exact, f"fp8 rowwise {M}x{N}x{K} path {path}")
    yf = run_product("qlin_gemm_fp8_rowwise", qx, sx, qw, sw, M, N, F32, path)
    assert np.all(np.abs(yf - y_exact) <= rowwise_bound(qx, qw, sx, sw, path)), (M, N, K, path)


@pytest.mark.parametrize("i", range(N_CASES))
def test_sweep_fp8_block(i):
    seed, M, N, K, path = draw(2, i)
    qx, sx, qw, sw = fp8_block_case(seed, M, N, K)
    y_exact = O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)
    y = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, BF16, path)
    assert_within_tol(y, y_exact, f"fp8 block {M}x{N}x{K} path {path}")
    yf = run_product("qlin_gemm_fp8_block", qx, sx, qw, sw, M, N, F32, path)
    assert np.all(np.abs(yf - y_exact) <= block_bound(qx, qw, sx, sw, path)), (M, N, K, path)


N_LINEAR = 20


def draw_linear(scheme, i):
    """Case i of a scheme: (seed, M, K, segment widths, staged)."""
    rng = np.random.default_rng(20261204 + 1000 * scheme + i)
    M = int(rng.choice([1, 1, 2, 3, 4, int(rng.integers(5, 33)), int(rng.integers(33, 300))]))
    nseg = int(rng.integers(1, 5))
    if scheme == 2:
        K = 128 * int(rng.integers(1, 40))
        ns = [128 * int(rng.integers(1, 5)) for _ in range(nseg)]
    else:
        K = 16 * int(rng.integers(1, 400))
        ns = [int(rng.integers(1, 600)) for _ in range(nseg)]
    return 8000 + 100 * scheme + i, M, K, ns, bool(rng.integers(0, 2))


@pytest.mark.parametrize("scheme", [0, 1, 2])
@pytest.mark.parametrize("i", range(N_LINEAR))
def test_sweep_linear(scheme, i):
    seed, M, K, ns, staged = draw_linear(scheme, i)
    x = W.x_bf16(seed, M, K)
    segs = make_segments(scheme, seed + 50, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys, qx, sx = run_linear(scheme, x, segs, BF16, staged)
    what = f"scheme {scheme} M {M} K {K} widths {ns} staged {staged}"
    if qx is not None:
        if scheme == 0:
            assert np.array_equal(qx.view(np.int8), qx_ref), what
        else:
            assert e4m3_equal_mod_zero(qx, qx_ref), what
        assert np.array_equal(sx.view(np.uint32), sx_ref.view(np.uint32)), what
    for (qw, sw), y in zip(segs, ys):
        assert_within_tol(y, linear_exact(scheme, qx_ref, sx_ref, qw, sw), what)
        if scheme == 0:
            assert np.array_equal(y, O.epilogue_f32_order(O.contract_int8(qx_ref, qw), sx_ref, sw)), what


N_SWIGLU = 12


@pytest.mark.parametrize("scheme", [0, 1, 2])
@pytest.mark.parametrize("i", range(N_SWIGLU))
def test_sweep_swiglu(scheme, i):
    rng = np.random.default_rng(20261205 + 1000 * scheme + i)
    M = int(rng.choice([1, 2, 3, 4, int(rng.integers(5, 33)), int(rng.integers(33, 300))]))
    if scheme == 2:
        K, I = 128 * int(rng.integers(1, 40)), 128 * int(rng.integers(1, 8))
    else:
        K, I = 16 * int(rng.integers(1, 400)), int(rng.integers(1, 900))
    staged = bool(rng.integers(0, 2))
    seed = 8500 + 100 * scheme + i
    x = W.x_bf16(seed, M, K)
    gate, up = make_pair(scheme, seed + 50, I, K)
    h_bits, _, _ = run_swiglu(scheme, x, gate, up, staged)
    swiglu_check(scheme, x, gate, up, h_bits, f"swiglu scheme {scheme} M {M} K {K} I {I} staged {staged}")


N_WEIGHT_ONLY = 12


@pytest.mark.parametrize("scheme", [0, 1, 2])
@pytest.mark.parametrize("i", range(N_WEIGHT_ONLY))
def test_sweep_weight_only(scheme, i):
    rng = np.random.default_rng(20261206 + 1000 * scheme + i)
    M = int(rng.choice([1, 1, 2, 4, int(rng.integers(5, 33))]))
    nseg = int(rng.integers(1, 5))
    if scheme == 2:
        K = 128 * int(rng.choice([int(rng.integers(1, 40)), 129]))     # 129 * 128 is past the one-token limit
        ns = [128 * int(rng.integers(1, 4)) for _ in range(nseg)]
    else:
        K = 16 * int(rng.choice([int(rng.integers(1, 400)), 1025]))    # 16400 is past the one-token limit
        ns = [int(rng.integers(1, 400)) for _ in range(nseg)]
    seed = 8700 + 100 * scheme + i
    x = W.x_bf16(seed, M, K)
    segs = wo_segments(scheme, seed + 50, ns, K)
    what = f"weight-only scheme {scheme} M {M} K {K} widths {ns}"
    ys_bf = run_weight_only(scheme, x, segs, BF16)
    ys_f = run_weight_only(scheme, x, segs, F32)
    for (qw, sw), yb, yf in zip(segs, ys_bf, ys_f):
        _, y_exact = O.linear_weight_only(x, qw, sw, WO_NAME[scheme])
        assert_within_tol(yb, y_exact, what)
        assert np.all(np.abs(yf.astype(np.float64) - y_exact) <= wo_f32_bound(scheme, x, qw, sw, True)), what


N_QUANT = 16


@pytest.mark.parametrize("kind", ["int8", "fp8_token", "fp8_group"])
@pytest.mark.parametrize("i", range(N_QUANT))
def test_sweep_quantizers(kind, i):
    rng = np.random.default_rng(20261207 + 100 * ["int8", "fp8_token", "fp8_group"].index(kind) + i)
    M = int(rng.choice([1, int(rng.integers(2, 40)), int(rng.integers(40, 600))]))
    if kind == "fp8_group":
        K = 128 * int(rng.integers(1, 130))
    else:
        K = 16 * int(rng.choice([int(rng.integers(1, 600)), int(rng.integers(600, 2600))]))
    # every fourth case with absmax below 2^-118 (Q / a overflows f32 there)
    e = int(rng.integers(-125, -119)) if i % 4 == 0 else int(rng.integers(-118, 121))
    x = O.round_to_bf16_bits(O.bf16_bits_to_f64(W.x_bf16(8900 + i, M, K)) * 2.0 ** e)
    what = f"{kind} M {M} K {K} scale 2^{e}"
    if kind == "int8":
        q, sc = quant_int8(x)
        qo, so = O.quant_act_int8(x)
        assert np.array_equal(q, qo), what
    else:
        group = 128 if kind == "fp8_group" else 0
        q, sc = quant_fp8(x, group)
        qo, so = O.quant_act_fp8(x, group)
        assert e4m3_equal_mod_zero(q, qo), what
    assert np.array_equal(sc.view(np.uint32), so.view(np.uint32)), what
