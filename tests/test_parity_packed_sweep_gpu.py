"""Seeded random sweep of the packed-weight entry points against the CPU
oracle, with the bars of the fixed packed cases (W8A8 bf16 output bit-exact in
the f32 epilogue order, int32 accumulators exact; FP8 within 4e-3 max|y_ref|;
SwiGLU inside the SwiGLU tests' bound on h): token counts from 33 to past a
thousand (every tile shape and K-group count, ragged last tiles), K from one
128-byte stage to 80, one to four segments with widths that are multiples of
128, all three schemes, bf16 / f32 / int32 outputs."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol
from test_parity_packed_gpu import (BF16, F32, FP8B, I32, W8A8, exact, oracle_quant, packed_segments, run_packed,
                                    run_swiglu_packed)

pytestmark = pytest.mark.gpu
N_CASES = 16


def draw(scheme, i):
    rng = np.random.default_rng(20261204 + 1000 * scheme + i)
    M = int(rng.choice([int(rng.integers(33, 130)), int(rng.integers(130, 600)), int(rng.integers(600, 1300))]))
    K = 128 * int(rng.integers(1, 81))
    nseg = int(rng.integers(1, 5))
    ns = [128 * int(rng.integers(1, 9)) for _ in range(nseg)]
    out = int(rng.choice([BF16, F32, I32] if scheme == W8A8 else [BF16, F32]))
    return 30000 + 97 * scheme + i, M, K, ns, out


@pytest.mark.parametrize("scheme", [0, 1, 2])
@pytest.mark.parametrize("i", range(N_CASES))
def test_packed_sweep(scheme, i):
    seed, M, K, ns, out = draw(scheme, i)
    x = W.x_bf16(seed, M, K)
    segs = packed_segments(scheme, seed + 1, ns, K)
    qx_ref, sx_ref = oracle_quant(scheme, x)
    ys = run_packed(scheme, x, segs, out)
    what = f"scheme {scheme} M={M} K={K} ns={ns} out={out}"
    for (qw, sw, _), y in zip(segs, ys):
        if scheme == W8A8:
            acc = O.contract_int8(qx_ref, qw)
            if out == I32:
                assert np.array_equal(y, acc), what
                continue
            if out == BF16:
                assert np.array_equal(y, O.epilogue_f32_order(acc, sx_ref, sw)), what
        assert_within_tol(y, exact(scheme, qx_ref, sx_ref, qw, sw), what, f32=(out == F32))


@pytest.mark.parametrize("scheme", [0, 1, 2])
@pytest.mark.parametrize("i", range(6))
def test_packed_swiglu_sweep(scheme, i):
    from test_parity_swiglu_gpu import check, make_pair
    rng = np.random.default_rng(20261205 + 1000 * scheme + i)
    M = int(rng.integers(33, 700))
    K = 128 * int(rng.integers(1, 40))
    I = 128 * int(rng.integers(1, 40))
    x = W.x_bf16(31000 + 97 * scheme + i, M, K)
    gate, up = make_pair(scheme, 31500 + 97 * scheme + i, I, K)
    check(scheme, x, gate, up, run_swiglu_packed(scheme, x, (gate, up)), f"scheme {scheme} M={M} K={K} I={I}")
