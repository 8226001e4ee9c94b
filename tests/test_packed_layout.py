"""CPU pin of the packed weight layout (include/qlin.h, qlin_pack_weights): the
numpy reshape the GPU tests compare the packing kernel with, checked entry by
entry against the layout formula, and as a permutation of the codes."""
import numpy as np
import pytest

from packed_layout import packed_reference


@pytest.mark.parametrize("S", [32, 64])
@pytest.mark.parametrize("N,K", [(32, 128), (64, 256), (96, 384)])
def test_packed_reference_matches_the_formula(S, N, K):
    rng = np.random.default_rng(N + K + S)
    w = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    p = packed_reference(w, S)
    H = S // 32
    # every entry, by the formula, in a plain loop over its indices
    expect = np.empty(N * K, dtype=np.uint8)
    for rb in range(N // 32):
        for s in range(K // S):
            for h in range(H):
                for l in range(64):
                    base = ((rb * (K // S) + s) * H + h) * 1024 + 16 * l
                    row, col = 32 * rb + l % 32, S * s + (S // 2) * (l // 32) + 16 * h
                    expect[base:base + 16] = w[row, col:col + 16]
    assert np.array_equal(p, expect)


def test_packed_reference_is_a_permutation():
    rng = np.random.default_rng(7)
    N, K = 64, 256
    w = np.arange(N * K, dtype=np.int64).reshape(N, K)        # distinct values
    for S in (32, 64):
        p = packed_reference(w, S)
        assert np.array_equal(np.sort(p), np.arange(N * K))
    # a 128-byte K stage of one 32-row block is 4 KB of consecutive units
    wb = rng.integers(0, 256, size=(32, 256), dtype=np.uint8)
    for S in (32, 64):
        p = packed_reference(wb, S)
        stage1 = p[4096:8192]
        assert np.array_equal(np.sort(stage1), np.sort(wb[:, 128:256].reshape(-1)))
