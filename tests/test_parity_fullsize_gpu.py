"""GPU parity at the benchmark workloads' full sizes, through the same calls
the benchmark times (one qlin_linear per layer input: q/k/v, o, gate/up,
down), checked on sampled outputs the oracle computes one by one.

Workloads (shapes from the "Command line" sections of the Llama 3.1 8B W8A8
and Qwen3 8B FP8 model cards):
  * one W8A8 projection, M = 16, N = K = 4096 (checked in full);
  * the Llama layer at M in {4, 8, 16, 32} (fused q/k/v and gate/up), W8A8,
    and at M in {4, 32} with FP8 per channel;
  * the Llama layer at M in {512, 1024}, W8A8 and FP8 per channel;
  * the Qwen3 layer with block FP8 at M in {1, 4, 8, 32, 512}.
Every output of a sampled token row is a function of that row alone (the
rounding is per token or per 128-input group), so the oracle quantizes only
the sampled rows and contracts them with the sampled weight rows (whole
128-row blocks for the block scheme).  The activation codes and scales the
call leaves in its staging buffers are compared in full, bit for bit (FP8
codes modulo the sign of zero)."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import assert_within_tol, dev, e4m3_equal_mod_zero, empty, host, torch_mod

pytestmark = pytest.mark.gpu
W8A8, FP8R, FP8B = 0, 1, 2
NAME = {W8A8: "int8", FP8R: "fp8_rowwise", FP8B: "fp8_block"}
GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def quant(scheme, x):
    if scheme == W8A8:
        return O.quant_act_int8(x)
    return O.quant_act_fp8(x, 128 if scheme == FP8B else 0)


def exact(scheme, qx, sx, qw, sw):
    if scheme == W8A8:
        return O.rescale_rowwise(O.contract_int8(qx, qw), sx, sw)
    if scheme == FP8R:
        return O.rescale_rowwise(O.contract_e4m3(qx, qw), sx, sw)
    return O.rescale_block(O.contract_e4m3_blocks(qx, qw), sx, sw)


def run_layer(scheme, shapes, M, seed, n_rows=48, n_cols=256):
    """One layer of the projection set at M tokens; returns the number of
    sampled outputs checked."""
    torch = torch_mod()
    shp = dict((n, (N, K)) for n, N, K in shapes)
    rng = np.random.default_rng(seed)
    checked = 0
    for gi, group in enumerate(GROUPS):
        K = shp[group[0]][1]
        x = W.x_bf16(seed + 17 * gi, M, K, heavy_tail=True)
        ws = []
        for j, name in enumerate(group):
            N = shp[name][0]
            s = seed + 100 * gi + 10 * j
            qw = W.w_int8(s, N, K) if scheme == W8A8 else W.w_e4m3(s, N, K)
            sw = W.scale_bf16(s + 1, (N // 128, K // 128) if scheme == FP8B else (N,))
            ws.append((qw, sw))
        ys = [empty(torch, (M * qw.shape[0] * 2 + 64,), torch.uint8, fill=0xFF) for qw, _ in ws]
        qx = empty(torch, (M, K), torch.uint8, fill=0x55)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
        print(f"{NAME[scheme]} M={M} {'/'.join(group)} K={K}", flush=True)
        Q().qlin_linear(scheme, dev(x), [(dev(qw), dev(sw), y) for (qw, sw), y in zip(ws, ys)], q_x=qx, s_x=sx)
        torch.cuda.synchronize()
        # staging: the full rounding of x, bit for bit
        q_ref, s_ref = quant(scheme, x)
        q_got, s_got = host(qx), host(sx)
        if scheme == W8A8:
            assert np.array_equal(q_got.view(np.int8), q_ref), "int8 codes differ"
        else:
            assert e4m3_equal_mod_zero(q_got, q_ref), "E4M3 codes differ"
        assert np.array_equal(s_got.reshape(s_ref.shape), s_ref), "activation scales differ"
        rows = np.sort(rng.choice(M, min(M, n_rows), replace=False))
        for (qw, sw), y in zip(ws, ys):
            N = qw.shape[0]
            raw = host(y)
            assert (raw[M * N * 2:] == 0xFF).all(), "guard band overwritten"
            yb = raw[:M * N * 2].view(np.uint16).reshape(M, N)
            if scheme == FP8B:
                blocks = np.sort(rng.choice(N // 128, min(N // 128, max(1, n_cols // 128)), replace=False))
                cols = (blocks[:, None] * 128 + np.arange(128)[None, :]).ravel()
                sw_s = sw[blocks]
            else:
                cols = np.sort(rng.choice(N, min(N, n_cols), replace=False))
                sw_s = sw[cols]
            ref = exact(scheme, q_ref[rows], s_ref[rows], qw[cols], sw_s)
            assert_within_tol(yb[np.ix_(rows, cols)], ref, f"{NAME[scheme]} M={M} N={N} K={K}")
            if scheme == W8A8:
                acc = O.contract_int8(q_ref[rows], qw[cols])
                assert np.array_equal(yb[np.ix_(rows, cols)], O.epilogue_f32_order(acc, s_ref[rows], sw_s)), \
                    "bf16 differs from the f32-order epilogue"
            checked += ref.size
    return checked


def test_single_projection_m16_full():
    # one W8A8 projection, M = 16, N = K = 4096, every output checked
    torch = torch_mod()
    M, N, K = 16, 4096, 4096
    x = W.x_bf16(1, M, K)
    qw, sw = W.w_int8(2, N, K), W.scale_bf16(3, N)
    y = empty(torch, (M, N), torch.int16)
    qx = empty(torch, (M, K), torch.uint8)
    sx = empty(torch, (M,), torch.float32)
    Q().qlin_linear(W8A8, dev(x), [(dev(qw), dev(sw), y)], q_x=qx, s_x=sx)
    yb = host(y).view(np.uint16)
    y_bits, y_exact, q_ref, s_ref, acc = O.linear_w8a8(x, qw, sw)
    assert np.array_equal(host(qx).view(np.int8), q_ref) and np.array_equal(host(sx), s_ref)
    assert_within_tol(yb, y_exact, "one W8A8 projection M=16 N=K=4096")
    assert np.array_equal(yb, O.epilogue_f32_order(acc, s_ref, sw))
    # the raw int32 accumulator of the same product
    yi = empty(torch, (M, N), torch.int32)
    Q().qlin_gemm_w8a8(qx, sx, dev(qw), dev(sw), yi, out=Q().OUT_I32)
    assert np.array_equal(host(yi), acc)


@pytest.mark.parametrize("M", [4, 8, 16, 32])
def test_llama_small_m_layer(M):
    assert run_layer(W8A8, W.LLAMA_8B, M, 200 + M) > 0


@pytest.mark.parametrize("M", [4, 32])
def test_llama_fp8_rowwise_small_m_layer(M):
    assert run_layer(FP8R, W.LLAMA_8B, M, 400 + M) > 0


@pytest.mark.parametrize("scheme", [W8A8, FP8R])
@pytest.mark.parametrize("M", [512, 1024])
def test_llama_prefill_layer(scheme, M):
    assert run_layer(scheme, W.LLAMA_8B, M, (300 if scheme == W8A8 else 400) + M) > 0


@pytest.mark.parametrize("M", [1, 4, 8, 32, 512])
def test_qwen3_block_fp8_layer(M):
    assert run_layer(FP8B, W.QWEN3_8B, M, 500 + M) > 0
