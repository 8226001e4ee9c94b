"""GPU parity of the gate/up pair with SwiGLU applied on the way out
(qlin_linear_swiglu) against the CPU oracle: the one-launch path (M = 1), the
small-M matrix-core kernel (2..32 tokens, or K past the one-launch limit; up to
4 tokens of up to 4096 inputs rounded inside it) and the tiled GEMM (more than
32 tokens), for the three schemes.

Bound.  g and u on the device are the projections under their own tolerance
(|dg| <= TOL max|g_ref|, likewise u; the projection tests hold them to it).
silu is 1.1-Lipschitz, each of the two further bf16 roundings adds at most
2^-8 of its value, so per element
    |h - silu(g) u| <= ds (|u| + du) + |silu(g)| du + 2^-8 (|silu(g)| + ds)(|u| + du),
    ds = 1.1 dg + 2^-8 (|silu(g)| + 1.1 dg),
with g, u the exact (unrounded) projections.  For W8A8 the accumulators are
exact integers and the epilogue order is fixed, so g and u match the oracle's
f32-order values bit for bit: h must then equal the oracle chain except where
the f32 silu rounds to the other bf16 neighbour (at most one bf16 step of
silu(g), times |u|), which the test also bounds in number."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import TOL, bf16_to_f64, dev, e4m3_equal_mod_zero, empty, host, torch_mod

pytestmark = pytest.mark.gpu
W8A8, FP8R, FP8B = 0, 1, 2
NAME = {W8A8: "int8", FP8R: "fp8_rowwise", FP8B: "fp8_block"}


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def make_pair(scheme, seed, I, K):
    # scales chosen so that the projections are O(1): silu's curved part is exercised
    lo, hi = (1e-4, 5e-4) if K <= 4096 else (5e-5, 2e-4)
    pair = []
    for i in range(2):
        qw = W.w_int8(seed + 10 * i, I, K) if scheme == W8A8 else W.w_e4m3(seed + 10 * i, I, K)
        sw = W.scale_bf16(seed + 10 * i + 1, (I // 128, K // 128) if scheme == FP8B else (I,), lo, hi)
        pair.append((qw, sw))
    return pair


def run(scheme, x, gate, up, staged):
    torch = torch_mod()
    M, K = x.shape
    I = gate[0].shape[0]
    h = empty(torch, (M * I * 2 + 64,), torch.uint8, fill=0xFF)
    qx = sx = None
    if staged or not (M == 1 and K <= 16384 or M <= 4 and K <= 4096):   # staging required
        qx = empty(torch, (M, K), torch.uint8, fill=0x55)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32, fill=0x55)
    Q().qlin_linear_swiglu(scheme, dev(x), (dev(gate[0]), dev(gate[1])), (dev(up[0]), dev(up[1])), h,
                           q_x=qx, s_x=sx)
    raw = host(h)
    assert (raw[M * I * 2:] == 0xFF).all(), "guard band overwritten"
    return (raw[:M * I * 2].view(np.uint16).reshape(M, I), None if qx is None else host(qx),
            None if sx is None else host(sx))


def check(scheme, x, gate, up, h_bits, what):
    h_or, g_bits, u_bits, g, u = O.swiglu_gate_up(x, gate, up, NAME[scheme])
    h = bf16_to_f64(h_bits)
    assert np.isfinite(h).all(), f"{what}: non-finite output"
    dg = TOL * np.abs(g).max()
    du = TOL * np.abs(u).max()
    s = O.silu(g)
    ds = 1.1 * dg + 2.0 ** -8 * (np.abs(s) + 1.1 * dg) + 1e-30
    bound = ds * (np.abs(u) + du) + np.abs(s) * du + 2.0 ** -8 * (np.abs(s) + ds) * (np.abs(u) + du)
    err = np.abs(h - s * u)
    assert np.all(err <= bound), f"{what}: worst excess {np.max(err - bound):.3g}"
    if scheme == W8A8:
        _, _, qx, sx, acc = O.linear_w8a8(x, *gate)
        g32 = O.epilogue_f32_order(acc, sx, gate[1])
        u32 = O.epilogue_f32_order(O.linear_w8a8(x, *up)[4], sx, up[1])
        s32 = O.round_to_bf16_bits(O.silu(bf16_to_f64(g32)))
        chain = O.round_to_bf16_bits(bf16_to_f64(s32) * bf16_to_f64(u32))
        same = h_bits == chain
        assert same.mean() >= 0.999, f"{what}: only {same.mean():.5f} of the outputs match the oracle chain"
        step = 2.0 ** -7 * np.abs(bf16_to_f64(s32)) * np.abs(bf16_to_f64(u32))
        assert np.all(np.abs(h - bf16_to_f64(chain)) <= 2 * step + 1e-30), f"{what}: off the chain by more than a step"
    return h_or


CASES = [
    # (M, K, I)
    (1, 128, 128),
    (1, 4096, 256),        # one-launch path, one gate/up pair per wavefront
    (1, 4096, 200),        # ragged I (rowwise schemes only)
    (1, 8192, 384),        # two pairs per wavefront in turn
    (1, 14336, 128),
    (1, 16512, 128),       # K past the one-launch limit: small-M kernel at M = 1
    (2, 1024, 256),
    (4, 4096, 8192),       # rounded in the kernel, wide tiles
    (3, 4112, 256),        # just past the in-kernel rounding: staged
    (5, 4096, 384),
    (17, 1152, 256),       # two token tiles
    (3, 512, 8192),        # wide small-M tiles (32 gate + 32 up rows)
    (8, 4096, 8192),       # staged, wide tiles, one token tile
    (24, 4096, 8192),      # staged, wide tiles, two token tiles
    (32, 4096, 200),
    (33, 512, 384),        # tiled GEMM
    (100, 1024, 200),      # ragged tiles, I % 8 != 0 stores
    (300, 512, 2048),
    (640, 128, 2560),      # 128 x 128 tiles
    (257, 128, 14336),     # FP8 rowwise: 256 x 256 tiles, ragged second token tile
]


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
@pytest.mark.parametrize("M,K,I", CASES)
def test_swiglu_matches_oracle(scheme, M, K, I):
    if scheme == FP8B and (I % 128 or K % 128):
        pytest.skip("block scheme needs I % 128 == 0 and K % 128 == 0")
    print(f"swiglu {NAME[scheme]} M={M} K={K} I={I}", flush=True)
    x = W.x_bf16(9000 + M + K, M, K)
    gate, up = make_pair(scheme, 9100 + I + K, I, K)
    h_bits, _, _ = run(scheme, x, gate, up, staged=False)
    check(scheme, x, gate, up, h_bits, f"swiglu {NAME[scheme]} M={M} K={K} I={I}")


@pytest.mark.parametrize("scheme", [W8A8, FP8R, FP8B])
def test_swiglu_one_launch_writes_codes(scheme):
    # M = 1 with staging given: the launch also writes the rounding of x
    M, K, I = 1, 4096, 256
    x = W.x_bf16(9300, M, K)
    gate, up = make_pair(scheme, 9310, I, K)
    h_bits, qx, sx = run(scheme, x, gate, up, staged=True)
    check(scheme, x, gate, up, h_bits, f"swiglu codes {NAME[scheme]}")
    if scheme == W8A8:
        q_ref, s_ref = O.quant_act_int8(x)
        assert np.array_equal(qx.view(np.int8), q_ref) and np.array_equal(sx, s_ref)
    else:
        q_ref, s_ref = O.quant_act_fp8(x, 128 if scheme == FP8B else 0)
        assert e4m3_equal_mod_zero(qx, q_ref) and np.array_equal(sx.reshape(s_ref.shape), s_ref)


def test_swiglu_matches_two_projections_then_silu():
    # the fused epilogue against the unfused pair: qlin_linear into g and u,
    # then the same chain on the host from the device's own g and u
    torch = torch_mod()
    M, K, I = 48, 1024, 384
    x = W.x_bf16(9400, M, K)
    gate, up = make_pair(W8A8, 9410, I, K)
    g = empty(torch, (M, I), torch.int16)
    u = empty(torch, (M, I), torch.int16)
    qx = empty(torch, (M, K), torch.uint8)
    sx = empty(torch, (M,), torch.float32)
    Q().qlin_linear(W8A8, dev(x), [(dev(gate[0]), dev(gate[1]), g), (dev(up[0]), dev(up[1]), u)], q_x=qx, s_x=sx)
    g_bits, u_bits = host(g).view(np.uint16), host(u).view(np.uint16)
    h_bits, _, _ = run(W8A8, x, gate, up, staged=False)
    s = O.round_to_bf16_bits(O.silu(bf16_to_f64(g_bits)))
    chain = O.round_to_bf16_bits(bf16_to_f64(s) * bf16_to_f64(u_bits))
    assert (h_bits == chain).mean() >= 0.999


def test_swiglu_validation():
    torch = torch_mod()
    q = Q()
    K, I = 256, 128
    x = dev(W.x_bf16(9500, 2, K))
    gq, gs = dev(W.w_int8(9501, I, K)), dev(W.scale_bf16(9502, I))
    uq, us = dev(W.w_int8(9503, I, K)), dev(W.scale_bf16(9504, I))
    h = empty(torch, (2, I), torch.int16)
    x5, h5 = dev(W.x_bf16(9505, 5, K)), empty(torch, (5, I), torch.int16)
    with pytest.raises(q.QlinError) as e:          # more than 4 tokens need the staging buffers
        q.qlin_linear_swiglu(W8A8, x5, (gq, gs), (uq, us), h5)
    assert e.value.status == q.QLIN_ERR_NULL
    q.qlin_linear_swiglu(W8A8, x, (gq, gs), (uq, us), h)   # two tokens: one launch, staging optional
    qx = empty(torch, (2, K), torch.uint8)
    sx = empty(torch, (2,), torch.float32)
    with pytest.raises(q.QlinError) as e:          # h over the gate weights
        q.qlin_linear_swiglu(W8A8, x, (gq, gs), (uq, us), gq, q_x=qx, s_x=sx)
    assert e.value.status == q.QLIN_ERR_ALIAS
    sxb = empty(torch, (2, K // 128), torch.float32)
    with pytest.raises(q.QlinError) as e:          # block scheme with I % 128 != 0
        q.qlin_linear_swiglu(FP8B, x, (gq[:64], gs), (uq[:64], us), h, q_x=qx, s_x=sxb)
    assert e.value.status == q.QLIN_ERR_SHAPE
    q.qlin_linear_swiglu(W8A8, x[:0], (gq, gs), (uq, us), h, q_x=qx, s_x=sx)   # M = 0: nothing to do
