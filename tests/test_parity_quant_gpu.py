"""GPU parity of the activation quantizers against the CPU oracle: codes and
scales must be bit-exact (E4M3 codes modulo the sign of zero)."""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import dev, e4m3_equal_mod_zero, empty, host, torch_mod

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def run_int8(x_bits):
    torch = torch_mod()
    M, K = x_bits.shape
    x = dev(x_bits)
    q = empty(torch, (M, K), torch.int8, fill=0x55)
    s = empty(torch, (M,), torch.float32, fill=0x55)
    Q().qlin_quant_act_int8(x, q, s)
    return host(q), host(s)


def run_fp8(x_bits, group):
    torch = torch_mod()
    M, K = x_bits.shape
    x = dev(x_bits)
    q = empty(torch, (M, K), torch.uint8, fill=0x55)
    s = empty(torch, (M, K // 128) if group else (M,), torch.float32, fill=0x55)
    Q().qlin_quant_act_fp8(x, q, s, group=group)
    return host(q), host(s)


SHAPES = [(1, 16), (1, 4096), (3, 4112), (16, 4096), (33, 14336), (2, 12288), (5, 2048 * 16 + 2048), (64, 48)]


@pytest.mark.parametrize("M,K", SHAPES)
def test_quant_int8_bitexact(M, K):
    x = W.x_bf16(1000 + M + K, M, K)
    if M > 2:
        x[1] = 0                                  # an all-zero token
    q, s = run_int8(x)
    qo, so = O.quant_act_int8(x)
    assert np.array_equal(q, qo)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("M,K", SHAPES)
def test_quant_fp8_token_bitexact(M, K):
    x = W.x_bf16(2000 + M + K, M, K)
    if M > 2:
        x[2] = 0
    q, s = run_fp8(x, 0)
    qo, so = O.quant_act_fp8(x, 0)
    assert e4m3_equal_mod_zero(q, qo)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))


@pytest.mark.parametrize("M,K", [(1, 128), (1, 4096), (3, 12288), (32, 4096), (17, 384), (512, 4096)])
def test_quant_fp8_group_bitexact(M, K):
    x = W.x_bf16(3000 + M + K, M, K)
    x[0, 128:256] = 0                             # an all-zero group (when K > 128)
    q, s = run_fp8(x, 128)
    qo, so = O.quant_act_fp8(x, 128)
    assert e4m3_equal_mod_zero(q, qo)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32))


def test_quant_golden_rows_on_gpu():
    with open(os.path.join(GOLD, "int8_token_rows.json")) as fh:
        gd = json.load(fh)
    x = np.array([[int(v, 16) for v in r] for r in gd["x_bf16"]], np.uint16)
    x = np.concatenate([x, np.zeros_like(x)], axis=1)          # K = 16 (zeros change nothing)
    q, s = run_int8(x)
    assert np.array_equal(q[:, :8], np.array(gd["q"], np.int8)) and not q[:, 8:].any()
    with open(os.path.join(GOLD, "e4m3_token_rows.json")) as fh:
        gd = json.load(fh)
    x = np.array([[int(v, 16) for v in r] for r in gd["x_bf16"]], np.uint16)
    x = np.concatenate([x, np.zeros_like(x)], axis=1)
    q, s = run_fp8(x, 0)
    exp = np.array([[int(v, 16) for v in r] for r in gd["q"]], np.uint8)
    assert e4m3_equal_mod_zero(q[:, :8], exp)
    assert list(map(float, s)) == gd["s"]


def test_e4m3_encode_every_bf16_value():
    # Rows whose absmax is 448 have s = inv = 1, so every other element is encoded
    # as it is: this walks the hardware conversion over every finite bf16 value in
    # [-448, 448] (subnormals, exact ties, the saturation edge).
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_bits_to_f32(bits)
    keep = np.isfinite(f) & (np.abs(f) <= 448)
    vals = bits[keep]
    per = 15
    pad = (-len(vals)) % per
    vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, per)
    x = np.concatenate([np.full((vals.shape[0], 1), 0x43E0, np.uint16), vals], axis=1)  # 448 first
    q, s = run_fp8(x, 0)
    qo, so = O.quant_act_fp8(x, 0)
    assert (so == 1.0).all() and (s == 1.0).all()
    assert e4m3_equal_mod_zero(q, qo)


def test_int8_rounding_ties_and_subnormal_inputs():
    # absmax 127 -> s = inv = 1: codes are x rounded half-to-even; bf16 subnormal
    # inputs (bf16 keeps f32's exponent range) must not be flushed before scaling.
    ties = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5, 3.5, 4.5, 127.0, 0.25, 1e-39, -1e-39, 2.0 ** -133, 0.0],
                    np.float32)
    bits = (ties.view(np.uint32) >> 16).astype(np.uint16)
    x = bits[None, :]
    q, s = run_int8(x)
    qo, so = O.quant_act_int8(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)
    # bf16 subnormal inputs scaled by a large (finite) inverse scale: absmax is the
    # normal value 2^-120 (int8) / 2^-118 (E4M3), so 127/a and 448/a stay finite and
    # m * 2^-133 * inv lands on codes 0..2 (int8) or a few E4M3 steps; flushing the
    # subnormal inputs to zero would change them.
    subs = np.array([1, 32, 33, 64, 100, 127, 0x8001, 0x8021, 0x8040, 0x807F, 0x0050, 0x8050, 0x0011, 0x0003, 0x0000],
                    np.uint16)
    for lead, run, quant in ((0x0380, run_int8, O.quant_act_int8),
                             (0x0480, lambda v: run_fp8(v, 0), lambda v: O.quant_act_fp8(v, 0))):
        row = np.concatenate([[lead], subs]).astype(np.uint16)[None, :]
        q, s = run(row)
        qo, so = quant(row)
        assert np.array_equal(s.view(np.uint32), so.view(np.uint32))
        assert e4m3_equal_mod_zero(q.view(np.uint8), qo.view(np.uint8))
        assert np.count_nonzero(qo.view(np.uint8) & 0x7F) > 5          # the case is not all zeros


def test_quant_large_prefill_bitexact():
    # the prefill activation shape (M = 1024, K = 4096) with heavy-tailed outliers
    x = W.x_bf16(3100, 1024, 4096, heavy_tail=True)
    q, s = run_int8(x)
    qo, so = O.quant_act_int8(x)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


def test_quant_m0_noop_and_guard():
    torch = torch_mod()
    x = dev(W.x_bf16(5, 2, 64))
    q = empty(torch, (2, 64), torch.int8, fill=0x5A)
    s = empty(torch, (2,), torch.float32, fill=0x5A)
    Q().lib().qlin_quant_act_int8(x.data_ptr(), 0, 64, q.data_ptr(), s.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert (host(q).view(np.uint8) == 0x5A).all() and (host(s).view(np.uint8) == 0x5A).all()
    # guard bytes right after q and s stay untouched
    big_q = empty(torch, (3 * 64 + 64,), torch.int8, fill=0x77)
    big_s = empty(torch, (3 + 16,), torch.float32, fill=0x77)
    xx = dev(W.x_bf16(6, 3, 64))
    st = Q().lib().qlin_quant_act_int8(xx.data_ptr(), 3, 64, big_q.data_ptr(), big_s.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert (host(big_q)[192:].view(np.uint8) == 0x77).all()
    assert (host(big_s)[3:].view(np.uint8) == 0x77).all()
