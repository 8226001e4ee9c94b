"""Host-side logic (CPU, no GPU): the benchmark's byte accounting and its
one-GPU contract, and the Python binding's argument checks that run before
any work reaches the device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                      # no JSON line for an unsupported run


def test_decode_step_bytes():
    import bench
    import workloads as W
    shp = {n: (N, K) for n, N, K in W.LLAMA_8B}
    per_layer = sum(bench.fused_bytes(shp[g[0]][1], [shp[n][0] for n in g]) for g in W.INPUT_GROUPS)
    # counted independently: every int8 weight once, a bf16 scale and a bf16
    # output per weight row, one bf16 input row per input group
    weights = sum(N * K for _, N, K in W.LLAMA_8B)
    rows = sum(N for _, N, _ in W.LLAMA_8B)
    inputs = sum(2 * shp[g[0]][1] for g in W.INPUT_GROUPS)
    assert per_layer == weights + 4 * rows + inputs == 218329088
    assert 32 * per_layer == 6986530816        # the decode step's bytes_per_step
    # one-row product with a pre-quantized input: codes and scale in, not bf16
    assert bench.decode_bytes(4096, 4096) == 4096 * 4096 + 4 * 4096 + 4096 + 4
    assert bench.quant_bytes(16, 4096) == 16 * 4096 * 3 + 16 * 4


def test_binding_rejects_bad_arguments():
    import torch
    import quantized_linear_layers_token_amd as Q
    w = torch.zeros((64, 256), dtype=torch.int8)
    with pytest.raises(ValueError):            # x must be 2-D
        Q.qlin_linear(Q.SCHEME_W8A8, torch.zeros(256, dtype=torch.int16), [(w, None, None)], stream=0)
    x = torch.zeros((1, 256), dtype=torch.int16)
    with pytest.raises(ValueError):            # q_w must be [n, K]
        Q.qlin_linear(Q.SCHEME_W8A8, x, [(torch.zeros((64, 128), dtype=torch.int8), None, None)], stream=0)
    with pytest.raises(ValueError):
        Q.qlin_linear_weight_only(Q.SCHEME_W8A8, x, [(torch.zeros((64, 128), dtype=torch.int8), None, None)],
                                  stream=0)
    # no segments: rejected by the library before any launch (fake address, never dereferenced)
    arr = Q.segments_array([])
    assert Q.lib().qlin_linear(Q.SCHEME_W8A8, 0x10000000, 1, 256, arr, 0, Q.OUT_BF16, None, None,
                               None) == Q.QLIN_ERR_SHAPE


def test_binding_checks_buffers_before_the_library():
    """Every tensor is checked for contiguity, element size and capacity, and
    for being on the device, before its address is handed over: the library
    sees only pointers and would write past an undersized buffer."""
    import torch
    import quantized_linear_layers_token_amd as Q
    M, N, K = 4, 64, 256
    x = torch.zeros((M, K), dtype=torch.int16)
    qx = torch.zeros((M, K), dtype=torch.int8)
    sx = torch.zeros((M,), dtype=torch.float32)
    qw = torch.zeros((N, K), dtype=torch.int8)
    sw = torch.zeros((N,), dtype=torch.int16)
    y = torch.zeros((M, N), dtype=torch.int16)

    def rejects(fn, *a, match, **k):
        with pytest.raises(ValueError, match=match):
            fn(*a, **k, stream=0)

    # output too small for the out mode (bf16 fits, i32 does not), scale arrays too short
    rejects(Q.qlin_gemm_w8a8, qx, sx, qw, sw, y, out=Q.OUT_I32, match="y holds")
    rejects(Q.qlin_gemm_w8a8, qx, sx[:2], qw, sw, y, match="s_x holds")
    rejects(Q.qlin_gemm_fp8_rowwise, qx, sx, qw, sw[:10], y, match="s_w holds")
    rejects(Q.qlin_gemm_fp8_block, qx, sx, qw[:128 if N >= 128 else N], sw, y, match="s_x holds")
    # element sizes: codes are bytes, activations 2-byte, scales 4-/2-byte
    rejects(Q.qlin_gemm_w8a8, qx.to(torch.int16), sx, qw, sw, y, match="q_x must have 1-byte")
    rejects(Q.qlin_gemm_w8a8, qx, sx.to(torch.float64), qw, sw, y, match="s_x must have 4-byte")
    rejects(Q.qlin_quant_act_int8, x.to(torch.float32), qx, sx, match="x must have 2-byte")
    rejects(Q.qlin_quant_act_int8, x, qx[:2], sx, match="q holds")
    rejects(Q.qlin_quant_act_fp8, x, qx, sx, group=128, match="s holds")
    rejects(Q.qlin_gemv_w8a8, qx[0], sx, qw, sw, torch.zeros(N - 1, dtype=torch.int16), match="y holds")
    # non-contiguous
    rejects(Q.qlin_gemm_w8a8, qx, sx, qw, sw, torch.zeros((N, M), dtype=torch.int16).t(), match="contiguous")
    # fused calls: segment outputs, staging buffers and SwiGLU's h
    rejects(Q.qlin_linear, Q.SCHEME_W8A8, x, [(qw, sw, y[:2])], match="segment 0 y holds")
    rejects(Q.qlin_linear, Q.SCHEME_W8A8, x, [(qw, sw, y)], q_x=qx[:1], s_x=sx, match="q_x holds")
    rejects(Q.qlin_linear_weight_only, Q.SCHEME_W8A8, x, [(qw, sw[:3], y)], match="segment 0 s_w holds")
    rejects(Q.qlin_linear_swiglu, Q.SCHEME_W8A8, x, (qw, sw), (qw, sw), y[:1], match="h holds")
    # everything sized right, but host memory: refused before the library sees it
    rejects(Q.qlin_gemm_w8a8, qx, sx, qw, sw, y, match="device tensor")
    rejects(Q.qlin_linear, Q.SCHEME_W8A8, x, [(qw, sw, y)], q_x=qx, s_x=sx, match="device tensor")
