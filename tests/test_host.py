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
    with pytest.raises(Q.QlinError) as e:      # no segments: rejected by the library before any launch
        Q.qlin_linear(Q.SCHEME_W8A8, x, [], stream=0)
    assert e.value.status == Q.QLIN_ERR_SHAPE
