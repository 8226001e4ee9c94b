"""The library's calls captured in one HIP graph and replayed: every launch
form of qlin_linear / qlin_linear_swiglu (one token; two tokens; four tokens
rounded in the small-M kernel; quantizer + small-M kernel; quantizer + tiled
GEMM, including its 8-wavefront 256 x 256 tile; quantizer + the packed-weight
GEMM on both token-tile widths, block FP8 included) must reproduce the eager results bit for bit on every replay, with
eager work (output poisoning, another library call) between the replays."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import dev, empty, host, torch_mod

pytestmark = pytest.mark.gpu
W8A8, FP8R, FP8B = 0, 1, 2


def Q():
    import quantized_linear_layers_token_amd as q
    return q


def build(torch):
    """Calls (closures) covering every launch form, and their outputs."""
    calls, outs = [], []
    forms = [(W8A8, 1, 4096), (W8A8, 2, 1024), (FP8R, 4, 4096), (W8A8, 16, 4096), (FP8R, 64, 1024),
             (FP8B, 4, 1024), (FP8B, 40, 512)]
    for i, (scheme, M, K) in enumerate(forms):
        x = dev(W.x_bf16(9900 + i, M, K))
        ns = [256, 128]
        segs = []
        for j, n in enumerate(ns):
            qw = W.w_int8(9910 + 10 * i + j, n, K) if scheme == W8A8 else W.w_e4m3(9910 + 10 * i + j, n, K)
            sw = W.scale_bf16(9950 + 10 * i + j, (n // 128, K // 128) if scheme == FP8B else (n,))
            y = empty(torch, (M, n), torch.int16)
            segs.append((dev(qw), dev(sw), y))
            outs.append(y)
        qx = empty(torch, (M, K), torch.uint8)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32)
        outs += [qx, sx]
        calls.append(lambda s=scheme, x=x, segs=segs, qx=qx, sx=sx: Q().qlin_linear(s, x, segs, q_x=qx, s_x=sx))
    # FP8 rowwise, 257 tokens over two 14336-row segments: the 256 x 256 tiles
    x = dev(W.x_bf16(9970, 257, 128))
    segs = []
    for j in range(2):
        y = empty(torch, (257, 14336), torch.int16)
        segs.append((dev(W.w_e4m3(9971 + j, 14336, 128)), dev(W.scale_bf16(9973 + j, (14336,))), y))
        outs.append(y)
    qx = empty(torch, (257, 128), torch.uint8)
    sx = empty(torch, (257,), torch.float32)
    outs += [qx, sx]
    calls.append(lambda x=x, segs=segs, qx=qx, sx=sx: Q().qlin_linear(FP8R, x, segs, q_x=qx, s_x=sx))
    # packed weights: W8A8 on 64-token tiles, FP8 rowwise on 128-token tiles
    for i, (scheme, M, K, ns) in enumerate([(W8A8, 100, 512, [256, 128]), (FP8R, 300, 256, [4096, 4096]),
                                            (FP8B, 150, 512, [256, 128])]):
        x = dev(W.x_bf16(9960 + i, M, K))
        segs = []
        for j, n in enumerate(ns):
            qw = dev(W.w_int8(9962 + 2 * i + j, n, K) if scheme == W8A8 else W.w_e4m3(9962 + 2 * i + j, n, K))
            pw = torch.empty_like(qw)
            Q().qlin_pack_weights(scheme, qw, pw)
            y = empty(torch, (M, n), torch.int16)
            sws = (n // 128, K // 128) if scheme == FP8B else (n,)
            segs.append((pw, dev(W.scale_bf16(9966 + 2 * i + j, sws)), y))
            outs.append(y)
        qx = empty(torch, (M, K), torch.uint8)
        sx = empty(torch, (M, K // 128) if scheme == FP8B else (M,), torch.float32)
        outs += [qx, sx]
        calls.append(lambda s=scheme, x=x, segs=segs, qx=qx, sx=sx: Q().qlin_linear_packed(s, x, segs, q_x=qx, s_x=sx))
    # SwiGLU on packed weights, block FP8
    x = dev(W.x_bf16(9975, 100, 256))
    pair = []
    for j in range(2):
        pw = torch.empty((256, 256), dtype=torch.uint8, device="cuda")
        Q().qlin_pack_weights(FP8B, dev(W.w_e4m3(9976 + j, 256, 256)), pw)
        pair.append((pw, dev(W.scale_bf16(9978 + j, (2, 2), 1e-4, 5e-4))))
    h = empty(torch, (100, 256), torch.int16)
    qx = empty(torch, (100, 256), torch.uint8)
    sx = empty(torch, (100, 2), torch.float32)
    outs += [h, qx, sx]
    calls.append(lambda x=x, p=pair, h=h, qx=qx, sx=sx: Q().qlin_linear_swiglu_packed(FP8B, x, p[0], p[1], h, q_x=qx,
                                                                                        s_x=sx))
    for i, (M, K) in enumerate([(1, 4096), (4, 1024), (40, 512)]):
        x = dev(W.x_bf16(9980 + i, M, K))
        gate = (dev(W.w_int8(9985 + i, 256, K)), dev(W.scale_bf16(9988 + i, 256, 1e-4, 5e-4)))
        up = (dev(W.w_int8(9991 + i, 256, K)), dev(W.scale_bf16(9994 + i, 256, 1e-4, 5e-4)))
        h = empty(torch, (M, 256), torch.int16)
        qx = empty(torch, (M, K), torch.uint8)
        sx = empty(torch, (M,), torch.float32)
        outs += [h, qx, sx]
        calls.append(lambda x=x, g=gate, u=up, h=h, qx=qx, sx=sx: Q().qlin_linear_swiglu(W8A8, x, g, u, h, q_x=qx, s_x=sx))
    return calls, outs


def test_graph_replays_match_eager():
    torch = torch_mod()
    calls, outs = build(torch)
    for c in calls:
        c()
    torch.cuda.synchronize()
    ref = [host(o).copy() for o in outs]
    # capture (warm up on a side stream first, as graph capture expects)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    other_x = dev(W.x_bf16(9999, 3, 256))
    other_q = empty(torch, (3, 256), torch.int8)
    other_s = empty(torch, (3,), torch.float32)
    for rep in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0xA5 + rep)          # eager poisoning between replays
        Q().qlin_quant_act_int8(other_x, other_q, other_s)   # an unrelated eager library call
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert np.array_equal(host(o), r), f"replay {rep}: output {i} differs from the eager result"
