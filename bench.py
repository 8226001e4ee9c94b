#!/usr/bin/env python3
"""Benchmark: quantized decoder projections on one MI355X.

Headline (`value`): W8A8 decode at one token -- the Llama-3.1-8B projection set
(per layer q 4096x4096, k/v 1024x4096, o 4096x4096, gate/up 14336x4096,
down 4096x14336), 32 layers with distinct weights (6.98 GB of int8, far above
the 256 MB Infinity Cache).  One step = one decoded token through all 32
layers: per layer four qlin_linear calls (q/k/v, o, gate/up, down), each one
launch that rounds the token to int8 and runs the one-row products of every
projection reading it -- 128 launches, replayed as one HIP graph.
value = algorithmic bytes of the step / step time, in GB/s.

Also reported (`secondary`): the same step as quantize + separate one-row
products; per-shape one-row bandwidth; small-M (4..32) fused-projection
bandwidth; M=512 and 1024 prefill TOPS for W8A8 int8, FP8 per-channel (Llama
shapes) and FP8 block (Qwen3-8B shapes), both as one qlin_linear call per
input group (quantization + one GEMM launch over q/k/v or gate/up) and as
separate per-projection GEMMs.

`roofline` is for the dominant kernel, the fused one-row decode kernel:
achieved = algorithmic bytes per launch / average launch duration measured with
HIP events around a graph of the 128 launches.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same decode workload (layers in order, passing
over the 32 layers again until --cpu-seconds of oracle time are spent).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_INT8_PEAK_TOPS = 5000.0   # dense int8, POP/s -> TOPS
MFMA_FP8_PEAK_TOPS = 5000.0    # dense fp8


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the pages' protocol: median of 10 runs after 3 warm-ups ("Llama 3.1 8B
    # Instruct FP8" benchmark page, section "Every number")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--quick", action="store_true", help="headline only (no secondary sweeps, no CPU baseline)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the CPU-oracle sample")
    ap.add_argument("--sections", default="shapes,configs,smallm,prefill,cpu",
                    help="comma list of the secondary legs to run besides the decode headline: shapes "
                         "(per-shape one-row products), configs (the other workload configurations), "
                         "smallm (products alone at 4..32 tokens), prefill, cpu (the CPU-oracle baseline)")
    ap.add_argument("--pmc-workload", action="store_true",
                    help="for hardware-counter runs: a 1 GiB copy (counter calibration), then two eager "
                         "decode steps; prints no JSON")
    ap.add_argument("--prefill-workload", action="store_true",
                    help="for kernel traces and counters of the prefill path: a 1 GiB copy (counter "
                         "calibration), then for each variant and M the layer set (4 layers, one qlin_linear "
                         "call per input group; Qwen3 shapes for fp8_block), three eager passes each; "
                         "prints no JSON")
    ap.add_argument("--prefill-variants", default="int8,fp8_row",
                    help="comma list of int8, fp8_row, fp8_block for --prefill-workload")
    ap.add_argument("--prefill-m", default="512", help="comma list of token counts for --prefill-workload")
    ap.add_argument("--prefill-packed", action="store_true",
                    help="--prefill-workload runs every projection on packed weights (gate/up as SwiGLU)")
    ap.add_argument("--smallm-workload", action="store_true",
                    help="for kernel traces and counters of the small-M path: a 1 GiB copy, then the W8A8 "
                         "projection M=16 N=K=4096 (32 weight copies) and the W8A8 Llama layer set at M=4, 16, "
                         "32 (4 layers each), one qlin_linear call per input, three eager passes each; "
                         "prints no JSON")
    ap.add_argument("--decode-workload", action="store_true",
                    help="for kernel traces and counters of the one-token path of every scheme: a 1 GiB "
                         "copy (counter calibration), then for each of --decode-schemes, 8 layers of the projection set at M=1 (Qwen3-8B shapes for "
                         "fp8_block), one qlin_linear launch per layer input, three eager passes each; "
                         "prints no JSON")
    ap.add_argument("--decode-schemes", default="int8,fp8_row,fp8_block",
                    help="comma list of int8, fp8_row, fp8_block for --decode-workload")
    ap.add_argument("--smallm-schemes", default="int8",
                    help="comma list of int8, fp8_row, fp8_block for --smallm-workload (int8 also runs the "
                         "16 x 4096 x 4096 projection; fp8_block uses the Qwen3-8B shapes)")
    return ap.parse_args()


class Launcher:
    """Pre-marshalled C-ABI calls (raw pointers), so a step is a list of calls."""

    def __init__(self, Q, torch):
        self.Q = Q
        self.L = Q.lib()
        self.torch = torch
        self.calls = []
        self.keep = []

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def quant_int8(self, x, q, s):
        M, K = x.shape
        self.calls.append((self.L.qlin_quant_act_int8, (x.data_ptr(), M, K, q.data_ptr(), s.data_ptr())))

    def quant_fp8(self, x, q, s, group):
        M, K = x.shape
        self.calls.append((self.L.qlin_quant_act_fp8, (x.data_ptr(), M, K, group, q.data_ptr(), s.data_ptr())))

    def linear(self, scheme, x, segs, out=0, qx=None, sx=None):
        """segs: [(q_w, s_w, y), ...] sharing x."""
        M, K = x.shape
        arr = self.Q.segments_array(segs)
        self.keep.append(arr)
        self.calls.append((self.L.qlin_linear, (scheme, x.data_ptr(), M, K, arr, len(segs), out,
                                                 None if qx is None else qx.data_ptr(),
                                                 None if sx is None else sx.data_ptr())))

    def linear_packed(self, scheme, x, segs, out=0, qx=None, sx=None):
        """segs: [(packed q_w, s_w, y), ...] sharing x (weights in operand order)."""
        M, K = x.shape
        arr = self.Q.segments_array(segs)
        self.keep.append(arr)
        self.calls.append((self.L.qlin_linear_packed, (scheme, x.data_ptr(), M, K, arr, len(segs), out,
                                                        qx.data_ptr(), sx.data_ptr())))

    def linear_weight_only(self, scheme, x, segs, out=0):
        """segs: [(q_w, s_w, y), ...] sharing x (weight-only numerics)."""
        M, K = x.shape
        arr = self.Q.segments_array(segs)
        self.keep.append(arr)
        self.calls.append((self.L.qlin_linear_weight_only, (scheme, x.data_ptr(), M, K, arr, len(segs), out)))

    def linear_swiglu(self, scheme, x, gate, up, h, qx=None, sx=None):
        """gate, up: (q_w, s_w) of one MLP; h [M, I] receives silu(gate) * up."""
        M, K = x.shape
        self.calls.append((self.L.qlin_linear_swiglu, (scheme, x.data_ptr(), M, K, gate[0].data_ptr(),
                                                        gate[1].data_ptr(), up[0].data_ptr(), up[1].data_ptr(),
                                                        gate[0].shape[0], h.data_ptr(),
                                                        None if qx is None else qx.data_ptr(),
                                                        None if sx is None else sx.data_ptr())))

    def linear_swiglu_packed(self, scheme, x, gate, up, h, qx, sx):
        """gate, up: (packed q_w, s_w) of one MLP; h [M, I] receives silu(gate) * up."""
        M, K = x.shape
        self.calls.append((self.L.qlin_linear_swiglu_packed, (scheme, x.data_ptr(), M, K, gate[0].data_ptr(),
                                                               gate[1].data_ptr(), up[0].data_ptr(), up[1].data_ptr(),
                                                               gate[0].shape[0], h.data_ptr(), qx.data_ptr(),
                                                               sx.data_ptr())))

    def gemm(self, fn, qx, sx, qw, sw, y, M, N, K, out=0, path=0):
        f = getattr(self.L, fn + "_ex")
        self.calls.append((f, (qx.data_ptr(), sx.data_ptr(), qw.data_ptr(), sw.data_ptr(), y.data_ptr(),
                               M, N, K, out, path)))

    def run(self, calls=None):
        st = self.stream()
        for f, a in (self.calls if calls is None else calls):
            r = f(*a, st)
            if r != 0:
                raise RuntimeError(f"{f.__name__} failed with status {r}")


def capture(torch, fn, use_graph=True):
    """Return a callable replaying fn (a HIP graph when use_graph)."""
    if not use_graph:
        return fn
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay


def time_runs(torch, fn, reps):
    """Milliseconds of each of `reps` back-to-back calls of fn, from HIP events
    recorded between the calls on the current stream (no synchronization in
    between)."""
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record(st)
    for i in range(reps):
        fn()
        ev[i + 1].record(st)
    ev[-1].synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


def time_events(torch, fn, reps):
    """Median milliseconds per call of fn over `reps` timed calls (the caller
    has run the warm-ups)."""
    return median(time_runs(torch, fn, reps))


def time_warm(torch, fn, reps=10, warmup=3):
    """The pages' protocol for one measurement: `warmup` untimed calls, then
    the median of `reps` timed calls."""
    for _ in range(warmup):
        fn()
    return time_events(torch, fn, reps)


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def decode_bytes(N, K):
    """Algorithmic bytes of one one-row product: weights once, row scales,
    the quantized activation row and its scale, the bf16 output."""
    return N * K + 2 * N + K + 4 + 2 * N


def quant_bytes(M, K):
    return 2 * M * K + M * K + 4 * M


def fused_bytes(K, ns):
    """Algorithmic bytes of one fused projection call at M = 1: the bf16 input
    row once, every weight byte once, the row scales, the bf16 outputs."""
    return 2 * K + sum(N * K + 2 * N + 2 * N for N in ns)


def build_decode(torch, Q, W, layers, dev):
    """32 layers of int8 projections with distinct weights + per-layer inputs.
    F: the fused step (one qlin_linear launch per layer input: q/k/v, o,
    gate/up, down); L: the two-kernel step (quantizer + one-row product per
    projection); G: the one-row products alone; WO: F under weight-only
    numerics; S: F with gate/up as one SwiGLU launch whose output h is down's
    input (returned with its algorithmic bytes)."""
    F = Launcher(Q, torch)
    S = Launcher(Q, torch)
    swiglu_step_bytes = 0
    L = Launcher(Q, torch)
    G = Launcher(Q, torch)
    WO = Launcher(Q, torch)
    gen = torch.Generator(device=dev)
    shapes = dict((n, (N, K)) for n, N, K in W.LLAMA_8B)
    bufs = []
    step_bytes = 0
    gemv_bytes = 0
    fused_step_bytes = 0
    per_shape = {}
    for layer in range(layers):
        gen.manual_seed(100 + layer)
        lw = {}
        for name, N, K in W.LLAMA_8B:
            qw = W.torch_w_int8(torch, gen, N, K, dev)
            sw = W.torch_scale_bf16(torch, gen, (N,), dev)
            y = torch.empty((1, N), dtype=torch.int16, device=dev)
            lw[name] = (qw, sw, y)
        for group in W.INPUT_GROUPS:
            K = shapes[group[0]][1]
            x = W.torch_x_bf16(torch, gen, 1, K, dev)
            q = torch.empty((1, K), dtype=torch.int8, device=dev)
            s = torch.empty((1,), dtype=torch.float32, device=dev)
            L.quant_int8(x, q, s)
            step_bytes += quant_bytes(1, K)
            lw["in_" + group[0]] = (x, q, s)
            F.linear(0, x, [(lw[name][0], lw[name][1], lw[name][2]) for name in group])
            WO.linear_weight_only(0, x, [(lw[name][0], lw[name][1], lw[name][2]) for name in group])
            fused_step_bytes += fused_bytes(K, [shapes[name][0] for name in group])
            if group == ("gate", "up"):
                I = shapes["gate"][0]
                h = torch.empty((1, I), dtype=torch.int16, device=dev)
                lw["h"] = h
                S.linear_swiglu(0, x, lw["gate"][:2], lw["up"][:2], h)
                # bf16 row in, both weights and scales once, h out
                swiglu_step_bytes += 2 * K + 2 * (I * K + 2 * I) + 2 * I
            elif group == ("down",):
                N = shapes["down"][0]
                S.linear(0, lw["h"], [lw["down"]])
                swiglu_step_bytes += fused_bytes(K, [N])
            else:
                S.linear(0, x, [(lw[name][0], lw[name][1], lw[name][2]) for name in group])
                swiglu_step_bytes += fused_bytes(K, [shapes[name][0] for name in group])
            for name in group:
                qw, sw, y = lw[name]
                N, K2 = shapes[name]
                L.gemm("qlin_gemm_w8a8", q, s, qw, sw, y, 1, N, K2)
                G.gemm("qlin_gemm_w8a8", q, s, qw, sw, y, 1, N, K2)
                b = decode_bytes(N, K2)
                step_bytes += b
                gemv_bytes += b
                per_shape.setdefault(name, []).append((q, s, qw, sw, y, N, K2))
        bufs.append(lw)
    return F, L, G, WO, (S, swiglu_step_bytes), bufs, fused_step_bytes, step_bytes, gemv_bytes, per_shape


def prefill_layer_set(torch, Q, W, variant, M, layers, dev, seed0):
    """Projection sweeps at M tokens: a launcher with quant + product per input
    group and one with products only; the fused calls (one per input group),
    with gate/up as one SwiGLU call, and that set with q/k/v, o and down on
    packed weights (rowwise schemes; None for fp8_block).
    variant: int8 | fp8_row | fp8_block."""
    shapes = W.LLAMA_8B if variant != "fp8_block" else W.QWEN3_8B
    shp = dict((n, (N, K)) for n, N, K in shapes)
    full = Launcher(Q, torch)
    prod = Launcher(Q, torch)
    fused = Launcher(Q, torch)
    swiglu = Launcher(Q, torch)     # fused, with gate/up as one SwiGLU launch
    packed = Launcher(Q, torch)     # swiglu's calls with q/k/v, o and down on packed weights
    packed_sg = Launcher(Q, torch)  # swiglu's calls, every projection on packed weights
    packed_all = Launcher(Q, torch)  # fused's calls, every projection on packed weights
    packed.outputs = []
    scheme = {"int8": Q.SCHEME_W8A8, "fp8_row": Q.SCHEME_FP8_ROWWISE, "fp8_block": Q.SCHEME_FP8_BLOCK}[variant]
    gen = torch.Generator(device=dev)
    ops = 0
    keep = []
    fn = {"int8": "qlin_gemm_w8a8", "fp8_row": "qlin_gemm_fp8_rowwise", "fp8_block": "qlin_gemm_fp8_block"}[variant]
    for layer in range(layers):
        gen.manual_seed(seed0 + layer)
        for group in W.INPUT_GROUPS:
            K = shp[group[0]][1]
            x = W.torch_x_bf16(torch, gen, M, K, dev)
            if variant == "int8":
                q = torch.empty((M, K), dtype=torch.int8, device=dev)
                s = torch.empty((M,), dtype=torch.float32, device=dev)
                full.quant_int8(x, q, s)
            else:
                q = torch.empty((M, K), dtype=torch.uint8, device=dev)
                g = 128 if variant == "fp8_block" else 0
                s = torch.empty((M, K // 128) if g else (M,), dtype=torch.float32, device=dev)
                full.quant_fp8(x, q, s, g)
            keep += [x, q, s]
            segs = []
            for name in group:
                N, _ = shp[name]
                if variant == "int8":
                    qw = W.torch_w_int8(torch, gen, N, K, dev)
                else:
                    qw = W.torch_w_e4m3(torch, gen, N, K, dev)
                sws = (N // 128, K // 128) if variant == "fp8_block" else (N,)
                sw = W.torch_scale_bf16(torch, gen, sws, dev)
                y = torch.empty((M, N), dtype=torch.int16, device=dev)
                keep += [qw, sw, y]
                full.gemm(fn, q, s, qw, sw, y, M, N, K)
                prod.gemm(fn, q, s, qw, sw, y, M, N, K)
                segs.append((qw, sw, y))
                ops += 2 * M * N * K
            # the group as one call: quantization + one GEMM launch over its segments
            fused.linear(scheme, x, segs, qx=q, sx=s)
            psegs = []
            for qw, sw, y in segs:
                pw = torch.empty_like(qw)
                Q.qlin_pack_weights(scheme, qw, pw)
                keep.append(pw)
                psegs.append((pw, sw, y))
            packed_all.linear_packed(scheme, x, psegs, qx=q, sx=s)
            if group == ("gate", "up"):
                swiglu.linear_swiglu(scheme, x, segs[0][:2], segs[1][:2], segs[0][2], qx=q, sx=s)
                packed.linear_swiglu(scheme, x, segs[0][:2], segs[1][:2], segs[0][2], qx=q, sx=s)
                packed_sg.linear_swiglu_packed(scheme, x, psegs[0][:2], psegs[1][:2], segs[0][2], q, s)
            else:
                swiglu.linear(scheme, x, segs, qx=q, sx=s)
                packed.linear_packed(scheme, x, psegs, qx=q, sx=s)
                packed_sg.linear_packed(scheme, x, psegs, qx=q, sx=s)
                packed.outputs += [y for _, _, y in segs]
    return full, prod, fused, swiglu, packed, packed_sg, packed_all, ops, keep


def layer_set(torch, Q, W, scheme, shapes, M, layers, dev, seed0):
    """`layers` layers of one projection set with distinct weights, one
    qlin_linear call per layer input (quantization + product; at M = 1 one
    launch).  Returns (launcher, algorithmic bytes, ops, buffers): bytes are
    the bf16 inputs, every weight byte and scale once and the bf16 outputs."""
    shp = dict((n, (N, K)) for n, N, K in shapes)
    block = scheme == Q.SCHEME_FP8_BLOCK
    Lr = Launcher(Q, torch)
    gen = torch.Generator(device=dev)
    nbytes = ops = 0
    keep = []
    for layer in range(layers):
        gen.manual_seed(seed0 + layer)
        for group in W.INPUT_GROUPS:
            K = shp[group[0]][1]
            x = W.torch_x_bf16(torch, gen, M, K, dev)
            qx = sx = None
            if M > 1:
                qx = torch.empty((M, K), dtype=torch.uint8, device=dev)
                sx = torch.empty((M, K // 128) if block else (M,), dtype=torch.float32, device=dev)
            segs = []
            nbytes += 2 * M * K
            for name in group:
                N = shp[name][0]
                if scheme == Q.SCHEME_W8A8:
                    qw = W.torch_w_int8(torch, gen, N, K, dev)
                else:
                    qw = W.torch_w_e4m3(torch, gen, N, K, dev)
                sw = W.torch_scale_bf16(torch, gen, (N // 128, K // 128) if block else (N,), dev)
                y = torch.empty((M, N), dtype=torch.int16, device=dev)
                segs.append((qw, sw, y))
                nbytes += N * K + 2 * sw.numel() + 2 * M * N
                ops += 2 * M * N * K
            keep += [x, qx, sx, segs]
            Lr.linear(scheme, x, segs, qx=qx, sx=sx)
    return Lr, nbytes, ops, keep


def time_launcher(torch, Lr, use_graph, reps=10, warmup=3):
    return time_warm(torch, capture(torch, Lr.run, use_graph), reps, warmup)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# CPU oracle leg
# ---------------------------------------------------------------------------

def cpu_baseline(torch, W, bufs, budget_s, runs=3):
    """Time the CPU oracle (as it stands) on a bounded sample of the decode
    workload, `runs` times (median reported): each run takes whole layers in
    order, passing over the 32 layers again until its share of the time budget
    is spent (host copies of a layer's operands are made once, outside the
    timed region).  Also returns the largest error of the GPU outputs against
    the oracle (checked on the first pass of the first run)."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1

    def to_host(lw):
        groups = []
        for group in W.INPUT_GROUPS:
            x = lw["in_" + group[0]][0].cpu().numpy().view(np.uint16)
            ws = []
            for name in group:
                qw_t, sw_t, y_t = lw[name]
                ws.append((qw_t.cpu().numpy(), sw_t.cpu().numpy().view(np.uint16), y_t.cpu().numpy().view(np.uint16)))
            groups.append((x, ws))
        return groups

    host_layers = []
    per_layer = sum(len(g) for g in W.INPUT_GROUPS)
    check = {"nproj": 0, "max_rel": 0.0, "exact": True}

    def one_run(budget, verify):
        t_total = 0.0
        nbytes = 0
        layers_done = 0
        first = True
        while first or t_total < budget:
            for li, lw in enumerate(bufs):
                if li == len(host_layers):
                    host_layers.append(to_host(lw))
                for x, ws in host_layers[li]:
                    t0 = time.perf_counter()
                    qx, sx = O.quant_act_int8(x)                       # one rounding per layer input
                    outs = []
                    for qw, sw, _ in ws:
                        acc = O.contract_int8(qx, qw)
                        outs.append((acc, O.rescale_rowwise(acc, sx, sw)))
                    t_total += time.perf_counter() - t0
                    nbytes += fused_bytes(x.shape[1], [qw.shape[0] for qw, _, _ in ws])
                    if first and verify:
                        for (qw, sw, yg), (acc, y_exact) in zip(ws, outs):
                            check["nproj"] += 1
                            yf = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                            check["max_rel"] = max(check["max_rel"],
                                                   float(np.max(np.abs(yf - y_exact)) / np.max(np.abs(y_exact))))
                            check["exact"] &= bool(np.array_equal(yg, O.epilogue_f32_order(acc, sx, sw)))
                layers_done += 1
                if t_total >= budget:
                    break
            first = False
        return nbytes / t_total / 1e9, layers_done, t_total

    results = [one_run(budget_s / runs, i == 0) for i in range(runs)]
    rates = [r[0] for r in results]
    return {
        "value": median(rates),
        "unit": "GB/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"median of {runs} runs, each whole decode layers in order over the {len(bufs)}-layer workload "
                  f"for about {budget_s / runs:.0f} s of oracle time ({', '.join(str(r[1]) for r in results)} "
                  f"layers of {per_layer} projections with their int8 activation quantization; GB/s "
                  f"{', '.join(f'{r:.3f}' for r in rates)}); outputs of the first {check['nproj']} projections "
                  f"checked",
    }, check["max_rel"], check["exact"]


# ---------------------------------------------------------------------------

def measured_traffic():
    """HBM bytes per fused decode launch from the committed counter summary
    (profiles/linear_decode_int8_llama8b_traffic.json), or None when the
    kernel's sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "linear_decode_int8_llama8b_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        for name, digest in rec["sources_sha256"].items():
            src = os.path.join(ROOT, "quantized_linear_layers_token_amd", "csrc", name)
            with open(src, "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != digest:
                    return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_linear_layers_token_amd as Q
    import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    use_graph = not args.no_graph

    def copy_calibration():
        # a plain copy of known size (1 GiB read + 1 GiB written) for scaling the byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.prefill_workload:
        copy_calibration()
        for variant in args.prefill_variants.split(","):
            for M in (int(m) for m in args.prefill_m.split(",")):
                _, _, fused, _, packed, packed_sg, packed_all, ops, keep = prefill_layer_set(
                    torch, Q, W, variant, M, 4, dev, {"int8": 300, "fp8_row": 400, "fp8_block": 500}[variant] + M)
                run = packed_sg if args.prefill_packed else fused
                torch.cuda.synchronize()
                for _ in range(3):
                    run.run()
                torch.cuda.synchronize()
                log(f"prefill workload {variant}{' packed' if run is packed else ''}: M={M}, 4 layers, "
                    f"{len(run.calls)} calls per pass x3, {ops} ops per pass")
                del keep, fused, packed, packed_sg, packed_all, run
        return
    if args.decode_workload:
        copy_calibration()
        for sname in args.decode_schemes.split(","):
            scheme = {"int8": Q.SCHEME_W8A8, "fp8_row": Q.SCHEME_FP8_ROWWISE, "fp8_block": Q.SCHEME_FP8_BLOCK}[sname]
            shapes = W.QWEN3_8B if sname == "fp8_block" else W.LLAMA_8B
            Lr, nbytes, ops, keep = layer_set(torch, Q, W, scheme, shapes, 1, 8, dev, 700)
            torch.cuda.synchronize()
            for _ in range(3):
                Lr.run()
            torch.cuda.synchronize()
            log(f"decode workload: {sname} M=1, 8 layers, {len(Lr.calls)} launches per pass x3, "
                f"{nbytes} algorithmic bytes per pass")
            del Lr, keep
        return
    if args.smallm_workload:
        copy_calibration()
        schemes = args.smallm_schemes.split(",")
        for sname in schemes:
            if sname == "int8":
                continue
            scheme = Q.SCHEME_FP8_ROWWISE if sname == "fp8_row" else Q.SCHEME_FP8_BLOCK
            shapes = W.QWEN3_8B if sname == "fp8_block" else W.LLAMA_8B
            for M in (4, 16, 32):
                Lr, nbytes, ops, keep = layer_set(torch, Q, W, scheme, shapes, M, 4, dev, 600 + M)
                torch.cuda.synchronize()
                for _ in range(3):
                    Lr.run()
                torch.cuda.synchronize()
                log(f"small-M workload: {sname} layer M={M}, 4 layers, {len(Lr.calls)} calls per pass x3, "
                    f"{nbytes} algorithmic bytes per pass")
                del Lr, keep
        if "int8" not in schemes:
            return
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        c1 = Launcher(Q, torch)
        keep = []
        for _ in range(32):
            x = W.torch_x_bf16(torch, gen, 16, 4096, dev)
            qw = W.torch_w_int8(torch, gen, 4096, 4096, dev)
            sw = W.torch_scale_bf16(torch, gen, (4096,), dev)
            y = torch.empty((16, 4096), dtype=torch.int16, device=dev)
            qx = torch.empty((16, 4096), dtype=torch.uint8, device=dev)
            sx = torch.empty((16,), dtype=torch.float32, device=dev)
            keep.append((x, qw, sw, y, qx, sx))
            c1.linear(Q.SCHEME_W8A8, x, [(qw, sw, y)], qx=qx, sx=sx)
        torch.cuda.synchronize()
        for _ in range(3):
            c1.run()
        torch.cuda.synchronize()
        log(f"small-M workload: W8A8 M=16 N=K=4096, {len(c1.calls)} calls per pass x3")
        del keep, c1
        for M in (4, 16, 32):
            Lr, nbytes, ops, keep = layer_set(torch, Q, W, Q.SCHEME_W8A8, W.LLAMA_8B, M, 4, dev, 200 + M)
            torch.cuda.synchronize()
            for _ in range(3):
                Lr.run()
            torch.cuda.synchronize()
            log(f"small-M workload: W8A8 Llama layer M={M}, 4 layers, {len(Lr.calls)} calls per pass x3, "
                f"{nbytes} algorithmic bytes per pass")
            del Lr, keep
        return

    # ---- headline: decode, M = 1, 32 distinct layers -------------------------
    log("building decode workload (32 layers, int8)")
    F, L, G, WO, (S, swiglu_step_bytes), bufs, fused_step_bytes, step_bytes, gemv_bytes, per_shape = build_decode(
        torch, Q, W, W.LLAMA_8B_LAYERS, dev)
    torch.cuda.synchronize()
    if args.pmc_workload:
        # calibration: a plain copy of known size (1 GiB read + 1 GiB written),
        # then the decode step's 128 launches, eagerly so each is its own dispatch
        copy_calibration()
        for _ in range(2):
            F.run()
        torch.cuda.synchronize()
        log(f"pmc workload done: copy 1 GiB x2, decode launches {len(F.calls)} x2, "
            f"algorithmic bytes per step {fused_step_bytes}")
        return
    step = capture(torch, F.run, use_graph)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} decode steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    runs = time_runs(torch, step, args.steps)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = median(runs)
    value = fused_step_bytes / (ms * 1e-3) / 1e9
    log(f"decode step median {ms:.4f} ms, mean {sum(runs) / len(runs):.4f} ms (wall {wall_ms:.4f} ms)  "
        f"{value:.1f} GB/s")

    # ---- roofline of the dominant kernel: the fused one-row projection -----
    # (the step is made of these launches only: avg launch = step time / 128)
    n_launch = len(F.calls)
    ms_f = ms
    avg_launch_us = ms_f * 1e3 / n_launch
    bytes_per_launch = fused_step_bytes / n_launch
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "linear_decode_kernel<VAR_INT8,...> (qlin_linear, M=1)",
                "bytes_per_launch": int(bytes_per_launch), "avg_launch_us": round(avg_launch_us, 3),
                "launches": n_launch}
    log(f"fused launches: {n_launch}, avg {avg_launch_us:.3f} us, {achieved:.1f} GB/s")

    secondary = {}
    # the two-kernel form of the same step (quantizer + one-row product per projection)
    two = capture(torch, L.run, use_graph)
    for _ in range(args.warmup):
        two()
    ms_two = time_events(torch, two, args.steps)
    gemv_only = capture(torch, G.run, use_graph)
    for _ in range(args.warmup):
        gemv_only()
    ms_gemv = time_events(torch, gemv_only, args.steps)
    # the same step under weight-only numerics (bf16 input never rounded)
    wo = capture(torch, WO.run, use_graph)
    for _ in range(args.warmup):
        wo()
    ms_wo = time_events(torch, wo, args.steps)
    secondary["decode_weight_only"] = {"ms_per_step": round(ms_wo, 4),
                                       "gbs": round(fused_step_bytes / (ms_wo * 1e-3) / 1e9, 1)}
    # gate/up with SwiGLU in the epilogue, down reading its output
    sg = capture(torch, S.run, use_graph)
    for _ in range(args.warmup):
        sg()
    ms_sg = time_events(torch, sg, args.steps)
    secondary["decode_swiglu_chained"] = {"ms_per_step": round(ms_sg, 4), "launches": len(S.calls),
                                          "gbs": round(swiglu_step_bytes / (ms_sg * 1e-3) / 1e9, 1)}
    log(f"swiglu-chained step {ms_sg:.4f} ms {secondary['decode_swiglu_chained']}")
    secondary["decode_two_kernel"] = {
        "ms_per_step": round(ms_two, 4), "gbs": round(step_bytes / (ms_two * 1e-3) / 1e9, 1),
        "gemv_only_gbs": round(gemv_bytes / (ms_gemv * 1e-3) / 1e9, 1),
        "gemv_avg_launch_us": round(ms_gemv * 1e3 / len(G.calls), 3)}
    log(f"two-kernel step {ms_two:.4f} ms; gemv-only {secondary['decode_two_kernel']}")
    sections = set() if args.quick else set(args.sections.split(","))
    if "shapes" in sections:
        # per-shape one-row bandwidth (all 32 layers of one projection back to back)
        shape_gbs = {}
        for name, items in per_shape.items():
            P = Launcher(Q, torch)
            for q, s, qw, sw, y, N, K in items:
                P.gemm("qlin_gemm_w8a8", q, s, qw, sw, y, 1, N, K)
            fn = capture(torch, P.run, use_graph)
            t = time_warm(torch, fn)
            shape_gbs[name] = round(len(items) * decode_bytes(N, K) / (t * 1e-3) / 1e9, 1)
        secondary["decode_gemv_gbs_per_shape"] = shape_gbs
        log(f"per-shape GB/s {shape_gbs}")

    if "configs" in sections:
        # the five workloads' other configurations, each with qlin_linear
        # (quantization included) over distinct weights larger than the MALL
        cfgs = {}
        # one W8A8 projection M = 16, N = K = 4096 (32 weight copies rotated)
        c1 = Launcher(Q, torch)
        gen = torch.Generator(device=dev)
        gen.manual_seed(1)
        keep = []
        for _ in range(32):
            x = W.torch_x_bf16(torch, gen, 16, 4096, dev)
            qw = W.torch_w_int8(torch, gen, 4096, 4096, dev)
            sw = W.torch_scale_bf16(torch, gen, (4096,), dev)
            y = torch.empty((16, 4096), dtype=torch.int16, device=dev)
            qx = torch.empty((16, 4096), dtype=torch.uint8, device=dev)
            sx = torch.empty((16,), dtype=torch.float32, device=dev)
            keep.append((x, qw, sw, y, qx, sx))
            c1.linear(Q.SCHEME_W8A8, x, [(qw, sw, y)], qx=qx, sx=sx)
        t = time_launcher(torch, c1, use_graph) / 32
        b1 = 2 * 16 * 4096 + 4096 * 4096 + 2 * 4096 + 2 * 16 * 4096
        cfgs["w8a8_M16_N4096_K4096"] = {"us_per_call": round(t * 1e3, 3), "gbs": round(b1 / (t * 1e-3) / 1e9, 1),
                                        "tops": round(2 * 16 * 4096 * 4096 / (t * 1e-3) / 1e12, 2)}
        del keep, c1
        for label, scheme, shapes, M, layers, seed in (
                ("w8a8_llama_M4", Q.SCHEME_W8A8, W.LLAMA_8B, 4, 4, 204),
                ("w8a8_llama_M8", Q.SCHEME_W8A8, W.LLAMA_8B, 8, 4, 208),
                ("w8a8_llama_M16", Q.SCHEME_W8A8, W.LLAMA_8B, 16, 4, 216),
                ("w8a8_llama_M32", Q.SCHEME_W8A8, W.LLAMA_8B, 32, 4, 232),
                ("fp8_rowwise_llama_M1", Q.SCHEME_FP8_ROWWISE, W.LLAMA_8B, 1, W.LLAMA_8B_LAYERS, 401),
                ("fp8_rowwise_llama_M32", Q.SCHEME_FP8_ROWWISE, W.LLAMA_8B, 32, 4, 432),
                ("fp8_block_qwen3_M1", Q.SCHEME_FP8_BLOCK, W.QWEN3_8B, 1, W.QWEN3_8B_LAYERS, 501),
                ("fp8_block_qwen3_M32", Q.SCHEME_FP8_BLOCK, W.QWEN3_8B, 32, 4, 532)):
            Lr, nbytes, ops, keep = layer_set(torch, Q, W, scheme, shapes, M, layers, dev, seed)
            t = time_launcher(torch, Lr, use_graph)
            cfgs[label] = {"ms_per_pass": round(t, 4), "layers": layers, "launches": len(Lr.calls),
                           "gbs": round(nbytes / (t * 1e-3) / 1e9, 1), "frac_hbm": round(nbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                           "tops": round(ops / (t * 1e-3) / 1e12, 2)}
            log(f"{label}: {cfgs[label]}")
            del Lr, keep
            torch.cuda.synchronize()
        secondary["configs_quantized_linear"] = cfgs

    if "smallm" in sections:
        # small batch (M = 4..32) on the fused projections, int8
        small = {}
        gen = torch.Generator(device=dev)
        gen.manual_seed(200)
        fused = [(n, N, K) for n, N, K in W.LLAMA_8B_FUSED]
        # four layers' distinct weights (873 MB, past the 256 MB Infinity Cache), one pass over them per replay
        SL = 4
        wts = [{n: (W.torch_w_int8(torch, gen, N, K, dev), W.torch_scale_bf16(torch, gen, (N,), dev))
                for n, N, K in fused} for _ in range(SL)]
        small_wo = {}
        for M in (4, 8, 16, 32):
            P = Launcher(Q, torch)
            PW = Launcher(Q, torch)
            nb = 0
            nbw = 0
            ops = 0
            keep = []
            for lw in wts:
                for n, N, K in fused:
                    x = W.torch_x_bf16(torch, gen, M, K, dev)
                    q = torch.empty((M, K), dtype=torch.int8, device=dev)
                    s = torch.empty((M,), dtype=torch.float32, device=dev)
                    y = torch.empty((M, N), dtype=torch.int16, device=dev)
                    keep += [x, q, s, y]
                    Q.qlin_quant_act_int8(x, q, s)
                    P.gemm("qlin_gemm_w8a8", q, s, lw[n][0], lw[n][1], y, M, N, K)
                    PW.linear_weight_only(0, x, [(lw[n][0], lw[n][1], y)])
                    nb += N * K + 2 * N + M * K + 4 * M + 2 * M * N
                    nbw += N * K + 2 * N + 2 * M * K + 2 * M * N
                    ops += 2 * M * N * K
            fn = capture(torch, P.run, use_graph)
            t = time_warm(torch, fn)
            small[str(M)] = {"gbs": round(nb / (t * 1e-3) / 1e9, 1), "tops": round(ops / (t * 1e-3) / 1e12, 2),
                             "us_per_layer": round(t * 1e3 / SL, 2)}
            fw = capture(torch, PW.run, use_graph)
            t = time_warm(torch, fw)
            small_wo[str(M)] = {"gbs": round(nbw / (t * 1e-3) / 1e9, 1), "us_per_layer": round(t * 1e3 / SL, 2)}
            del keep
        secondary["small_m_products_only_int8"] = small
        secondary["small_m_weight_only_int8"] = small_wo
        log(f"small-M fused {small}")
        log(f"small-M weight-only {small_wo}")
        del wts

    if "prefill" in sections:
        # prefill TOPS
        for variant, peak in (("int8", MFMA_INT8_PEAK_TOPS), ("fp8_row", MFMA_FP8_PEAK_TOPS),
                              ("fp8_block", MFMA_FP8_PEAK_TOPS)):
            for M in (512, 1024):
                full, prod, fused, swiglu, packed, packed_sg, packed_all, ops, keep = prefill_layer_set(
                    torch, Q, W, variant, M, 4, dev, {"int8": 300, "fp8_row": 400, "fp8_block": 500}[variant] + M)
                f_full = capture(torch, full.run, use_graph)
                f_prod = capture(torch, prod.run, use_graph)
                f_fused = capture(torch, fused.run, use_graph)
                f_sg = capture(torch, swiglu.run, use_graph)
                f_pk = capture(torch, packed.run, use_graph)
                f_pa = capture(torch, packed_all.run, use_graph)
                f_ps = capture(torch, packed_sg.run, use_graph)
                t_full = time_warm(torch, f_full)
                t_prod = time_warm(torch, f_prod)
                t_fused = time_warm(torch, f_fused)
                t_sg = time_warm(torch, f_sg)
                t_pk = time_warm(torch, f_pk)
                t_pa = time_warm(torch, f_pa)
                t_ps = time_warm(torch, f_ps)
                key = f"prefill_{variant}_M{M}"
                secondary[key] = {
                    "tops_fused_linear": round(ops / (t_fused * 1e-3) / 1e12, 1),
                    "frac_fused_linear": round(ops / (t_fused * 1e-3) / 1e12 / peak, 4),
                    "tops_gemm_per_projection": round(ops / (t_prod * 1e-3) / 1e12, 1),
                    "frac_gemm_per_projection": round(ops / (t_prod * 1e-3) / 1e12 / peak, 4),
                    "tops_quant_then_per_projection": round(ops / (t_full * 1e-3) / 1e12, 1),
                    "ms_per_layer_fused": round(t_fused / 4, 4),
                    "tops_fused_linear_swiglu": round(ops / (t_sg * 1e-3) / 1e12, 1),
                    "shapes": "qwen3-8b" if variant == "fp8_block" else "llama-3.1-8b",
                }
                # same outputs as the row-major calls (int8: bit for bit)
                swiglu.run()
                torch.cuda.synchronize()
                ref = [y.clone() for y in packed.outputs]
                for y in packed.outputs:
                    y.fill_(0)
                packed.run()
                torch.cuda.synchronize()
                if variant == "int8":
                    same = all(torch.equal(a, b) for a, b in zip(ref, packed.outputs))
                else:
                    same = all(((a.view(torch.bfloat16).float() - b.view(torch.bfloat16).float()).abs().max()
                                <= 4e-3 * a.view(torch.bfloat16).float().abs().max()).item()
                               for a, b in zip(ref, packed.outputs))
                secondary[key]["packed_matches_row_major"] = bool(same)
                del ref
                secondary[key]["tops_packed_qkv_o_down_swiglu"] = round(ops / (t_pk * 1e-3) / 1e12, 1)
                secondary[key]["frac_packed_qkv_o_down_swiglu"] = round(ops / (t_pk * 1e-3) / 1e12 / peak, 4)
                secondary[key]["ms_per_layer_packed"] = round(t_pk / 4, 4)
                secondary[key]["tops_packed_all"] = round(ops / (t_pa * 1e-3) / 1e12, 1)
                secondary[key]["tops_packed_all_swiglu"] = round(ops / (t_ps * 1e-3) / 1e12, 1)
                secondary[key]["frac_packed_all_swiglu"] = round(ops / (t_ps * 1e-3) / 1e12 / peak, 4)
                log(f"{key}: {secondary[key]}")
                del keep, full, prod, fused, swiglu, packed, packed_sg, packed_all, f_full, f_prod, f_fused, f_sg, f_pk, f_pa, f_ps
                torch.cuda.synchronize()

    cpu = None
    if "cpu" in sections:
        log("CPU oracle sample")
        cpu, max_rel, exact = cpu_baseline(torch, W, bufs, args.cpu_seconds)
        secondary["max_rel_err_vs_oracle"] = max_rel
        secondary["bf16_bitexact_vs_oracle_f32_order"] = exact
        log(f"cpu baseline {cpu}; max rel err {max_rel:.3g}; bitexact {exact}")

    out = {
        "metric": "W8A8 M=1 GEMV HBM GB/s + M=512 int8/fp8 TOPS, Llama-8B projection set",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_mean": round(sum(runs) / len(runs), 4),
        "timing": f"median of {args.steps} steps after {args.warmup} warm-up steps (HIP events between steps)",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "Llama-3.1-8B W8A8 decode, M=1, 32 layers with distinct int8 weights (q, k, v, o, gate, "
                        "up, down as separate tensors); per token 128 fused launches (per-token int8 activation "
                        "rounding + one-row products of the projections reading that input), " +
                        ("replayed as one HIP graph" if use_graph else "launched eagerly"),
            "bytes_per_step": fused_step_bytes,
            "hip_graph": use_graph,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
