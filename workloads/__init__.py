"""Seeded synthetic inputs and projection shape sets.

This module holds no arithmetic of the quantized projection itself: it only
draws random operands with the shapes, dtypes and value distributions of the
workloads, as raw bit patterns (bf16 as uint16, int8, E4M3 codes as uint8).
Both the CPU oracle's callers and the GPU callers take their inputs from here.

Shapes come from the "Command line" sections of the Llama 3.1 8B Instruct W8A8
model card (H=4096, Heads=32, KvHeads=8, Inner=14336, Layers=32) and of the
Qwen3 8B FP8 model card (H=4096, Heads=32, KvHeads=8, HeadDim=128,
Inner=12288, Layers=36).  A weight is [N, K]: N output rows, K inputs.
"""
from __future__ import annotations

import numpy as np

# (name, N, K) for each decoder projection of one layer.
LLAMA_8B = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 14336, 4096),
    ("up", 14336, 4096),
    ("down", 4096, 14336),
)
LLAMA_8B_LAYERS = 32
# Same layer with q/k/v and gate/up concatenated along N.
LLAMA_8B_FUSED = (
    ("qkv", 6144, 4096),
    ("o", 4096, 4096),
    ("gate_up", 28672, 4096),
    ("down", 4096, 14336),
)
QWEN3_8B = (
    ("q", 4096, 4096),
    ("k", 1024, 4096),
    ("v", 1024, 4096),
    ("o", 4096, 4096),
    ("gate", 12288, 4096),
    ("up", 12288, 4096),
    ("down", 4096, 12288),
)
QWEN3_8B_LAYERS = 36

# Which projections read the same layer input (they share one activation
# quantization): attention input -> q, k, v; attention output -> o;
# MLP input -> gate, up; MLP hidden -> down.
INPUT_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))

N_OUTLIERS = 8
OUTLIER_GAIN = 20.0


def _f32_to_bf16_bits_trunc(x: np.ndarray) -> np.ndarray:
    # Keep the upper half of each binary32 word: a bf16 value drawn from (close
    # to) the f32 distribution.  Only used to make synthetic inputs.
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def x_bf16(seed: int, M: int, K: int, heavy_tail: bool = False) -> np.ndarray:
    """Activations [M, K] as bf16 bits: N(0, 1), with 8 outlier channels
    (fixed per seed) multiplied by 20.  heavy_tail additionally scales the
    outlier channels per token by |t_3| (Student-t, 3 degrees of freedom)."""
    g = rng(seed)
    x = g.standard_normal((M, K), dtype=np.float32)
    if K:
        ch = g.choice(K, min(N_OUTLIERS, K), replace=False)
        gain = np.float32(OUTLIER_GAIN)
        if heavy_tail:
            t = np.abs(g.standard_t(3, size=(M, 1))).astype(np.float32)
            x[:, ch] *= gain * (1.0 + t)
        else:
            x[:, ch] *= gain
    return _f32_to_bf16_bits_trunc(x)


def w_int8(seed: int, N: int, K: int) -> np.ndarray:
    """int8 weights [N, K], uniform integers in [-127, 127]."""
    return rng(seed).integers(-127, 128, size=(N, K), dtype=np.int8)


def scale_bf16(seed: int, shape, lo: float = 1e-3, hi: float = 5e-3) -> np.ndarray:
    """bf16 scales (bits), uniform in [lo, hi)."""
    return _f32_to_bf16_bits_trunc(rng(seed).uniform(lo, hi, size=shape).astype(np.float32))


def w_e4m3(seed: int, N: int, K: int) -> np.ndarray:
    """E4M3 weight codes [N, K]: random sign, magnitude code uniform over the
    127 finite magnitudes 0x00..0x7E (zero, subnormals, normals up to 448)."""
    g = rng(seed)
    mag = g.integers(0, 0x7F, size=(N, K), dtype=np.uint8)
    sgn = (g.integers(0, 2, size=(N, K), dtype=np.uint8) << np.uint8(7)).astype(np.uint8)
    return (mag | sgn).astype(np.uint8)


# --------------------------------------------------------------------------
# Device-side generation for the large benchmark footprints (torch RNG,
# seeded per tensor).  Same distributions as above, different random streams.
# --------------------------------------------------------------------------

def torch_w_int8(torch, gen, N, K, device):
    return torch.randint(-127, 128, (N, K), dtype=torch.int8, device=device, generator=gen)


def torch_w_e4m3(torch, gen, N, K, device):
    mag = torch.randint(0, 0x7F, (N, K), dtype=torch.uint8, device=device, generator=gen)
    sgn = torch.randint(0, 2, (N, K), dtype=torch.uint8, device=device, generator=gen) << 7
    return mag | sgn


def torch_scale_bf16(torch, gen, shape, device, lo=1e-3, hi=5e-3):
    u = torch.rand(shape, dtype=torch.float32, device=device, generator=gen) * (hi - lo) + lo
    return (u.view(torch.int32) >> 16).to(torch.int16)


def torch_x_bf16(torch, gen, M, K, device):
    x = torch.randn((M, K), dtype=torch.float32, device=device, generator=gen)
    ch = torch.randperm(K, device=device, generator=gen)[:N_OUTLIERS]
    x[:, ch] *= OUTLIER_GAIN
    return (x.view(torch.int32) >> 16).to(torch.int16)
