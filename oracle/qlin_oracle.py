"""CPU oracle for the quantized decoder projection.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The HIP library never calls it and
shares no code, tables or constants with it.

What is computed (the three schemes the pages describe):

* W8A8 int8 -- "Llama 3.1 8B Instruct W8A8" model card, intro and section
  "Loading": int8 weights with one bf16 scale per output row; inputs rounded to
  int8 one token (row) at a time; int8 x int8 products summed in int32.
* FP8 per-channel -- "Llama 3.1 8B Instruct FP8" benchmark page, intro, and the
  "Meta-Llama-3.1-8B-Instruct-FP8-dynamic" README, sections "Model
  Optimizations" and "Creation" (weights: 8-bit float, per channel, static,
  symmetric; inputs: 8-bit float, per token, dynamic, symmetric).
* FP8 block -- "Qwen3 8B FP8" model card, intro and section "Loading": one bf16
  scale per 128x128 weight block, used as a multiplier; inputs rounded to FP8
  128 inputs at a time; widths are multiples of 128.

Readings where the pages are silent (each is also listed in the design notes):

* the dynamic scale is absmax/Q with Q = 127 (int8) or Q = 448 (largest finite
  OCP E4M3 value); symmetric, no zero point;
* one correctly rounded f32 divide gives s = a/Q and one gives inv = Q/a; the
  element is then fl32(x * inv), rounded half to even and saturated to +-Q;
* for a < 2^-64 (where Q/a may exceed the f32 range) the reciprocal is taken
  with an unbounded exponent: x and a are first scaled by 2^64 (exactly), so
  the element is fl32(fl32(x * 2^64) * fl32(Q / (a * 2^64))); wherever Q/a is
  finite this equals fl32(x * inv) (power-of-two scaling commutes with f32
  rounding), so the scaling only defines the tokens that would overflow;
* an all-zero token (or group) gets s = 0 and codes 0;
* the E4M3 flavour is OCP E4M3 (bias 7, max 448, codes 0x7F/0xFF are NaN, no
  infinities), rounding to nearest with ties to the even code;
* x_bf16 widens exactly to f32; scales of activations are f32; weight scales
  are bf16; the output is bf16, rounded to nearest-even from the exact value.

Arithmetic conventions: float32 steps are done in numpy.float32 (IEEE-754,
round to nearest even, subnormals kept); the contraction is exact (integers or
exactly scaled integers); the rescale is fp64.  No blocking, fusion or
reordering beyond what the definition states.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "Q_INT8", "Q_E4M3",
    "bf16_bits_to_f32", "round_to_bf16_bits", "bf16_bits_to_f64",
    "e4m3_decode", "e4m3_encode",
    "quant_act_int8", "quant_act_fp8",
    "contract_int8", "contract_e4m3", "contract_e4m3_blocks",
    "rescale_rowwise", "rescale_block",
    "linear_w8a8", "linear_fp8_rowwise", "linear_fp8_block",
    "epilogue_f32_order",
    "dequantize_weights", "linear_weight_only",
    "silu", "swiglu_gate_up",
]

# Largest code magnitude of each target format.
Q_INT8 = 127.0      # symmetric int8: -128 is never produced
Q_E4M3 = 448.0      # largest finite OCP E4M3 value: (1 + 6/8) * 2**8


# --------------------------------------------------------------------------
# bf16 <-> float
# --------------------------------------------------------------------------

def bf16_bits_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32.

    bf16 is the upper half of an IEEE binary32 word, so the widening is a
    16-bit left shift of the pattern (inputs are bf16: "--bind T=bf16" in the
    "Command line" sections of the W8A8 and Qwen3 model cards)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def round_to_bf16_bits(v) -> np.ndarray:
    """Round real values (float64/float32 array) to the nearest bf16 value,
    ties to an even significand, and return the uint16 bit patterns.

    bf16: 1 sign bit, 8 exponent bits (same range as binary32), 7 stored
    significand bits.  Written from that definition: find the binade of |v|,
    scale so one bf16 ulp is 1, round half-even, scale back.  Values whose
    rounded magnitude reaches 2**128 become infinity.  NaN stays NaN."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    a = np.abs(v)
    sign = np.signbit(v)
    nan = np.isnan(v)
    # exponent of the binade: a = f * 2**E, f in [0.5, 1)  =>  e = E - 1
    with np.errstate(divide="ignore", invalid="ignore"):
        _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(E.astype(np.int64) - 1, -126)          # subnormal binade clamps at 2**-126
    ulp = np.ldexp(1.0, (e - 7).astype(np.int32))          # 7 stored significand bits
    r = np.rint(a / ulp) * ulp                             # exact scaling; rint is half-even
    r = np.where(a == 0, 0.0, r)
    inf = (r >= 2.0 ** 128) | np.isinf(a)
    r32 = np.where(inf, np.inf, r).astype(np.float32)      # r is exactly representable
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(sign, bits | np.uint16(0x8000), bits)
    out[...] = np.where(nan, np.uint16(0x7FC0), bits)
    return out


# --------------------------------------------------------------------------
# OCP E4M3 codec
# --------------------------------------------------------------------------

def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3 code (float64; NaN for 0x7F/0xFF).

    Layout: s eeee mmm, exponent bias 7.  Exponent field 0 encodes the
    subnormals m * 2**-9; otherwise (1 + m/8) * 2**(e - 7).  The all-ones
    exponent with mantissa 7 is NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nor = (1.0 + m / 8.0) * np.ldexp(1.0, (e - 7).astype(np.int32))
    val = s * np.where(e == 0, sub, nor)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_encode(v) -> np.ndarray:
    """Nearest finite OCP E4M3 code of each float32 value, ties to the even
    code, sign kept (a negative value that rounds to zero gives 0x80).

    Inputs must already be saturated to [-448, 448] (the quantizer clamps
    before encoding).  NaN maps to 0x7F.

    From the format: below the smallest normal 2**-6 the spacing is 2**-9 and
    the code is the count of steps; in the binade [2**e, 2**(e+1)) the spacing is
    2**(e-3) and the code is (e + 7) * 8 + (steps - 8).  Codes are monotone in
    the value, so rounding up across a binade boundary lands on the next
    binade's first code without a special case."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    a = np.abs(v)
    if np.any(a[~np.isnan(a)] > Q_E4M3):
        raise ValueError("e4m3_encode expects values saturated to +-448")
    with np.errstate(divide="ignore", invalid="ignore"):
        _, E = np.frexp(np.where(a > 0, a, 1.0))
    e = E.astype(np.int64) - 1
    sub = a < 2.0 ** -6
    steps_sub = np.rint(a * 2.0 ** 9)                                   # 0..8
    steps_nor = np.rint(np.ldexp(a, (3 - e).astype(np.int32)))          # 8..16
    code = np.where(sub, steps_sub, (e + 7) * 8 + (steps_nor - 8))
    code = np.where(np.isnan(a), 0x7F, code).astype(np.int64)
    code = np.where(np.signbit(v) & ~np.isnan(a), code | 0x80, code)
    return code.astype(np.uint8)


# --------------------------------------------------------------------------
# Dynamic activation quantizers
# --------------------------------------------------------------------------

TINY = np.float32(2.0 ** -64)      # absmax below this: operands pre-scaled by 2^64
PRE = np.float32(2.0 ** 64)


def _scales(a: np.ndarray, Q: float):
    """s = fl32(a / Q) and the element factors (pre, inv): pre = 2^64 and
    inv = fl32(Q / (a * 2^64)) when a < 2^-64, else pre = 1 and inv = fl32(Q / a)
    (correctly rounded f32 divides); a zero absmax gives s = inv = 0 (the
    token's codes are then 0).  An element is rounded from fl32(fl32(x * pre) * inv)."""
    a = a.astype(np.float32)
    q = np.float32(Q)
    tiny = a < TINY
    pre = np.where(tiny, PRE, np.float32(1)).astype(np.float32)
    ap = (a * pre).astype(np.float32)                      # exact: a power-of-two scaling
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        s = (a / q).astype(np.float32)
        inv = np.where(a > 0, q / ap, np.float32(0)).astype(np.float32)
    return s, pre, inv


def quant_act_int8(x_bits):
    """Per-token dynamic int8 quantization of bf16 activations [M, K].

    W8A8 model card, intro and section "Loading": inputs are rounded to int8
    one token (row) at a time.  For each row m:
        a = max_k |x[m, k]|,  s = fl32(a / 127),  inv = fl32(127 / a),
        q[m, k] = clamp(rint_half_even(fl32(x[m, k] * inv)), -127, 127)
    (for a < 2^-64, x and a scaled by 2^64 first: see _scales).
    Returns (q int8 [M, K], s float32 [M])."""
    x = bf16_bits_to_f32(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s, pre, inv = _scales(a, Q_INT8)
    xp = (x * pre[:, None]).astype(np.float32)             # exact (1 or 2^64)
    t = (xp * inv[:, None]).astype(np.float32)             # one rounding f32 multiply, RNE
    q = np.clip(np.rint(t), -Q_INT8, Q_INT8).astype(np.int8)
    return q, s


def quant_act_fp8(x_bits, group: int = 0):
    """Dynamic symmetric FP8 (OCP E4M3) quantization of bf16 activations.

    group == 0: one scale per token (FP8-dynamic README, "Model Optimizations"
    and the "Creation" recipe: strategy token, dynamic, symmetric).
    group == 128: one scale per 128 consecutive inputs of a token, groups
    aligned at k = 128 g (Qwen3 8B FP8 model card, "Loading": inputs rounded to
    FP8 128 inputs at a time).
    Per token or group: a = max |x|, s = fl32(a/448), inv = fl32(448/a),
    q = E4M3_rne(clamp(fl32(x * inv), -448, 448)) (for a < 2^-64, x and a
    scaled by 2^64 first: see _scales).
    Returns (q uint8 codes [M, K], s float32 [M] or [M, K/128])."""
    x = bf16_bits_to_f32(x_bits)
    if x.ndim != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    if group == 0:
        xs = x.reshape(M, 1, K)
    elif group == 128:
        if K % 128:
            raise ValueError("K must be a multiple of 128 for group scales")
        xs = x.reshape(M, K // 128, 128)
    else:
        raise ValueError("group must be 0 or 128")
    a = np.max(np.abs(xs), axis=2) if xs.shape[2] else np.zeros(xs.shape[:2], np.float32)
    s, pre, inv = _scales(a, Q_E4M3)
    xp = (xs * pre[:, :, None]).astype(np.float32)         # exact (1 or 2^64)
    t = (xp * inv[:, :, None]).astype(np.float32)
    t = np.clip(t, -Q_E4M3, Q_E4M3).astype(np.float32)
    q = e4m3_encode(t).reshape(M, K)
    return q, (s[:, 0] if group == 0 else s)


# --------------------------------------------------------------------------
# Exact contractions
# --------------------------------------------------------------------------

def contract_int8(q_x, q_w) -> np.ndarray:
    """acc[m, n] = sum_k q_x[m, k] * q_w[n, k], exactly (int64).

    W8A8 model card, "Loading": int8 products summed in int32.  The matmul runs
    in fp64 on integer values; every partial sum is an integer of magnitude
    below 128*128*K < 2**53 for K < 2**39, so the library matmul is exact in any
    order.  The result is checked to fit int32."""
    qx = np.asarray(q_x, dtype=np.int8)
    qw = np.asarray(q_w, dtype=np.int8)
    K = qx.shape[1]
    assert qw.shape[1] == K and 128 * 128 * max(K, 1) < 2 ** 53
    acc = qx.astype(np.float64) @ qw.astype(np.float64).T
    acc = acc.astype(np.int64)
    assert np.all(np.abs(acc) < 2 ** 31), "accumulator exceeds int32"
    return acc


def _e4m3_as_int(codes) -> np.ndarray:
    """E4M3 value * 2**9 as an exact integer-valued float64 (|.| <= 229376)."""
    v = e4m3_decode(codes)
    if np.any(np.isnan(v)):
        raise ValueError("NaN E4M3 code in a contraction operand")
    return v * 2.0 ** 9


def contract_e4m3(q_x, q_w) -> np.ndarray:
    """acc[m, n] = sum_k dec(q_x[m, k]) * dec(q_w[n, k]), exactly (float64).

    Every E4M3 value times 2**9 is an integer of magnitude <= 448 * 512, so the
    products are integers below 2**36 and a K-term sum stays below 2**53 for
    K < 2**17; the fp64 matmul of the scaled operands is therefore exact, and
    the final 2**-18 is an exact power-of-two scaling."""
    X = _e4m3_as_int(q_x)
    W = _e4m3_as_int(q_w)
    assert X.shape[1] < 2 ** 17
    return (X @ W.T) * 2.0 ** -18


def contract_e4m3_blocks(q_x, q_w, block: int = 128) -> np.ndarray:
    """Per-K-block exact partial sums P[kb, m, n] over k in [128 kb, 128 kb + 128)."""
    X = _e4m3_as_int(q_x)
    W = _e4m3_as_int(q_w)
    K = X.shape[1]
    assert K % block == 0
    nb = K // block
    P = np.empty((nb, X.shape[0], W.shape[0]), dtype=np.float64)
    for kb in range(nb):
        sl = slice(kb * block, (kb + 1) * block)
        P[kb] = (X[:, sl] @ W[:, sl].T) * 2.0 ** -18
    return P


# --------------------------------------------------------------------------
# Rescale
# --------------------------------------------------------------------------

def rescale_rowwise(acc, s_x, s_w_bits) -> np.ndarray:
    """y_exact[m, n] = acc[m, n] * s_x[m] * s_w[n] in fp64 (the projection's
    definition: product of token scale and row scale times the sum)."""
    sw = bf16_bits_to_f64(s_w_bits)
    sx = np.asarray(s_x, dtype=np.float32).astype(np.float64)
    return np.asarray(acc, dtype=np.float64) * sx[:, None] * sw[None, :]


def rescale_block(P, s_x, s_w_bits, block: int = 128) -> np.ndarray:
    """y_exact[m, n] = sum_kb s_x[m, kb] * s_w[n // 128, kb] * P[kb, m, n] (fp64).

    Qwen3 8B FP8 model card: one bf16 scale per 128x128 weight block, a
    multiplier (W ~ s_w * q_w); one activation scale per 128-input group."""
    nb, M, N = P.shape
    sx = np.asarray(s_x, dtype=np.float32).astype(np.float64)     # [M, nb]
    sw = bf16_bits_to_f64(s_w_bits)                                # [N/128, nb]
    assert sx.shape == (M, nb) and sw.shape == ((N + block - 1) // block, nb)
    swn = np.repeat(sw, block, axis=0)[:N]                         # [N, nb]
    y = np.zeros((M, N), dtype=np.float64)
    for kb in range(nb):
        y += sx[:, kb][:, None] * swn[:, kb][None, :] * P[kb]
    return y


def epilogue_f32_order(acc_i32, s_x, s_w_bits) -> np.ndarray:
    """One concrete f32 evaluation order of the rowwise rescale, for a stronger
    (bit-exact) report on int8 paths: bf16_rne(fl32(fl32(acc) * fl32(s_x * s_w))).
    The accepted result is the fp64 rescale under the tolerance; this order is a
    reading, not part of the definition."""
    accf = np.asarray(acc_i32, dtype=np.int64).astype(np.float32)
    sx = np.asarray(s_x, dtype=np.float32)
    sw = bf16_bits_to_f32(s_w_bits)
    f = (sx[:, None] * sw[None, :]).astype(np.float32)
    y32 = (accf * f).astype(np.float32)
    return round_to_bf16_bits(y32)


# --------------------------------------------------------------------------
# Whole projections (the definition end to end)
# --------------------------------------------------------------------------

def linear_w8a8(x_bits, q_w, s_w_bits):
    """y = bf16_rne(s_x[m] * s_w[n] * sum_k q_x[m, k] q_w[n, k]) with q_x, s_x from
    quant_act_int8.  Returns (y_bits [M, N], y_exact [M, N] fp64, q_x, s_x, acc)."""
    q_x, s_x = quant_act_int8(x_bits)
    acc = contract_int8(q_x, q_w)
    y = rescale_rowwise(acc, s_x, s_w_bits)
    return round_to_bf16_bits(y), y, q_x, s_x, acc


def linear_fp8_rowwise(x_bits, q_w, s_w_bits):
    """FP8 per-channel weights, per-token dynamic FP8 activations."""
    q_x, s_x = quant_act_fp8(x_bits, 0)
    acc = contract_e4m3(q_x, q_w)
    y = rescale_rowwise(acc, s_x, s_w_bits)
    return round_to_bf16_bits(y), y, q_x, s_x


def linear_fp8_block(x_bits, q_w, s_w_bits):
    """FP8 with 128x128 weight-block scales and 1x128 activation-group scales."""
    q_x, s_x = quant_act_fp8(x_bits, 128)
    P = contract_e4m3_blocks(q_x, q_w)
    y = rescale_block(P, s_x, s_w_bits)
    return round_to_bf16_bits(y), y, q_x, s_x


# --------------------------------------------------------------------------
# Weight-only ("equivalent") numerics
# --------------------------------------------------------------------------

def dequantize_weights(q_w, s_w_bits, scheme: str, block: int = 128) -> np.ndarray:
    """W[n, k] = s_w * value(q_w[n, k]) in fp64 (exact: a bf16 scale times an
    int8 or E4M3 value has at most 8 + 8 significant bits).  scheme: "int8",
    "fp8_rowwise" (s_w [N]) or "fp8_block" (s_w [N/128, K/128], a multiplier;
    Qwen3 8B FP8 card, intro)."""
    if scheme == "int8":
        v = np.asarray(q_w, dtype=np.int8).astype(np.float64)
    else:
        v = e4m3_decode(q_w)
    N, K = v.shape
    sw = bf16_bits_to_f64(s_w_bits)
    if scheme == "fp8_block":
        assert sw.shape == ((N + block - 1) // block, (K + block - 1) // block)
        full = np.repeat(np.repeat(sw, block, axis=0)[:N], block, axis=1)[:, :K]
        return v * full
    return v * sw[:, None]


def linear_weight_only(x_bits, q_w, s_w_bits, scheme: str):
    """Weight-only ("equivalent") numerics: the input is never rounded; the
    product uses the bf16 activations and the dequantized weights
    (W8A8 model card and Qwen3 8B FP8 card, "Against bf16": the "equivalent"
    mode keeps the input unrounded; "Loading": the numerics option).

        y_exact[m, n] = sum_k x[m, k] * W[n, k],   W = dequantize_weights(...)

    The products are exact in fp64 (8 + 16 significant bits); the fp64 sum is
    within K * 2**-53 of the exact sum, far below the bf16 output's resolution.
    Returns (y_bits [M, N] bf16_rne(y_exact), y_exact [M, N] fp64)."""
    x = bf16_bits_to_f64(x_bits)
    w = dequantize_weights(q_w, s_w_bits, scheme)
    y = x @ w.T
    return round_to_bf16_bits(y), y


# --------------------------------------------------------------------------
# SwiGLU on a gate/up pair (the step right after the projections)
# --------------------------------------------------------------------------
#
# The pages stop at the projections; what follows is the plain definition of
# the gated MLP that the Llama 3.1 and Qwen3 layers (the models of the pages'
# "Command line" sections) feed into the down projection:
#     h = silu(x W_gate^T) * (x W_up^T),   silu(t) = t * sigmoid(t) = t / (1 + e^-t).
# Reading: gate and up are computed as the quantized projections above (one
# shared rounding of x) and rounded to bf16 like any projection output; silu is
# applied to that bf16 value and rounded to bf16, and the product with the bf16
# up value is rounded to bf16 -- the order in which a bf16 model evaluates
# act(gate) * up.

_LINEAR = {"int8": linear_w8a8, "fp8_rowwise": linear_fp8_rowwise, "fp8_block": linear_fp8_block}


def silu(t) -> np.ndarray:
    """silu(t) = t / (1 + exp(-t)) in fp64.  For t below about -709, exp(-t)
    overflows to inf and the quotient is -0 (the true value is below 1e-305)."""
    t = np.asarray(t, dtype=np.float64)
    with np.errstate(over="ignore"):
        return t / (1.0 + np.exp(-t))


def swiglu_gate_up(x_bits, gate, up, scheme: str):
    """h[m, j] = bf16(bf16(silu(g[m, j])) * u[m, j]) with g, u the bf16 outputs
    of the gate and up projections of the same input x under `scheme` ("int8",
    "fp8_rowwise", "fp8_block"); gate and up are (q_w, s_w_bits) pairs of
    equal shape.

    Returns (h_bits, g_bits, u_bits, g_exact, u_exact): h as bf16 bits [M, I],
    the two projections' bf16 outputs, and their exact (fp64, unrounded)
    values."""
    lin = _LINEAR[scheme]
    g_bits, g_exact = lin(x_bits, *gate)[:2]
    u_bits, u_exact = lin(x_bits, *up)[:2]
    s_bits = round_to_bf16_bits(silu(bf16_bits_to_f64(g_bits)))
    h_bits = round_to_bf16_bits(bf16_bits_to_f64(s_bits) * bf16_bits_to_f64(u_bits))
    return h_bits, g_bits, u_bits, g_exact, u_exact
