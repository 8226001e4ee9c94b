"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- hand-worked fixtures (tests/golden), closed forms, exact rational
arithmetic, brute force over the code tables, invariants, and library
cross-checks (torch's bf16 / float8_e4m3fn conversions) used only as
independent references.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hex_arr(rows, dtype):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=dtype)


# --------------------------------------------------------------------------
# Independent exact helpers (Fraction based)
# --------------------------------------------------------------------------

def f32_round(r: Fraction) -> Fraction:
    """Nearest binary32 value of an exact rational, ties to even (no overflow)."""
    if r == 0:
        return Fraction(0)
    sgn = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    return sgn * round(a / ulp) * ulp          # round() on Fraction is half-to-even


def bf16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits << 16], np.uint32).view(np.float32)[0]))


def e4m3_table():
    """(code, exact value) for every finite E4M3 code, from the format's
    definition, written independently of the oracle's decoder."""
    out = []
    for sign in (0, 1):
        for E in range(16):
            for m in range(8):
                if E == 15 and m == 7:
                    continue
                v = Fraction(m, 2 ** 9) if E == 0 else Fraction(8 + m) * Fraction(2) ** (E - 10)
                out.append(((sign << 7) | (E << 3) | m, -v if sign else v))
    return out


E4M3_TABLE = e4m3_table()


def e4m3_nearest_bruteforce(v: Fraction, negative: bool = None) -> int:
    """Nearest finite code by scanning every code; ties -> even code; sign kept
    (pass negative=True for a negative zero, which a Fraction cannot carry)."""
    neg = (v < 0) if negative is None else negative
    best = None
    for code, val in E4M3_TABLE:
        if (code >> 7) != (1 if neg else 0):
            continue
        d = abs(val - v)
        if best is None or d < best[0] or (d == best[0] and (code & 1) == 0):
            best = (d, code)
    return best[1]


# --------------------------------------------------------------------------
# bf16
# --------------------------------------------------------------------------

def test_bf16_widen_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_bits_to_f32(bits)
    assert np.array_equal(f.view(np.uint32) >> 16, bits.astype(np.uint32))
    assert np.array_equal(f.view(np.uint32) & 0xFFFF, np.zeros_like(bits, dtype=np.uint32))


def test_bf16_round_hand_values():
    # nearest bf16 with ties to even significand
    cases = {
        1.0: 0x3F80, -1.0: 0xBF80, 64.5: 0x4281, -4032.25: 0xC57C,
        1.0 + 2 ** -8: 0x3F80,              # exact tie -> even (1.0)
        1.0 + 3 * 2 ** -8: 0x3F82,          # exact tie -> even (1 + 2^-6)
        1.0 + 2 ** -8 + 2 ** -30: 0x3F81,   # just above the tie
        0.0: 0x0000, 2.0 ** 128 * 0.999999: 0x7F80,
    }
    for v, b in cases.items():
        assert int(O.round_to_bf16_bits(np.array([v]))[0]) == b, v


def test_bf16_round_vs_torch_f32():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(7)
    u = g.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # add every exact tie pattern (low 16 bits = 0x8000) for a spread of values
    ties = (g.integers(0, 2 ** 16, size=1 << 16, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties.astype(np.uint32)])
    f = u.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.38e38)]
    ours = O.round_to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# --------------------------------------------------------------------------
# E4M3 codec
# --------------------------------------------------------------------------

def test_e4m3_decode_hand_values():
    d = O.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3A, 0x7E, 0x80, 0xB8, 0xFE], np.uint8))
    exp = [0.0, 2 ** -9, 7 * 2 ** -9, 2 ** -6, 1.0, 1.25, 448.0, -0.0, -1.0, -448.0]
    assert np.array_equal(d, np.array(exp))
    assert np.signbit(d[7])
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_decode_matches_table_and_torch():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    for code, val in E4M3_TABLE:
        assert Fraction(float(ours[code])) == val
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(ours), ~fin)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c, _ in E4M3_TABLE], np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_e4m3_encode_bruteforce():
    g = np.random.default_rng(3)
    vals = []
    # every midpoint between neighbouring finite values (exact ties) and a hair either side
    pos = sorted(v for c, v in E4M3_TABLE if c < 0x80)
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        for v in (mid, lo, hi):
            vals.append(float(v))
        vals.append(float(np.nextafter(np.float32(mid), np.float32(0))))
        vals.append(float(np.nextafter(np.float32(mid), np.float32(1e9))))
    vals += list(g.uniform(-448, 448, 2000)) + list(g.uniform(-0.05, 0.05, 2000))
    vals += list(np.exp(g.uniform(-25, 6, 2000)) * g.choice([-1, 1], 2000))
    v32 = np.clip(np.array(vals, np.float32), -448, 448)
    v32 = np.concatenate([v32, -v32])
    ours = O.e4m3_encode(v32)
    for x, c in zip(v32, ours):
        assert int(c) == e4m3_nearest_bruteforce(Fraction(float(x)), bool(np.signbit(x))), float(x)


def test_e4m3_encode_vs_torch_all_bf16():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_bits_to_f32(bits)
    f = f[np.isfinite(f)]
    f = np.clip(f, -448, 448).astype(np.float32)
    ours = O.e4m3_encode(f)
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    same = (ours == ref) | (((ours & 0x7F) == 0) & ((ref & 0x7F) == 0))   # modulo +-0
    assert same.all()


# --------------------------------------------------------------------------
# Quantizers
# --------------------------------------------------------------------------

def test_int8_golden_rows():
    with open(os.path.join(GOLD, "int8_token_rows.json")) as fh:
        gd = json.load(fh)
    x = _hex_arr(gd["x_bf16"], np.uint16)
    q, s = O.quant_act_int8(x)
    assert np.array_equal(q, np.array(gd["q"], np.int8))
    for i, sv in enumerate(gd["s"]):
        if sv is not None:
            assert float(s[i]) == sv


def test_e4m3_golden_rows():
    with open(os.path.join(GOLD, "e4m3_token_rows.json")) as fh:
        gd = json.load(fh)
    x = _hex_arr(gd["x_bf16"], np.uint16)
    q, s = O.quant_act_fp8(x, 0)
    assert np.array_equal(q, _hex_arr(gd["q"], np.uint8))
    assert list(map(float, s)) == gd["s"]


def _bruteforce_int8_row(xbits):
    xs = [bf16_value(int(b)) for b in xbits]
    a = max(abs(v) for v in xs)
    if a == 0:
        return [0] * len(xs), Fraction(0)
    s = f32_round(a / 127)
    inv = f32_round(Fraction(127) / a)
    out = []
    for v in xs:
        t = f32_round(v * inv)
        out.append(max(-127, min(127, round(t))))
    return out, s


def _bruteforce_e4m3_row(xbits):
    xs = [bf16_value(int(b)) for b in xbits]
    a = max(abs(v) for v in xs)
    if a == 0:
        return [0x80 if np.signbit(float(v)) else 0 for v in xs], Fraction(0)
    s = f32_round(a / 448)
    inv = f32_round(Fraction(448) / a)
    out = []
    for v, b in zip(xs, xbits):
        t = f32_round(v * inv)
        t = max(Fraction(-448), min(Fraction(448), t))
        c = e4m3_nearest_bruteforce(t, bool(int(b) & 0x8000))
        out.append(c)
    return out, s


@pytest.mark.parametrize("seed", range(6))
def test_int8_quant_bruteforce(seed):
    x = W.x_bf16(seed, 3, 48)
    if seed == 5:
        x[1] = 0                      # an all-zero token
    q, s = O.quant_act_int8(x)
    for m in range(x.shape[0]):
        qb, sb = _bruteforce_int8_row(x[m])
        assert list(map(int, q[m])) == qb
        assert Fraction(float(s[m])) == sb


@pytest.mark.parametrize("seed", range(4))
def test_e4m3_quant_bruteforce(seed):
    x = W.x_bf16(50 + seed, 2, 32)
    q, s = O.quant_act_fp8(x, 0)
    for m in range(x.shape[0]):
        qb, sb = _bruteforce_e4m3_row(x[m])
        got = [int(c) for c in q[m]]
        assert [c & 0x7F for c in got] == [c & 0x7F for c in qb]
        assert all((g == b) or (g & 0x7F) == 0 for g, b in zip(got, qb))
        assert Fraction(float(s[m])) == sb


def test_int8_special_cases():
    # x = +-absmax -> +-127; a single non-zero element; a zero row
    x = np.zeros((3, 16), np.uint16)
    x[0, 3] = 0x4120          # 10.0
    x[0, 7] = 0xC120          # -10.0
    x[1, 5] = 0xBC00          # -0.0078125
    q, s = O.quant_act_int8(x)
    assert q[0, 3] == 127 and q[0, 7] == -127
    assert q[1, 5] == -127 and np.count_nonzero(q[1]) == 1
    assert s[2] == 0 and not q[2].any()


def test_power_of_two_equivariance():
    x = W.x_bf16(11, 4, 64)
    f = O.bf16_bits_to_f32(x)
    for j in (-3, 1, 5):
        xs = O.round_to_bf16_bits(f.astype(np.float64) * 2.0 ** j)     # exact: a power-of-two scaling
        q0, s0 = O.quant_act_int8(x)
        q1, s1 = O.quant_act_int8(xs)
        assert np.array_equal(q0, q1) and np.array_equal(s1, (s0 * np.float32(2.0 ** j)).astype(np.float32))
        e0, t0 = O.quant_act_fp8(x, 0)
        e1, t1 = O.quant_act_fp8(xs, 0)
        assert np.array_equal(e0, e1) and np.array_equal(t1, (t0 * np.float32(2.0 ** j)).astype(np.float32))


def test_tiny_tokens_codes_scale_free():
    """The codes depend on x only through x / a, so a token scaled by a power of
    two keeps its codes: tokens and 128-groups with absmax from 2^-133 (the
    smallest bf16 subnormal) to 2^-60, where Q/a can overflow f32, must give the
    codes of the same values moved to absmax ~1 (a dropped 2^64 pre-scaling
    gives +-Q for every nonzero element there)."""
    base = W.x_bf16(12, 6, 256)
    f = O.bf16_bits_to_f64(base)
    for e in (-60, -64, -90, -110, -118, -122, -126, -127):
        xs = O.round_to_bf16_bits(f * 2.0 ** e)
        xb = O.round_to_bf16_bits(O.bf16_bits_to_f64(xs) * 2.0 ** -e)   # exact back-scaling
        assert np.array_equal(O.bf16_bits_to_f64(xb) * 2.0 ** e, O.bf16_bits_to_f64(xs))
        assert np.array_equal(O.quant_act_int8(xs)[0], O.quant_act_int8(xb)[0]), e
        assert np.array_equal(O.quant_act_fp8(xs, 0)[0], O.quant_act_fp8(xb, 0)[0]), e
        assert np.array_equal(O.quant_act_fp8(xs, 128)[0], O.quant_act_fp8(xb, 128)[0]), e
    # a token whose only nonzero values are the smallest bf16 subnormals (a = 2^-133)
    x = np.zeros((1, 32), np.uint16)
    x[0, 3], x[0, 7] = 0x0001, 0x8001
    q, s = O.quant_act_int8(x)
    assert q[0, 3] == 127 and q[0, 7] == -127 and np.count_nonzero(q) == 2
    assert s[0] == np.float32(2.0 ** -133 / 127)
    e, _ = O.quant_act_fp8(x, 0)
    assert O.e4m3_decode(e)[0, 3] == 448 and O.e4m3_decode(e)[0, 7] == -448 and np.count_nonzero(O.e4m3_decode(e)) == 2


def test_int8_roundtrip_bound():
    x = W.x_bf16(12, 64, 4096)
    q, s = O.quant_act_int8(x)
    xf = O.bf16_bits_to_f64(x)
    err = np.abs(xf - s.astype(np.float64)[:, None] * q)
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 * (1 + 2 ** -10))


def _e4m3_ulp(v):
    v = np.abs(v)
    _, E = np.frexp(np.where(v > 0, v, 1.0))
    e = np.maximum(E - 1, -6)
    return np.ldexp(1.0, (e - 3).astype(np.int32))


@pytest.mark.parametrize("group", [0, 128])
def test_e4m3_roundtrip_bound(group):
    x = W.x_bf16(13, 32, 1024)
    q, s = O.quant_act_fp8(x, group)
    xf = O.bf16_bits_to_f64(x)
    sf = s.astype(np.float64)
    sf = sf[:, :, None].repeat(128, 2).reshape(32, 1024) if group else sf[:, None]
    safe = np.where(sf > 0, sf, 1.0)
    err = np.abs(xf - sf * O.e4m3_decode(q))
    assert np.all(err <= sf * _e4m3_ulp(xf / safe) / 2 * (1 + 2 ** -10))


def test_group_quant_is_per_token_quant_of_each_slice():
    x = W.x_bf16(14, 5, 512)
    qg, sg = O.quant_act_fp8(x, 128)
    qt, st = O.quant_act_fp8(x.reshape(20, 128), 0)
    assert np.array_equal(qg, qt.reshape(5, 512))
    assert np.array_equal(sg, st.reshape(5, 4))
    q1, s1 = O.quant_act_fp8(x[:, :128], 128)
    q0, s0 = O.quant_act_fp8(x[:, :128], 0)
    assert np.array_equal(q1, q0) and np.array_equal(s1[:, 0], s0)


# --------------------------------------------------------------------------
# Contractions and rescale
# --------------------------------------------------------------------------

def test_contract_int8_bruteforce_and_invariants():
    g = np.random.default_rng(5)
    qx = g.integers(-127, 128, (3, 40), dtype=np.int8)
    qw = g.integers(-128, 128, (5, 40), dtype=np.int8)     # a weight of -128 is accepted
    acc = O.contract_int8(qx, qw)
    brute = [[sum(int(a) * int(b) for a, b in zip(qx[m], qw[n])) for n in range(5)] for m in range(3)]
    assert acc.tolist() == brute
    p = g.permutation(40)
    assert np.array_equal(O.contract_int8(qx[:, p], qw[:, p]), acc)
    # the largest accumulator of the projection shapes fits int32
    K = 14336
    big = O.contract_int8(np.full((1, K), -127, np.int8), np.full((1, K), -128, np.int8))
    assert int(big[0, 0]) == 127 * 128 * K < 2 ** 31


def test_contract_int8_negation():
    g = np.random.default_rng(6)
    qx = g.integers(-127, 128, (4, 64), dtype=np.int8)
    qw = g.integers(-127, 128, (6, 64), dtype=np.int8)
    assert np.array_equal(O.contract_int8(qx, -qw), -O.contract_int8(qx, qw))


def test_contract_e4m3_exact_fraction():
    g = np.random.default_rng(8)
    qx = W.w_e4m3(21, 3, 32)
    qw = W.w_e4m3(22, 4, 32)
    acc = O.contract_e4m3(qx, qw)
    val = {c: v for c, v in E4M3_TABLE}
    for m in range(3):
        for n in range(4):
            ex = sum(val[int(a)] * val[int(b)] for a, b in zip(qx[m], qw[n]))
            assert Fraction(float(acc[m, n])) == ex
    P = O.contract_e4m3_blocks(W.w_e4m3(23, 2, 256), W.w_e4m3(24, 3, 256))
    full = O.contract_e4m3(W.w_e4m3(23, 2, 256), W.w_e4m3(24, 3, 256))
    assert np.array_equal(P.sum(0), full)
    del g


def test_golden_projection_small():
    with open(os.path.join(GOLD, "projection_small.json")) as fh:
        gd = json.load(fh)
    r = gd["rowwise_int8"]
    acc = O.contract_int8(np.array(r["q_x"], np.int8), np.array(r["q_w"], np.int8))
    assert acc.tolist() == r["acc"]
    sw = np.array([int(v, 16) for v in r["s_w_bf16"]], np.uint16)
    y = O.rescale_rowwise(acc, np.array(r["s_x"], np.float32), sw)
    assert y.tolist() == r["y_exact"]
    assert O.round_to_bf16_bits(y).tolist() == [[int(v, 16) for v in row] for row in r["y_bf16"]]
    b = gd["block_fp8"]
    M, N, K = b["M"], b["N"], b["K"]
    qx = np.empty((M, K), np.uint8)
    for i, c in enumerate(b["q_x_fill_per_block"]):
        qx[:, i * 128:(i + 1) * 128] = int(c, 16)
    qw = np.full((N, K), int(b["q_w_fill"], 16), np.uint8)
    P = O.contract_e4m3_blocks(qx, qw)
    assert [float(P[kb, 0, 0]) for kb in range(2)] == b["P"]
    swb = np.array([[int(v, 16) for v in row] for row in b["s_w_bf16"]], np.uint16)
    yb = O.round_to_bf16_bits(O.rescale_block(P, np.array(b["s_x"], np.float32), swb))
    assert (yb == int(b["y_bf16_all"], 16)).all()


def test_dequantize_then_multiply_equivalence():
    x = W.x_bf16(31, 8, 512)
    qw = W.w_int8(32, 64, 512)
    sw = W.scale_bf16(33, 64)
    _, y, qx, sx, acc = O.linear_w8a8(x, qw, sw)
    deq = (sx.astype(np.float64)[:, None] * qx) @ (O.bf16_bits_to_f64(sw)[:, None] * qw).T
    assert np.allclose(deq, y, rtol=1e-12, atol=0)
    # FP8 rowwise: the same identity with decoded E4M3 values
    qw8 = W.w_e4m3(34, 64, 512)
    _, y8, qx8, sx8 = O.linear_fp8_rowwise(x, qw8, sw)
    deq8 = (sx8.astype(np.float64)[:, None] * O.e4m3_decode(qx8)) @ (O.bf16_bits_to_f64(sw)[:, None] * O.e4m3_decode(qw8)).T
    assert np.allclose(deq8, y8, rtol=1e-12, atol=1e-300)


def test_block_reduces_to_rowwise():
    g = np.random.default_rng(40)
    M, N, K = 6, 256, 512
    qx = W.w_e4m3(41, M, K)
    qw = W.w_e4m3(42, N, K)
    sx_row = g.uniform(0.01, 1, M).astype(np.float32)
    sw_blk = W.scale_bf16(43, (N // 128,))
    P = O.contract_e4m3_blocks(qx, qw)
    yb = O.rescale_block(P, np.repeat(sx_row[:, None], K // 128, 1), np.repeat(sw_blk[:, None], K // 128, 1))
    yr = O.rescale_rowwise(O.contract_e4m3(qx, qw), sx_row, np.repeat(sw_blk, 128))
    assert np.allclose(yb, yr, rtol=1e-12, atol=1e-300)
    # a single K block: block form equals rowwise form (up to fp64 product order)
    P1 = O.contract_e4m3_blocks(qx[:, :128], qw[:, :128])
    yb1 = O.rescale_block(P1, sx_row[:, None], sw_blk[:, None])
    yr1 = O.rescale_rowwise(O.contract_e4m3(qx[:, :128], qw[:, :128]), sx_row, np.repeat(sw_blk, 128))
    assert np.allclose(yb1, yr1, rtol=5e-16, atol=0)


def test_block_scale_indexing_planted():
    # a block scale that is wrong for exactly one (row block, k block) must move
    # exactly the outputs of that row block
    M, N, K = 2, 256, 384
    qx = W.w_e4m3(51, M, K)
    qw = W.w_e4m3(52, N, K)
    sx = np.random.default_rng(53).uniform(0.5, 1, (M, 3)).astype(np.float32)
    sw = W.scale_bf16(54, (2, 3))
    P = O.contract_e4m3_blocks(qx, qw)
    y0 = O.rescale_block(P, sx, sw)
    sw2 = sw.copy()
    sw2[1, 2] = 0x4000                                       # 2.0 for row block 1, k block 2
    y1 = O.rescale_block(P, sx, sw2)
    assert np.array_equal(y0[:, :128], y1[:, :128])
    assert not np.array_equal(y0[:, 128:], y1[:, 128:])


def test_epilogue_order_within_tolerance():
    x = W.x_bf16(61, 16, 4096)
    qw = W.w_int8(62, 256, 4096)
    sw = W.scale_bf16(63, 256)
    yb, y, qx, sx, acc = O.linear_w8a8(x, qw, sw)
    ye = O.epilogue_f32_order(acc, sx, sw)
    yb_f = O.bf16_bits_to_f64(yb)
    ye_f = O.bf16_bits_to_f64(ye)
    assert np.max(np.abs(ye_f - y)) <= 4e-3 * np.max(np.abs(y))
    assert np.max(np.abs(yb_f - y)) <= 4e-3 * np.max(np.abs(y))
    # both are within one bf16 ulp of each other
    assert np.all(np.abs(ye_f - yb_f) <= np.abs(y) * 2 ** -7 + 1e-30)


def bf16_round(r: Fraction) -> Fraction:
    """Nearest bf16 value of an exact rational, ties to even (8 significant bits,
    binary32's exponent range; no overflow)."""
    if r == 0:
        return Fraction(0)
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 7)
    return (-1 if r < 0 else 1) * round(a / ulp) * ulp


def _epilogue_fraction(acc: int, sx: float, sw_bits: int) -> Fraction:
    """bf16_RNE(fl32(fl32(acc) * fl32(s_x * s_w))), every step an exact rational
    rounded once."""
    f = f32_round(Fraction(float(sx)) * bf16_value(sw_bits))
    return bf16_round(f32_round(f32_round(Fraction(int(acc))) * f))


def test_epilogue_f32_order_fraction_bruteforce():
    # random accumulators over the whole int32 range the products reach, with
    # rounding ties planted at each of the three rounding steps
    rng = np.random.default_rng(464)
    acc = rng.integers(-231225344, 231225345, 160, dtype=np.int64)
    acc[:8] = [257, -259, 16777217, -16777219, 2 ** 24 + 3, 33554435, 0, -1]    # bf16 ties; f32 ties of acc
    sx = rng.uniform(1e-3, 0.5, 160).astype(np.float32)
    sx[:8] = 1.0
    sx[8:16] = np.float32(1.0 + 2.0 ** -23)                                    # s_x * s_w needs rounding
    swb = W.scale_bf16(465, 160)
    swb[:8] = 0x3F80                                                           # s_w = 1
    swb[8:16] = 0x3F81                                                         # 1 + 2^-7
    got = O.epilogue_f32_order(acc[:, None], sx, swb)                          # [160, 160]
    for m in range(0, 160, 7):
        for n in list(range(16)) + list(range(16, 160, 11)):
            want = _epilogue_fraction(acc[m], sx[m], int(swb[n]))
            assert bf16_value(int(got[m, n])) == want, (m, n, acc[m], sx[m], hex(swb[n]))
    # the ties resolve to even significands
    assert bf16_value(int(got[0, 0])) == 256 and bf16_value(int(got[1, 0])) == -260
    assert bf16_value(int(got[2, 0])) == 2 ** 24 and bf16_value(int(got[3, 0])) == -(2 ** 24)


def test_epilogue_f32_order_is_not_another_order():
    # The pin has power: products placed within an f32 ulp of a bf16 rounding
    # tie, where the order of the roundings decides the bf16 result.  The
    # oracle must match the Fraction chain on every case and differ from two
    # plausible other orders on some: fl32(fl32(acc * s_x) * s_w), and one
    # rounding of the exact product.
    rng = np.random.default_rng(466)
    accs, sxs, sws = [], [], []
    for _ in range(300):
        acc = int(rng.integers(2 ** 20, 2 ** 27)) * (1 if rng.random() < 0.5 else -1)
        swb = int(rng.integers(0x3A00, 0x3C00))                       # bf16 scales 4.9e-4 .. 7.8e-3
        tie = Fraction(2 * int(rng.integers(128, 256)) + 1, 2 ** 9) * Fraction(2) ** int(rng.integers(-4, 6))
        accs.append(acc)
        sxs.append(np.float32(float(tie / (abs(acc) * bf16_value(swb)))))
        sws.append(swb)
    acc = np.array(accs, np.int64)
    sx = np.array(sxs, np.float32)
    sw = np.array(sws, np.uint16)
    got = np.diag(O.epilogue_f32_order(acc[:, None], sx, sw))
    differs_b = differs_c = 0
    for i in range(len(acc)):
        a, x, w = Fraction(int(acc[i])), Fraction(float(sx[i])), bf16_value(int(sw[i]))
        chain = _epilogue_fraction(acc[i], sx[i], int(sw[i]))
        assert bf16_value(int(got[i])) == chain, i
        differs_b += bf16_round(f32_round(f32_round(a * x) * w)) != chain
        differs_c += bf16_round(a * x * w) != chain
    assert differs_b > 0 and differs_c > 0, (differs_b, differs_c)


def test_math_constants():
    assert O.Q_E4M3 == float(O.e4m3_decode(np.array([0x7E], np.uint8))[0])
    assert math.isclose(O.Q_INT8, 127.0)


# ---------------------------------------------------------------------------
# Weight-only ("equivalent") numerics
# ---------------------------------------------------------------------------

def _weight_only_fraction(xbits, q_w, sw_bits, scheme):
    """Exact rational evaluation of sum_k x[m,k] * s_w * value(q_w[n,k])."""
    M, K = xbits.shape
    N = q_w.shape[0]
    tab = dict(e4m3_table())                 # code -> exact value
    out = np.zeros((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                if scheme == "int8":
                    v = Fraction(int(np.int8(q_w[n, k])))
                else:
                    v = tab[int(q_w[n, k])]
                sc = bf16_value(int(sw_bits[n // 128, k // 128])) if scheme == "fp8_block" else bf16_value(int(sw_bits[n]))
                tot += bf16_value(int(xbits[m, k])) * sc * v
            out[m, n] = tot
    return out


@pytest.mark.parametrize("scheme", ["int8", "fp8_rowwise", "fp8_block"])
def test_weight_only_fraction_bruteforce(scheme):
    M, N, K = 2, 3 if scheme != "fp8_block" else 130, 256
    x = W.x_bf16(900, M, K)
    qw = W.w_int8(901, N, K) if scheme == "int8" else W.w_e4m3(901, N, K)
    sw = W.scale_bf16(902, ((N + 127) // 128, K // 128) if scheme == "fp8_block" else (N,))
    _, y = O.linear_weight_only(x, qw, sw, scheme)
    cols = [0, 1, 129] if scheme == "fp8_block" else list(range(N))   # rows from both 128-row blocks
    ref = _weight_only_fraction(x, qw[cols], sw, scheme) if scheme != "fp8_block" else None
    if scheme == "fp8_block":
        full = _weight_only_fraction(x, qw[: 130], sw, scheme)
        ref = full[:, cols]
    for m in range(M):
        for i, n in enumerate(cols):
            exact = float(ref[m, i])
            assert abs(y[m, n] - exact) <= 1e-13 * max(1.0, abs(exact)), (m, n, y[m, n], exact)


def test_weight_only_equals_w8a8_when_rounding_is_exact():
    # x = 2**-5 * q with max|q| = 127: the per-token int8 rounding reproduces q
    # and s exactly, so the two numerics define the same value
    rng = np.random.default_rng(903)
    M, N, K = 4, 96, 512
    q = rng.integers(-127, 128, (M, K), dtype=np.int64)
    q[:, 7] = 127
    xbits = O.round_to_bf16_bits(q.astype(np.float64) * 2.0 ** -5)
    qw = W.w_int8(904, N, K)
    sw = W.scale_bf16(905, N)
    _, y_w8a8, qx, sx, _ = O.linear_w8a8(xbits, qw, sw)
    assert np.array_equal(qx.astype(np.int64), q) and np.all(sx == np.float32(2.0 ** -5))
    _, y_wo = O.linear_weight_only(xbits, qw, sw, "int8")
    assert np.allclose(y_wo, y_w8a8, rtol=1e-14, atol=0)


def test_weight_only_equals_fp8_rowwise_when_rounding_is_exact():
    # x = 2**-3 * (E4M3 values) with max |value| = 448: per-token FP8 rounding is exact
    rng = np.random.default_rng(906)
    M, N, K = 3, 64, 384
    codes = (rng.integers(0, 0x7E, (M, K)) | (rng.integers(0, 2, (M, K)) << 7)).astype(np.uint8)
    codes[:, 3] = 0x7E
    xbits = O.round_to_bf16_bits(O.e4m3_decode(codes) * 2.0 ** -3)
    qw = W.w_e4m3(907, N, K)
    sw = W.scale_bf16(908, N)
    _, y_fp8, qx, sx = O.linear_fp8_rowwise(xbits, qw, sw)
    assert np.all(sx == np.float32(2.0 ** -3))
    _, y_wo = O.linear_weight_only(xbits, qw, sw, "fp8_rowwise")
    assert np.allclose(y_wo, y_fp8, rtol=1e-14, atol=0)


def test_weight_only_block_reduces_to_rowwise_and_scales_exactly():
    M, N, K = 2, 256, 384
    x = W.x_bf16(909, M, K)
    qw = W.w_e4m3(910, N, K)
    row = W.scale_bf16(911, N // 128)                    # one scale per 128-row band
    blk = np.repeat(row[:, None], K // 128, axis=1)      # equal along K
    _, yb = O.linear_weight_only(x, qw, blk, "fp8_block")
    _, yr = O.linear_weight_only(x, qw, np.repeat(row, 128), "fp8_rowwise")
    assert np.allclose(yb, yr, rtol=1e-14, atol=0)
    # power-of-two homogeneity in x is exact
    x2 = O.round_to_bf16_bits(O.bf16_bits_to_f64(x) * 4.0)
    _, y4 = O.linear_weight_only(x2, qw, blk, "fp8_block")
    assert np.array_equal(y4, yb * 4.0)


# --------------------------------------------------------------------------
# SwiGLU on a gate/up pair
# --------------------------------------------------------------------------

def test_silu_closed_forms_and_identities():
    ln3 = math.log(3.0)
    # sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(ln3) - 0.75 * ln3) <= 4e-16
    assert abs(O.silu(-ln3) + 0.25 * ln3) <= 4e-16
    # silu(t) - silu(-t) = t, and silu(t) = t * sigmoid(t) through scipy's logistic
    import scipy.special as sp
    t = np.random.default_rng(7).normal(0.0, 6.0, 4096)
    assert np.allclose(O.silu(t) - O.silu(-t), t, rtol=0, atol=1e-13 * np.abs(t).max())
    assert np.allclose(O.silu(t), t * sp.expit(t), rtol=1e-14, atol=1e-300)
    # limits: large t passes through, very negative t gives (negative) zero
    assert O.silu(60.0) == 60.0
    v = O.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0


def _bf16_rne_via_f64_bits(v):
    """bf16 rounding of fp64 values in one step, on the fp64 bit pattern:
    round-half-even of the significand at its 8th bit, then the exponent
    re-biased from 1023 to 127 (a different route from the oracle's; normal
    bf16 range and zero only)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    assert np.all((a == 0) | ((a >= 2.0 ** -126) & (a < 2.0 ** 127))), "outside the normal bf16 range"
    u = v.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45)      # sign | 11-bit exponent | 7-bit significand
    sign = (r >> np.uint64(18)) & np.uint64(1)
    exp = ((r >> np.uint64(7)) & np.uint64(0x7FF)).astype(np.int64)
    man = r & np.uint64(0x7F)
    bits = (sign << np.uint64(15)) | (np.where(a == 0, 0, exp - 1023 + 127).astype(np.uint64) << np.uint64(7)) | \
        np.where(a == 0, np.uint64(0), man)
    return bits.astype(np.uint16)


def test_bf16_single_rounding_helper():
    # ties and near-ties that a double rounding through f32 would get wrong
    one = 1.0
    cases = {one + 2.0 ** -8: 0x3F80,                          # tie -> even (1.0)
             one + 3 * 2.0 ** -8: 0x3F82,                      # tie -> even (1 + 2^-6)
             one + 2.0 ** -8 + 2.0 ** -40: 0x3F81,             # just above the tie: up (f32 would drop 2^-40)
             -(one + 2.0 ** -8 - 2.0 ** -40): 0xBF80,          # just below: down
             3.0: 0x4040, 0.0: 0x0000}
    for v, want in cases.items():
        assert int(_bf16_rne_via_f64_bits(np.array([v]))[0]) == want, v
    assert int(O.round_to_bf16_bits(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0]) == 0x3F81


@pytest.mark.parametrize("scheme", ["int8", "fp8_rowwise", "fp8_block"])
def test_swiglu_chain_independent(scheme):
    """h = bf16(bf16(silu(g)) * u) with g, u the gate and up projections,
    recomputed with silu in its tanh form, t (1 + tanh(t/2)) / 2."""
    M, K, I = 3, 256, 256
    x = W.x_bf16(900, M, K)
    if scheme == "int8":
        gate = (W.w_int8(901, I, K), W.scale_bf16(902, I, 1e-4, 5e-4))
        up = (W.w_int8(903, I, K), W.scale_bf16(904, I, 1e-4, 5e-4))
        lin = O.linear_w8a8
    else:
        shp = (I // 128, K // 128) if scheme == "fp8_block" else (I,)
        gate = (W.w_e4m3(901, I, K), W.scale_bf16(902, shp, 1e-4, 5e-4))
        up = (W.w_e4m3(903, I, K), W.scale_bf16(904, shp, 1e-4, 5e-4))
        lin = O.linear_fp8_rowwise if scheme == "fp8_rowwise" else O.linear_fp8_block
    h, g_bits, u_bits, g_exact, u_exact = O.swiglu_gate_up(x, gate, up, scheme)
    # the pair is (gate, up) in that order, each the pinned projection
    assert np.array_equal(g_bits, lin(x, *gate)[0]) and np.array_equal(u_bits, lin(x, *up)[0])
    g = O.bf16_bits_to_f64(g_bits)
    u = O.bf16_bits_to_f64(u_bits)
    assert (g < -2).any() and (np.abs(g) < 2).any() and (g > 2).any(), "inputs span the curved part of silu"
    s = O.bf16_bits_to_f64(_bf16_rne_via_f64_bits(g * (1.0 + np.tanh(g / 2.0)) / 2.0))
    want = _bf16_rne_via_f64_bits(s * u)
    assert np.array_equal(h, want)
    # the intermediate rounding matters: a single rounding of silu(g) * u differs somewhere
    assert not np.array_equal(h, _bf16_rne_via_f64_bits(g * (1.0 + np.tanh(g / 2.0)) / 2.0 * u))
    # gate and up do not commute
    h_swapped = O.swiglu_gate_up(x, up, gate, scheme)[0]
    assert not np.array_equal(h, h_swapped)
    assert np.allclose(g, g_exact, rtol=2.0 ** -8, atol=0) and np.allclose(u, u_exact, rtol=2.0 ** -8, atol=0)
