"""Pins of the oracle's NVFP4 activation quantizer and of the W4A4 FFN.

The quantizer is checked against an exact-rational brute force written
independently of it (fractions.Fraction: the nearest E4M3 value to
amax / (6 g) by bisection over every finite E4M3 magnitude, then the nearest
E2M1 value to v / (s g) by distance over the eight E2M1 magnitudes of the OCP
MX table, ties to the even code) on dense grids of v and g: ties, their
binary32 neighbours, every E4M3 midpoint for the block scale, and sweeps of
12-bit mantissas across the binades of a block.  A variant that takes the
element quotient in binary32 (v times the rounded reciprocal of s g)
disagrees with it on that grid, so the grid separates the exact rule from
its binary32 approximations.  Also: a worked block that round-trips exactly,
saturation, zero and underflow.  The FFN's use of the two activation scales
is checked through exact power-of-two scaling (ReLU^2 is homogeneous of
degree two) and invariance under relabeling the experts."""
import bisect
from fractions import Fraction

import numpy as np
import pytest

from oracle import Weights, e4m3_decode, fused_moe, nvfp4_roundtrip, nvfp4_values, quantize_nvfp4

# OCP MX v1.0 E2M1: codes 0..7 are the magnitudes below, bit 3 the sign
E2M1_TABLE = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
              Fraction(6)]


def _e4m3_table():
    """Every finite E4M3 (FN) magnitude in code order 0x00 .. 0x7E, from the
    bit fields (exponent bias 7, 3 mantissa bits, e = 0 subnormal)."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return out


E4M3_TABLE = _e4m3_table()


def _nearest_even(table, x):
    """Index of the entry of the ascending Fraction table nearest to x >= 0
    (ties to the even index; beyond the last entry, the last)."""
    i = bisect.bisect_left(table, x)
    if i == 0:
        return 0
    if i == len(table):
        return len(table) - 1
    lo, hi = x - table[i - 1], table[i] - x
    if lo < hi:
        return i - 1
    if hi < lo:
        return i
    return i - 1 if (i - 1) % 2 == 0 else i


def _brute_force(v, g):
    """Codes and scales by the exact rule in rational arithmetic."""
    v = np.asarray(v, dtype=np.float64)
    gq = Fraction(float(np.float32(g)))
    blocks = v.reshape(-1, 16)
    codes = np.zeros(blocks.shape, np.uint8)
    scales = np.zeros(len(blocks), np.uint8)
    for b, blk in enumerate(blocks):
        fr = [Fraction(float(x)) for x in blk]
        amax = max(abs(x) for x in fr)
        sc = _nearest_even(E4M3_TABLE, amax / (6 * gq))
        scales[b] = sc
        unit = E4M3_TABLE[sc] * gq
        if unit == 0:
            continue
        for i, x in enumerate(fr):
            codes[b, i] = _nearest_even(E2M1_TABLE, abs(x) / unit) | (8 if x < 0 else 0)
    return codes.reshape(v.shape), scales.reshape(v.shape[:-1] + (v.shape[-1] // 16,))


def _fp32_quotient_rule(v, g):
    """The element magnitude codes with the quotient taken in binary32 as v
    times the rounded reciprocal of s g (scales from the exact rule): a
    plausible implementation that is not the exact rule."""
    _, scales = quantize_nvfp4(v, g)
    s = e4m3_decode(scales).astype(np.float32)
    u = (s * np.float32(g)).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(u > 0, (np.float32(1) / u).astype(np.float32), np.float32(0))
    q = (np.asarray(v, np.float32).reshape(r.shape + (16,)) * r[..., None]).astype(np.float32).astype(np.float64)
    out = np.array([_nearest_even(E2M1_TABLE, Fraction(float(min(abs(x), 6.0)))) for x in q.reshape(-1)])
    return out.reshape(np.shape(v)).astype(np.uint8)


# per-tensor scales: exact small-mantissa ones (ties representable in binary32) and full-mantissa ones
G_VALUES = [1.0, 0.75, 1.25 * 2.0 ** -8, float(np.float32(1 / 336)), float(np.float32(3.7e-3)), 250.0,
            float(np.float32(0.0123456789)), float(np.float32(7.77e2))]
MIDS = [Fraction(1, 4), Fraction(3, 4), Fraction(5, 4), Fraction(7, 4), Fraction(5, 2), Fraction(7, 2), Fraction(5)]


def _tie_grid(g, scale_codes):
    """Blocks with scale s = E4M3(code) pinned by a maximum of 6 s g: each
    E2M1 midpoint times s g rounded to binary32, with its binary32 neighbours
    two ulps either way, both signs."""
    rows = []
    for sc in scale_codes:
        unit = float(E4M3_TABLE[sc]) * float(np.float32(g))
        vals = []
        for m in MIDS:
            t = np.float32(float(m) * unit)
            up, down = [t], [t]
            for _ in range(2):
                up.append(np.nextafter(up[-1], np.float32(np.inf), dtype=np.float32))
                down.append(np.nextafter(down[-1], np.float32(0), dtype=np.float32))
            vals.extend(up + down[1:])
        vals = np.array(vals, np.float64)
        vals = np.concatenate([vals, -vals])
        # 15 values after the block maximum, which pins the scale
        for i in range(0, len(vals), 15):
            chunk = vals[i:i + 15]
            blk = np.zeros(16)
            blk[0] = float(np.float32(6.0 * unit))
            blk[1:1 + len(chunk)] = chunk
            rows.append(blk)
    return np.stack(rows)


def _scale_grid(g):
    """Blocks whose maximum sweeps every E4M3 midpoint times 6 g (rounded to
    binary32) and its binary32 neighbours, with one smaller value."""
    gf = float(np.float32(g))
    rows = []
    for i in range(len(E4M3_TABLE) - 1):
        mid = float((E4M3_TABLE[i] + E4M3_TABLE[i + 1]) / 2)
        t = np.float32(mid * 6.0 * gf)
        for a in (t, np.nextafter(t, np.float32(np.inf), dtype=np.float32), np.nextafter(t, np.float32(0), dtype=np.float32)):
            blk = np.zeros(16)
            blk[3] = -float(a)
            blk[7] = float(a) * 0.37
            rows.append(blk)
    blk = np.zeros(16)
    blk[0] = float(np.float32(1e4 * gf))                 # far above 448 * 6 g: saturated scale
    rows.append(blk)
    return np.stack(rows)


def _sweep_grid(g, scale_code, rng):
    """A 12-bit mantissa sweep over the binades [unit/8, 8 unit) of a block
    with scale E4M3(scale_code), random signs."""
    unit = float(E4M3_TABLE[scale_code]) * float(np.float32(g))
    e0 = int(np.floor(np.log2(unit))) - 3
    mant = 1.0 + np.arange(4096) / 4096.0
    vals = np.concatenate([np.ldexp(mant, e) for e in range(e0, e0 + 6)])
    vals = vals.astype(np.float32).astype(np.float64)
    vals *= np.where(rng.random(len(vals)) < 0.5, -1.0, 1.0)
    vals = vals[: len(vals) // 15 * 15].reshape(-1, 15)
    head = np.full((len(vals), 1), float(np.float32(6.0 * unit)))
    return np.concatenate([head, vals], axis=1)


@pytest.mark.parametrize("g", G_VALUES)
def test_quantizer_matches_exact_rule_on_ties_and_neighbours(g):
    v = np.concatenate([_tie_grid(g, [0x08, 0x1B, 0x30, 0x3F, 0x55, 0x7E, 0x03]), _scale_grid(g)])
    codes, scales = quantize_nvfp4(v, g)
    bc, bs = _brute_force(v, g)
    np.testing.assert_array_equal(scales, bs)
    # -0 and +0 encode differently but decode alike; compare magnitudes and nonzero signs
    np.testing.assert_array_equal(codes & 7, bc & 7)
    nz = (codes & 7) != 0
    np.testing.assert_array_equal(codes[nz], bc[nz])


@pytest.mark.parametrize("g,scale_code", [(1.0, 0x38), (float(np.float32(1 / 336)), 0x41),
                                          (float(np.float32(0.0123456789)), 0x2D), (250.0, 0x0A)])
def test_quantizer_matches_exact_rule_on_mantissa_sweeps(g, scale_code):
    v = _sweep_grid(g, scale_code, np.random.default_rng(scale_code))
    codes, scales = quantize_nvfp4(v, g)
    bc, bs = _brute_force(v, g)
    np.testing.assert_array_equal(scales, bs)
    np.testing.assert_array_equal(codes & 7, bc & 7)
    nz = (codes & 7) != 0
    np.testing.assert_array_equal(codes[nz], bc[nz])


def test_grid_separates_the_exact_rule_from_binary32_quotients():
    # with full-mantissa g the binary32 quotient v * RN(1 / (s g)) lands on the
    # wrong side of a midpoint for some of the neighbours of a tie
    differ = 0
    for g in G_VALUES[3:]:
        v = _tie_grid(g, [0x08, 0x1B, 0x30, 0x3F, 0x55, 0x7E, 0x03])
        codes, _ = quantize_nvfp4(v, g)
        approx = _fp32_quotient_rule(v, g)
        differ += int(np.sum((codes & 7) != approx))
    assert differ > 0


@pytest.mark.parametrize("seed,g", [(0, 1.0), (1, 0.01), (2, 3.7e-3), (3, 250.0)])
def test_quantizer_matches_exact_rule_on_random_rows(seed, g):
    rng = np.random.default_rng(seed)
    v = rng.normal(size=(6, 64)) * np.exp(rng.normal(size=(6, 1)) * 2)
    v[0, :16] = 0.0                                       # an all-zero block
    v[1, 16:32] *= 1e-9                                   # a block whose scale underflows
    codes, scales = quantize_nvfp4(v, g)
    bc, bs = _brute_force(v, g)
    np.testing.assert_array_equal(scales, bs)
    np.testing.assert_array_equal(codes & 7, bc & 7)
    nz = (codes & 7) != 0
    np.testing.assert_array_equal(codes[nz], bc[nz])


def test_ties_round_to_even_codes():
    # g = 1 and a block maximum of 6 make s = 1, so the quotients are the values themselves
    v = np.zeros(16)
    v[:11] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -5.0, 0.2501, 6.0]
    codes, scales = quantize_nvfp4(v[None, :], 1.0)
    assert e4m3_decode(scales)[0, 0] == 1.0
    vals = nvfp4_values(codes, scales)[0]
    np.testing.assert_array_equal(vals[:11], [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -1.0, -4.0, 0.5, 6.0])


def test_representable_block_round_trips_exactly():
    # s = 2 (exact in E4M3), g = 0.5: every value below is g * s * (an E2M1 value), and the
    # block maximum 6 * s * g makes the scale rule pick s again
    g, s = 0.5, 2.0
    v = g * s * np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6, 6], dtype=np.float64)
    np.testing.assert_array_equal(nvfp4_roundtrip(v[None, :], g)[0], v)


def test_saturation_and_zero():
    g = 1.0 / 64
    v = np.zeros((2, 16))
    v[0, 0] = 1e6                    # amax / (6 g) far above 448: the scale saturates at 448
    v[0, 1] = -3.0
    v[0, 2] = 1.0
    codes, scales = quantize_nvfp4(v, g)
    assert scales[0, 0] == 0x7E and e4m3_decode(0x7E) == 448.0
    rt = nvfp4_values(codes, scales) * g
    assert rt[0, 0] == 6 * 448 * g           # the element saturates at 6
    assert rt[0, 1] == -0.5 * 7              # s g = 7: -3 / 7 = -0.43 rounds to -0.5
    assert rt[0, 2] == 0.0                   # 1 / 7 = 0.14 rounds to 0
    assert (codes[1] & 7).max() == 0 and scales[1, 0] == 0


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        quantize_nvfp4(np.zeros((1, 8)), 1.0)
    with pytest.raises(ValueError):
        quantize_nvfp4(np.zeros((1, 16)), 0.0)
    with pytest.raises(ValueError):
        quantize_nvfp4(np.full((1, 16), np.inf), 1.0)


def _w4a4_problem(gated, E=4, H=64, I=32, k=2, T=5, seed=0):
    rng = np.random.default_rng(seed)
    n1 = 2 * I if gated else I

    def fp4(n, kk):
        return rng.integers(0, 256, size=(E, n, kk // 2), dtype=np.uint8), \
            rng.integers(0x20, 0x40, size=(E, n, kk // 16), dtype=np.uint8)

    c13, s13 = fp4(n1, H)
    c2, s2 = fp4(H, I)
    w = Weights("nvfp4", gated, c13, s13, c2, s2,
                w13_global=rng.uniform(0.5, 2, E).astype(np.float32),
                w2_global=rng.uniform(0.5, 2, E).astype(np.float32),
                a13_global=np.float32(0.02), a2_global=rng.uniform(0.5, 4, E).astype(np.float32))
    x = (rng.normal(size=(T, H)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    tw = rng.uniform(0.1, 1, size=(T, k)).astype(np.float32)
    return w, x, ids, tw


def test_w4a4_scales_apply_exactly():
    # ReLU^2 is homogeneous of degree 2: doubling x and its scale keeps every
    # x code, quadruples h, and with h's scales quadrupled keeps every h code
    w, x, ids, tw = _w4a4_problem(gated=False)
    base = fused_moe(x, ids, tw, w, act_format="nvfp4")
    x2 = x + np.uint16(1 << 7)          # +1 in the bf16 exponent field: exactly 2x (normal inputs)
    w2 = Weights(w.weight_format, w.gated, w.w13_codes, w.w13_scales, w.w2_codes, w.w2_scales,
                 w.w13_global, w.w2_global, a13_global=np.float32(2 * w.a13_global),
                 a2_global=(4 * w.a2_global).astype(np.float32))
    assert np.abs(base).max() > 0
    np.testing.assert_array_equal(fused_moe(x2, ids, tw, w2, act_format="nvfp4"), 4 * base)
    # and a changed h scale does change the result (the scale is not ignored)
    w3 = Weights(w.weight_format, w.gated, w.w13_codes, w.w13_scales, w.w2_codes, w.w2_scales,
                 w.w13_global, w.w2_global, a13_global=w.a13_global,
                 a2_global=(w.a2_global * 1.37).astype(np.float32))
    assert not np.array_equal(fused_moe(x, ids, tw, w3, act_format="nvfp4"), base)


def test_w4a4_expert_relabeling():
    w, x, ids, tw = _w4a4_problem(gated=True, seed=3)
    perm = np.array([2, 0, 3, 1])          # new label of old expert e is perm[e]
    inv = np.argsort(perm)

    def re(a):
        return None if a is None else np.asarray(a)[inv]

    wp = Weights("nvfp4", True, re(w.w13_codes), re(w.w13_scales), re(w.w2_codes), re(w.w2_scales),
                 re(w.w13_global), re(w.w2_global), a13_global=w.a13_global, a2_global=re(w.a2_global))
    np.testing.assert_array_equal(fused_moe(x, perm[ids].astype(np.int32), tw, wp, act_format="nvfp4"),
                                  fused_moe(x, ids, tw, w, act_format="nvfp4"))


def test_w4a4_needs_nvfp4_weights_and_scales():
    w, x, ids, tw = _w4a4_problem(gated=True)
    w.a2_global = None
    with pytest.raises(ValueError):
        fused_moe(x, ids, tw, w, act_format="nvfp4")
