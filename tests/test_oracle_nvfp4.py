"""Pins of the oracle's NVFP4 activation quantizer and of the W4A4 FFN.

The quantizer is checked against brute force over explicit value tables
(the eight E2M1 magnitudes of the OCP MX definition and every finite E4M3
magnitude), a worked block that round-trips exactly, and its saturation,
zero and underflow cases.  The FFN's use of the two activation scales is
checked through exact power-of-two scaling (ReLU^2 is homogeneous of degree
two) and invariance under relabeling the experts."""
import numpy as np
import pytest

from oracle import Weights, e4m3_decode, fused_moe, nvfp4_roundtrip, nvfp4_values, quantize_nvfp4

# OCP MX v1.0 E2M1: codes 0..7 are the magnitudes below, bit 3 the sign
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_even(table, q):
    """Index of the table entry nearest to |q|; ties go to the even index."""
    d = np.abs(table[None, :] - np.abs(q)[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    idx = np.where(cand, np.arange(len(table))[None, :], 10 ** 6)
    even = np.where(cand & (np.arange(len(table)) % 2 == 0)[None, :], np.arange(len(table))[None, :], 10 ** 6)
    return np.where(even.min(axis=1) < 10 ** 6, even.min(axis=1), idx.min(axis=1))


def _brute_force(v, g):
    """Codes and scales by exhaustive search, with the quotients in fp32
    (the element quotient as v times the rounded reciprocal of s g)."""
    v = np.asarray(v, dtype=np.float32)
    g = np.float32(g)
    e4m3_mag = e4m3_decode(np.arange(0x7F))           # codes 0x00..0x7E: every finite magnitude
    blocks = v.reshape(-1, 16)
    codes = np.zeros(blocks.shape, np.uint8)
    scales = np.zeros(len(blocks), np.uint8)
    for b, blk in enumerate(blocks):
        t = np.float32(np.abs(blk).max() / np.float32(np.float32(6.0) * g))
        sc = 0x7E if t >= 448.0 else int(_nearest_even(e4m3_mag, np.array([float(t)]))[0])
        scales[b] = sc
        s = np.float32(e4m3_mag[sc])
        u = np.float32(s * g)
        if u == 0:
            continue
        r = np.float32(min(np.float32(np.float32(1.0) / u), np.finfo(np.float32).max))
        q = (blk * r).astype(np.float32).astype(np.float64)
        mag = _nearest_even(E2M1_TABLE, np.minimum(np.abs(q), 6.0))
        codes[b] = mag | np.where(np.signbit(q), 8, 0)
    return codes.reshape(v.shape), scales.reshape(v.shape[:-1] + (v.shape[-1] // 16,))


@pytest.mark.parametrize("seed,g", [(0, 1.0), (1, 0.01), (2, 3.7e-3), (3, 250.0)])
def test_quantizer_matches_brute_force(seed, g):
    rng = np.random.default_rng(seed)
    v = rng.normal(size=(6, 64)) * np.exp(rng.normal(size=(6, 1)) * 2)
    v[0, :16] = 0.0                                       # an all-zero block
    v[1, 16:32] *= 1e-9                                   # a block whose scale underflows
    codes, scales = quantize_nvfp4(v, g)
    bc, bs = _brute_force(v, g)
    np.testing.assert_array_equal(scales, bs)
    # -0 and +0 encode differently but decode alike; compare magnitudes and nonzero signs
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
