"""Pins of the oracle FFN: a hand-derived worked example, a scalar brute force
(table decode, explicit loops, torch for the roundings), the E=1/top_k=1
dense special case, and invariances (token and slot permutation, linearity in
topk_weights, dropped ids, duplicate ids, power-of-two global scales).
SwiGLU-OAI is pinned by identities of the logistic function (its odd part is
the identity map, its even part is g tanh(alpha g / 2)), by its clamps and by
its zero at up = -1."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import fused_moe, swiglu_oai, Weights
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                c, v = line.split()
                vals[int(c)] = float(v)
    return [vals[c] for c in range(16)]


E2M1 = _table()
E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()


def bf16(v):
    return torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()


def x_bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- worked examples

def test_worked_example_silu_gated():
    E, H, I = 1, 32, 32
    w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13[0, 0, 0] = 0x02        # gate row 0, k=0: 1.0
    w13[0, I, 0] = 0x04        # up row 0, k=0: 2.0
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2[0, 0, 0] = 0x02         # row 0, k=0: 1.0
    w2[0, 1, 0] = 0x71         # row 1, k=0: 0.5, k=1: 6.0
    wts = Weights("mxfp4", True, w13, np.full((E, 2 * I, 1), 127, np.uint8),
                  w2, np.full((E, H, 1), 127, np.uint8))
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    out = fused_moe(x_bits(x), np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), wts)
    with open(os.path.join(GOLDEN, "ffn_worked_example.txt")) as f:
        want = [float(v) for line in f if line.strip() and not line.startswith("#") for v in line.split()]
    assert out[0, :4].tolist() == want
    assert np.count_nonzero(out) == 2


def test_worked_example_relu2():
    E, H, I = 1, 32, 32
    w1 = np.zeros((E, I, H // 2), np.uint8)
    w1[0, 0, 0] = 0x0A         # row 0, k=0: -1.0  -> relu^2 = 0
    w1[0, 1, 0] = 0x05         # row 1, k=0: 3.0   -> 9
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2[0, 0, 0] = 0x10         # row 0: k=1 is 0.5 (high nibble of byte 0)
    wts = Weights("mxfp4", False, w1, np.full((E, I, 1), 127, np.uint8),
                  w2, np.full((E, H, 1), 127, np.uint8))
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    out = fused_moe(x_bits(x), np.zeros((1, 1), np.int32), np.full((1, 1), 0.5, np.float32), wts)
    assert out[0, 0] == 0.5 * 0.5 * 9.0 and np.count_nonzero(out) == 1


# ---------------------------------------------------------------- SwiGLU-OAI

def test_swiglu_oai_odd_part_is_the_gate():
    # sigmoid(z) + sigmoid(-z) = 1, so below the clamp f(g) - f(-g) = g (up + 1)
    g = np.linspace(-6.9, 6.9, 139)
    for u in (-3.0, 0.0, 0.5, 6.0):
        d = swiglu_oai(g, np.full_like(g, u)) - swiglu_oai(-g, np.full_like(g, u))
        assert np.allclose(d, g * (u + 1.0), rtol=0, atol=1e-13)


def test_swiglu_oai_even_part_fixes_alpha():
    # sigmoid(z) - sigmoid(-z) = tanh(z / 2): f(g) + f(-g) = g tanh(1.702 g / 2) at up = 0
    for g in (1e-3, 0.25, 1.0, 3.0, 6.5):
        got = swiglu_oai(np.float64(g), 0.0) + swiglu_oai(np.float64(-g), 0.0)
        assert math.isclose(got, g * math.tanh(0.851 * g), rel_tol=1e-12)


def test_swiglu_oai_clamps():
    g = np.array([-3.0, 0.3, 2.0, 6.99])
    u = np.array([-2.0, 0.0, 1.5, 6.0])
    # the gate is clamped from above at 7 only
    assert np.array_equal(swiglu_oai(np.full(4, 7.0), u), swiglu_oai(np.full(4, 100.0), u))
    assert swiglu_oai(np.float64(-100.0), 1.0) < 0 and swiglu_oai(np.float64(-100.0), 1.0) > -1e-60
    # up is clamped to [-7, 7]
    assert np.array_equal(swiglu_oai(g, np.full(4, 7.0)), swiglu_oai(g, np.full(4, 1e6)))
    assert np.array_equal(swiglu_oai(g, np.full(4, -7.0)), swiglu_oai(g, np.full(4, -1e6)))
    # and h vanishes at up = -1 and at gate = 0
    assert np.all(swiglu_oai(g, np.full(4, -1.0)) == 0)
    assert np.all(swiglu_oai(np.zeros(4), u) == 0)
    # below the clamps: gate 2, up 1.5 -> 2 (1 + tanh(1.702)) / 2 * 2.5
    assert math.isclose(float(swiglu_oai(np.float64(2.0), 1.5)), 2.5 * (1.0 + math.tanh(1.702)), rel_tol=1e-13)


def test_worked_example_swiglu_oai():
    # the SiLU worked example's weights: gate 1, up 2 -> h = sigmoid(1.702) * 3, rounded to bf16
    E, H, I = 1, 32, 32
    w13 = np.zeros((E, 2 * I, H // 2), np.uint8)
    w13[0, 0, 0] = 0x02
    w13[0, I, 0] = 0x04
    w2 = np.zeros((E, H, I // 2), np.uint8)
    w2[0, 0, 0] = 0x02
    wts = Weights("mxfp4", True, w13, np.full((E, 2 * I, 1), 127, np.uint8),
                  w2, np.full((E, H, 1), 127, np.uint8))
    x = np.zeros((1, H), np.float32)
    x[0, 0] = 1.0
    out = fused_moe(x_bits(x), np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32), wts,
                    activation="swiglu_oai")
    h = 3.0 * (1.0 + math.tanh(0.851)) / 2.0
    assert out[0, 0] == float(bf16([h])[0]) and np.count_nonzero(out) == 1
    with pytest.raises(ValueError):
        fused_moe(x_bits(x), np.zeros((1, 1), np.int32), np.ones((1, 1), np.float32),
                  Weights("mxfp4", False, w13[:, :I], np.full((E, I, 1), 127, np.uint8),
                          w2, np.full((E, H, 1), 127, np.uint8)), activation="swiglu_oai")


# ---------------------------------------------------------------- random tiny problems

def random_weights(rng, fmt, gated, E, H, I):
    n1 = 2 * I if gated else I
    G = 32 if fmt == "mxfp4" else 16
    if fmt == "mxfp4":
        s13 = rng.integers(118, 128, size=(E, n1, H // G)).astype(np.uint8)
        s2 = rng.integers(118, 128, size=(E, H, I // G)).astype(np.uint8)
        g13 = g2 = None
    else:
        s13 = rng.integers(0x18, 0x48, size=(E, n1, H // G)).astype(np.uint8)
        s2 = rng.integers(0x18, 0x48, size=(E, H, I // G)).astype(np.uint8)
        g13 = rng.uniform(0.01, 0.2, size=E).astype(np.float32)
        g2 = rng.uniform(0.01, 0.2, size=E).astype(np.float32)
    return Weights(fmt, gated,
                   rng.integers(0, 256, size=(E, n1, H // 2)).astype(np.uint8), s13,
                   rng.integers(0, 256, size=(E, H, I // 2)).astype(np.uint8), s2, g13, g2)


def scalar_weight(codes, scales, glob, fmt, e, n, k):
    byte = int(codes[e][n][k // 2])
    code = byte & 15 if k % 2 == 0 else byte >> 4
    if fmt == "mxfp4":
        return E2M1[code] * 2.0 ** (int(scales[e][n][k // 32]) - 127)
    return E2M1[code] * E4M3[int(scales[e][n][k // 16])] * float(np.float32(glob[e]))


def torch_mxfp8(v):
    """MXFP8 round trip of a 1-D float64 vector with torch's E4M3 conversion."""
    out = []
    for b in range(0, len(v), 32):
        blk = np.array(v[b:b + 32], dtype=np.float64)
        amax = float(np.abs(blk).max())
        s = -127 if amax == 0 else max(-127, min(127, math.floor(math.log2(amax)) - 8))
        q = torch.tensor(np.clip(blk / 2.0 ** s, -448, 448), dtype=torch.float64).to(torch.float32)
        out += (q.to(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** s).tolist()
    return out


def brute_force(xb, ids, tw, w, act, activation=None):
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    T, H = x.shape
    E = w.E
    n1 = w.w13_codes.shape[1]
    inter = n1 // 2 if w.gated else n1
    out = [[0.0] * H for _ in range(T)]
    for t in range(T):
        xa = torch_mxfp8(x[t].tolist()) if act == "mxfp8" else x[t].tolist()
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                continue
            z = [sum(xa[kk] * scalar_weight(w.w13_codes, w.w13_scales, w.w13_global, w.weight_format, e, n, kk)
                     for kk in range(H)) for n in range(n1)]
            if activation == "swiglu_oai":
                # logistic through tanh: sigmoid(a g) = (1 + tanh(a g / 2)) / 2
                h = [min(z[i], 7.0) * (1.0 + math.tanh(0.851 * min(z[i], 7.0))) / 2.0
                     * (min(max(z[inter + i], -7.0), 7.0) + 1.0) for i in range(inter)]
            elif w.gated:
                h = [z[i] / (1.0 + math.exp(-z[i])) * z[inter + i] for i in range(inter)]
            else:
                h = [max(z[i], 0.0) ** 2 for i in range(inter)]
            h = torch_mxfp8(h) if act == "mxfp8" else bf16(h).tolist()
            for n in range(H):
                y = sum(h[i] * scalar_weight(w.w2_codes, w.w2_scales, w.w2_global, w.weight_format, e, n, i)
                        for i in range(inter))
                out[t][n] += float(np.float32(tw[t, j])) * y
    return np.array(out)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_matches_scalar_brute_force(fmt, gated, act):
    rng = np.random.default_rng([len(fmt), int(gated), len(act)])
    E, H, I, T, k = 3, 64, 32, 3, 2
    w = random_weights(rng, fmt, gated, E, H, I)
    xb = x_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.array([[0, 2], [1, 1], [2, -1]], np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    got = fused_moe(xb, ids, tw, w, act_format=act)
    want = brute_force(xb, ids, tw, w, act)
    scale = np.abs(want).max()
    assert scale > 0
    assert np.abs(got - want).max() <= 1e-12 * scale


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_swiglu_oai_matches_scalar_brute_force(fmt, act):
    rng = np.random.default_rng([len(fmt), 7, len(act)])
    E, H, I, T, k = 3, 64, 32, 3, 2
    w = random_weights(rng, fmt, True, E, H, I)
    # wide inputs so that both clamps are reached
    xb = x_bits(4.0 * rng.standard_normal((T, H)).astype(np.float32))
    ids = np.array([[0, 2], [1, 1], [2, -1]], np.int32)
    tw = rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
    got = fused_moe(xb, ids, tw, w, act_format=act, activation="swiglu_oai")
    want = brute_force(xb, ids, tw, w, act, activation="swiglu_oai")
    scale = np.abs(want).max()
    assert scale > 0
    assert np.abs(got - want).max() <= 1e-12 * scale


def dense_gated(x, w13, w2):
    inter = w13.shape[0] // 2
    z = x @ w13.T
    h = bf16(z[:, :inter] / (1.0 + np.exp(-z[:, :inter])) * z[:, inter:])
    return h @ w2.T


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_single_expert_equals_dense_ffn(fmt):
    rng = np.random.default_rng(11)
    H, I, T = 128, 64, 5
    w = random_weights(rng, fmt, True, 1, H, I)
    W13 = np.array([[scalar_weight(w.w13_codes, w.w13_scales, w.w13_global, fmt, 0, n, k) for k in range(H)]
                    for n in range(2 * I)])
    W2 = np.array([[scalar_weight(w.w2_codes, w.w2_scales, w.w2_global, fmt, 0, n, k) for k in range(I)]
                   for n in range(H)])
    xb = x_bits(rng.standard_normal((T, H)).astype(np.float32))
    x = F.bf16_decode(xb)
    got = fused_moe(xb, np.zeros((T, 1), np.int32), np.ones((T, 1), np.float32), w)
    want = dense_gated(x, W13, W2)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def _problem(seed, fmt="mxfp4", gated=True, E=6, H=64, I=64, T=9, k=3):
    rng = np.random.default_rng(seed)
    w = random_weights(rng, fmt, gated, E, H, I)
    xb = x_bits(rng.standard_normal((T, H)).astype(np.float32))
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    tw = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    return w, xb, ids, tw


@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_token_permutation_is_exact(act):
    w, xb, ids, tw = _problem(21)
    perm = np.random.default_rng(3).permutation(xb.shape[0])
    a = fused_moe(xb, ids, tw, w, act_format=act)
    b = fused_moe(xb[perm], ids[perm], tw[perm], w, act_format=act)
    assert np.array_equal(a[perm], b)


def test_slot_permutation():
    w, xb, ids, tw = _problem(22)
    perm = [2, 0, 1]
    a = fused_moe(xb, ids, tw, w)
    b = fused_moe(xb, ids[:, perm], tw[:, perm], w)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max()


def test_linear_in_topk_weights():
    w, xb, ids, tw = _problem(23)
    a = fused_moe(xb, ids, tw, w)
    b = fused_moe(xb, ids, 2 * tw, w)
    assert np.array_equal(2 * a, b)


def test_out_of_range_id_drops_the_pair():
    w, xb, ids, tw = _problem(24, E=6)
    bad = ids.copy()
    bad[0, 1], bad[4, 0] = 6, -3
    zeroed = tw.copy()
    zeroed[0, 1] = zeroed[4, 0] = 0.0
    assert np.array_equal(fused_moe(xb, bad, tw, w), fused_moe(xb, ids, zeroed, w))


def test_duplicate_ids_count_per_slot():
    w, xb, ids, tw = _problem(25, k=2)
    tw = np.round(tw * 16) / 16          # dyadic weights: their fp32 sum is exact
    dup = ids.copy()
    dup[:, 1] = dup[:, 0]
    single = fused_moe(xb, dup[:, :1], (tw[:, :1] + tw[:, 1:]), w)
    both = fused_moe(xb, dup, tw, w)
    assert np.abs(single - both).max() <= 1e-13 * np.abs(single).max()


def test_nvfp4_global_scales_apply_to_their_matrix():
    w, xb, ids, tw = _problem(26, fmt="nvfp4", gated=False)
    base = fused_moe(xb, ids, tw, w)
    w.w13_global = w.w13_global * np.float32(2.0)      # h = relu(z)^2 scales by 4
    assert np.array_equal(fused_moe(xb, ids, tw, w), 4 * base)
    w.w2_global = w.w2_global * np.float32(0.5)
    assert np.array_equal(fused_moe(xb, ids, tw, w), 2 * base)


def test_per_expert_mapping_weights():
    w, xb, ids, tw = _problem(27)
    touched = sorted(set(ids.reshape(-1).tolist()))
    m = Weights(w.weight_format, w.gated,
                {e: w.w13_codes[e] for e in touched}, {e: w.w13_scales[e] for e in touched},
                {e: w.w2_codes[e] for e in touched}, {e: w.w2_scales[e] for e in touched},
                num_experts=w.E)
    assert np.array_equal(fused_moe(xb, ids, tw, w), fused_moe(xb, ids, tw, m))
