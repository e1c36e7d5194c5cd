"""Property-based pins of the oracle (hypothesis, derandomized so that every run
draws the same cases): the MXFP8 quantizer's error bound and idempotence, the
routing stage's invariants on arbitrary id lists (dropped and repeated ids
included), and the SwiGLU-OAI activation's logistic identities."""
import math

import numpy as np
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

from oracle import dequant_mxfp8, quantize_mxfp8, swiglu_oai
from oracle.routing import check_tiles, route

SETTINGS = settings(max_examples=200, derandomize=True, deadline=None)
F32_1E30 = float(np.float32(1e30))


def _bf16(a):
    """float32 values truncated to bf16 (a finite bf16 value each)."""
    a = np.asarray(a, dtype=np.float32)
    return (a.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


blocks = hnp.arrays(np.float32, (2, 32), elements=st.floats(-F32_1E30, F32_1E30, width=32, allow_nan=False,
                                                              allow_infinity=False)).map(_bf16)
scaled = st.tuples(blocks, st.integers(-100, 60)).map(lambda t: t[0] * 2.0 ** t[1])


@SETTINGS
@given(scaled)
def test_mxfp8_error_bound(x):
    """Each element is within half a step of the E4M3 grid scaled by the block's
    2^s (the step of its own binade, or the subnormal step 2^(s-9) below
    2^(s-6)), or saturated at 448 * 2^s."""
    codes, scales = quantize_mxfp8(x)
    deq = dequant_mxfp8(codes, scales)
    s = scales.astype(np.int64) - 127
    unit = np.repeat(np.ldexp(1.0, s), 32, axis=-1)
    q = np.abs(x) / unit
    binade = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
    half_step = np.ldexp(1.0, (binade - 4).astype(np.int64)) * unit
    err = np.abs(x - deq)
    saturated = q > 448.0
    assert np.all(np.where(saturated, np.abs(deq) == 448.0 * unit, err <= half_step))
    # the sign survives (a zero keeps its sign bit in the code)
    assert np.all((codes >= 0x80) == np.signbit(x))


@SETTINGS
@given(scaled)
def test_mxfp8_round_trip_is_a_fixed_point(x):
    codes, scales = quantize_mxfp8(x)
    deq = dequant_mxfp8(codes, scales)
    codes2, scales2 = quantize_mxfp8(deq)
    assert np.array_equal(scales2, scales)
    assert np.array_equal(codes2, codes)


id_lists = st.integers(1, 9).flatmap(lambda E: st.tuples(
    st.just(E),
    hnp.arrays(np.int32, st.tuples(st.integers(0, 12), st.integers(1, 4)),
               elements=st.integers(-2, E + 1))))


@SETTINGS
@given(id_lists)
def test_routing_invariants(case):
    E, ids = case
    r = route(ids, E, 16, 128)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(r.counts, np.bincount(flat[valid], minlength=E)[:E])
    assert r.offsets[-1] == valid.sum()
    for e in range(E):
        rows = r.sorted_ids[r.padded_offsets[e]:r.padded_offsets[e + 1]]
        pairs = np.flatnonzero(flat == e)
        # the expert's pairs in ascending order, then padding
        assert np.array_equal(rows[:len(pairs)], pairs)
        assert np.all(rows[len(pairs):] == -1)
        assert (r.padded_offsets[e + 1] - r.padded_offsets[e]) % 16 == 0
        assert r.padded_offsets[e + 1] - r.padded_offsets[e] - len(pairs) < 16
    # pos inverts sorted_ids on the valid pairs and is -1 on the dropped ones
    for p in range(flat.size):
        if valid[p]:
            assert r.sorted_ids[r.pos[p]] == p
        else:
            assert r.pos[p] == -1
    assert check_tiles(r.tiles, len(r.tiles), r.padded_offsets, E, 16, 128) == []


@SETTINGS
@given(st.floats(-6.99, 6.99), st.floats(-6.99, 6.99))
def test_swiglu_oai_odd_and_even_parts(g, u):
    f, f_neg = float(swiglu_oai(np.float64(g), u)), float(swiglu_oai(np.float64(-g), u))
    # sigmoid(z) + sigmoid(-z) = 1 and sigmoid(z) - sigmoid(-z) = tanh(z / 2)
    assert math.isclose(f - f_neg, g * (u + 1.0), rel_tol=1e-12, abs_tol=1e-12)
    assert math.isclose(f + f_neg, g * math.tanh(0.851 * g) * (u + 1.0), rel_tol=1e-12, abs_tol=1e-12)


@SETTINGS
@given(st.floats(-50.0, 50.0), st.floats(-50.0, 50.0))
def test_swiglu_oai_clamps_everywhere(g, u):
    f = float(swiglu_oai(np.float64(g), u))
    assert f == float(swiglu_oai(np.float64(min(g, 7.0)), min(max(u, -7.0), 7.0)))
    # |h| <= |gate| * 8 below the clamps, and h has the sign of gate * (up + 1)
    assert abs(f) <= 8.0 * min(abs(g), 7.0) + 1e-12
    if f != 0.0:
        assert math.copysign(1.0, f) == math.copysign(1.0, min(g, 7.0) * (min(max(u, -7.0), 7.0) + 1.0))
