"""Pins of the oracle's format code against things other than itself: the OCP
E2M1 table, torch's float8 / bfloat16 conversions (library routines), closed
form special cases and invariants of the MXFP8 scale rule."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_matches_ocp_table():
    rows = _golden_table("e2m1_table.txt")
    assert len(rows) == 16
    codes = np.array([int(r[0]) for r in rows])
    want = np.array([float(r[1]) for r in rows])
    got = F.e2m1_decode(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))   # code 8 is -0


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2                      # 0x7F and 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e8m0_decode_matches_torch():
    codes = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.e8m0_decode(codes), ref)
    assert np.isnan(F.e8m0_decode(np.array([255])))[0]
    assert F.e8m0_decode(np.array([127]))[0] == 1.0


def test_fp4_nibble_order():
    # byte 0x72: element 0 in the low nibble (code 2 = 1.0), element 1 high (code 7 = 6.0)
    assert F.unpack_fp4(np.array([[0x72, 0x9A]], dtype=np.uint8)).tolist() == [[2, 7, 10, 9]]


def test_dequant_mxfp4_scale_applies_per_32():
    packed = np.zeros((1, 32), dtype=np.uint8)          # one row, K = 64
    packed[0, 0] = 0x72                                 # k=0: 1.0, k=1: 6.0
    packed[0, 16] = 0x0D                                # k=32: -3.0
    scales = np.array([[128, 125]], dtype=np.uint8)     # x2 for k<32, x1/4 for k>=32
    w = F.dequant_mxfp4(packed, scales)
    assert w.shape == (1, 64)
    assert w[0, 0] == 2.0 and w[0, 1] == 12.0 and w[0, 32] == -0.75
    assert np.count_nonzero(w) == 3


def test_dequant_nvfp4_block_and_global_scale():
    packed = np.zeros((1, 16), dtype=np.uint8)          # K = 32, two blocks of 16
    packed[0, 0] = 0x05                                 # k=0: 3.0
    packed[0, 8] = 0x0F                                 # k=16: -6.0
    scales = np.array([[0x3C, 0x30]], dtype=np.uint8)   # E4M3 1.5 and 0.5
    w = F.dequant_nvfp4(packed, scales, np.float32(0.25))
    assert w[0, 0] == 3.0 * 1.5 * 0.25 and w[0, 16] == -6.0 * 0.5 * 0.25


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.0e38)]
    # add exact ties (low half 0x8000) with both parities of the kept bit
    tie_bits = (rng.integers(0, 2 ** 16, size=4096).astype(np.uint32) << 16) | 0x8000
    ties = tie_bits.view(np.float32)
    v = np.concatenate([v, ties[np.isfinite(ties) & (np.abs(ties) < 3.0e38)],
                        np.array([0.0, -0.0, 1e-45, -1e-40], dtype=np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.bf16_encode(v.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(F.bf16_decode(ref), torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy())


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.bf16_decode(bits)
    return vals[np.isfinite(vals)]


def test_mxfp8_elements_match_torch_rne():
    """Every finite bf16 value with |v| < 464, placed in a block whose maximum
    is 448 (so the scale is 2^0 and q = v), encodes like torch's fp32 ->
    float8_e4m3fn conversion (round half to even)."""
    vals = _all_finite_bf16()
    vals = vals[np.abs(vals) <= 448.0]
    n = -(-vals.size // 31) * 31
    padded = np.zeros(n)
    padded[:vals.size] = vals
    rows = padded.reshape(-1, 31)
    block = np.concatenate([np.full((rows.shape[0], 1), 448.0), rows], axis=1)
    codes, scales = F.quantize_mxfp8(block)
    assert np.all(scales == 127)
    ref = torch.from_numpy(block.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)


@pytest.mark.parametrize("shift", [-90, -60, -9, -1, 1, 7, 40, 90])
def test_mxfp8_scale_shift_invariance(shift):
    """Scaling a row by 2^n moves every scale code by n and keeps every
    element code (the scale is a pure exponent)."""
    rng = np.random.default_rng(shift + 1000)
    x = rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)) * 3)
    x = F.bf16_decode(F.bf16_encode(x))
    c0, s0 = F.quantize_mxfp8(x)
    c1, s1 = F.quantize_mxfp8(np.ldexp(x, shift))
    assert np.array_equal(c0, c1)
    assert np.array_equal(s1.astype(int), s0.astype(int) + shift)


def test_mxfp8_block_max_lands_in_top_binade_and_round_trip():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((200, 96)) * np.exp(rng.standard_normal((200, 1)) * 4)
    codes, scales = F.quantize_mxfp8(x)
    dq = F.dequant_mxfp8(codes, scales)
    s = scales.astype(int) - 127
    q = np.abs(x).reshape(200, 3, 32) / np.exp2(s)[..., None]
    qmax = q.max(-1)
    assert np.all((qmax >= 256.0) & (qmax < 512.0))
    # error bound: half an E4M3 ulp at |q| for unsaturated elements, <= 12.5% when saturated
    a = q.reshape(200, 96)
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6) - 3)
    err = np.abs(dq - x) / np.repeat(np.exp2(s), 32, axis=1)
    sat = a >= 448.0
    assert np.all(err[~sat] <= 0.5 * ulp[~sat] * (1 + 1e-12))
    assert np.all(err[sat] <= 0.125 * a[sat])
    # idempotent: quantizing the dequantized values gives the same codes
    c2, s2 = F.quantize_mxfp8(dq)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)


def test_mxfp8_saturation_and_zero_cases():
    row = np.zeros((1, 32))
    row[0, :6] = [449.0, 463.99, 464.0, 511.9, -500.0, 300.0]
    codes, scales = F.quantize_mxfp8(row)
    assert scales[0, 0] == 127
    assert codes[0, :6].tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, F.quantize_mxfp8(np.full((1, 32), 300.0))[0][0, 0]]
    assert F.e4m3_decode(codes[0, 5]) == 288.0          # 300 -> nearest E4M3 (ulp 32) = 288
    z = np.zeros((2, 32))
    z[1, 3] = -0.0
    codes, scales = F.quantize_mxfp8(z)
    assert np.all(scales == 0) and codes[0].max() == 0
    assert codes[1, 3] == 0x80 and np.count_nonzero(codes[1]) == 1
    # negative underflow keeps its sign: -2^-11 in a block with max 1.0 (s = -8)
    u = np.zeros((1, 32))
    u[0, 0], u[0, 1] = 1.0, -2.0 ** -20
    codes, scales = F.quantize_mxfp8(u)
    assert scales[0, 0] == 119 and codes[0, 0] == 0x78 and codes[0, 1] == 0x80


def test_mxfp8_rejects_nonfinite():
    with pytest.raises(ValueError):
        F.quantize_mxfp8(np.array([[np.inf] + [0.0] * 31]))
