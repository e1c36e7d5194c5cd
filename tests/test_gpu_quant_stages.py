"""Element-exact checks of the quantizing stages on the GPU.

* The activation stage (STAGE_QUANT_X) of every binding that quantizes or
  copies a: MXFP8 codes and scales (MXFP4 weights x MXFP8 activations), the
  copy of a's MXFP8 round trips (NVFP4 weights x MXFP8 activations) and of
  a's NVFP4 round trips (W4A4), each on the grouped path (f16 copy scaled by
  a power of two per row) and on the decode path (bf16 copy).  Inputs cover
  every finite bf16 value, each under several block maxima, so that every
  MXFP8 block exponent and every E4M3 block scale occurs, plus rows of exact
  and near NVFP4 ties.  Expected values come from the oracle's quantizers.
* The gate/up epilogues that requantize h: the stored h must be a fixed point
  of the oracle's quantizer (MXFP8 codes and scales, MXFP8 round trips), or,
  for NVFP4 round trips, a block of E2M1 values times one E4M3 scale that is
  a fixed point wherever that scale is a normal E4M3 value.
"""
import numpy as np
import pytest
import torch

import synth
from moe_cases import Problem, small_workload
from oracle import (dequant_mxfp8, e2m1_decode, e4m3_decode, nvfp4_values, quantize_mxfp8, quantize_nvfp4,
                    round_to_bf16)

pytestmark = pytest.mark.gpu


def _bf16_values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bits_of(v):
    """fp64 values that are bf16 values -> uint16 bits."""
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _block_grid(block, cols, shifts):
    """Rows of bf16 bits: every finite bf16 magnitude once per shift d, in
    blocks of `block` values (sorted magnitudes, random signs) whose first
    element is the largest magnitude of the block times 2^d (so that the
    others sit d binades and more below the block maximum).  Rows hold
    blocks of one shift and neighbouring magnitudes."""
    rng = np.random.default_rng(block * 1000 + cols)
    mags = np.arange(0x0000, 0x7F80, dtype=np.uint32)          # sorted by magnitude
    rows = []
    per = block - 1
    for d in shifts:
        n = len(mags) // per * per
        chunk = mags[:n].reshape(-1, per)
        top = _bf16_values(chunk[:, -1].astype(np.uint16)) * 2.0 ** d
        ok = top <= _bf16_values(np.array([0x7F7F], np.uint16))[0]     # the largest finite bf16
        chunk, top = chunk[ok], top[ok]
        # the maximum is a bf16 value times a power of two: exact in bf16
        vals = np.concatenate([top[:, None], _bf16_values(chunk.astype(np.uint16))], axis=1)
        signs = np.where(rng.random(vals.shape) < 0.5, -1.0, 1.0)
        blocks = vals * signs
        per_row = cols // block
        nb = len(blocks) // per_row * per_row
        rows.append(blocks[:nb].reshape(-1, cols))
    return _bits_of(np.concatenate(rows))


def _nv_tie_rows(g, cols):
    """bf16 rows with exact and near NVFP4 ties for a power-of-two scale g:
    blocks whose maximum 6 s g pins the scale s and whose other values are
    the E2M1 midpoints times s g and their bf16 neighbours."""
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    blocks = []
    for sc in (0x08, 0x1B, 0x30, 0x3F, 0x55, 0x7E, 0x03, 0x01):
        s = float(e4m3_decode(np.array([sc]))[0])
        unit = s * g
        vals = []
        for m in mids:
            t = np.float32(m * unit)
            b = int(_bits_of(np.array([t]))[0])
            vals += [b, b + 1, b - 1]
        vals = _bf16_values(np.array(vals, np.uint16))
        vals = np.concatenate([vals, -vals])
        for i in range(0, len(vals), 15):
            blk = np.zeros(16)
            blk[0] = 6.0 * unit
            part = vals[i:i + 15]
            blk[1:1 + len(part)] = part
            blocks.append(blk)
    per_row = cols // 16
    blocks += [np.zeros(16)] * (-len(blocks) % per_row)
    return _bits_of(np.concatenate(blocks).reshape(-1, cols))


def _problem(wfmt, afmt, H, T, decode, a13=None, gated=True):
    wl = small_workload("qstage", 2, H, 128, 1, gated, wfmt, afmt)
    w = synth.make_weights(wl)
    if a13 is not None:
        w["a13_global"] = torch.tensor([a13], dtype=torch.float32)
    # the decode path's two-phase kernels read the copy; the split-K kernel quantizes in registers
    return Problem(wl, T, weights=w, decode_max_pairs=0 if decode else -1, splitk_max_pairs=-1)


def _run_quant_stage(pr, xbits):
    import fp8_moe_amd as fm
    T, H = xbits.shape
    x = torch.from_numpy(xbits.view(np.int16).copy()).view(torch.bfloat16).cuda()
    ids = torch.zeros(T, pr.wl.k, dtype=torch.int32, device="cuda")
    tw = torch.ones(T, pr.wl.k, dtype=torch.float32, device="cuda")
    b, _ = pr.model.bind(x, ids, tw)
    fm.run_stage(b, "quant_x")
    torch.cuda.synchronize()
    return b


def _region(pr, name, dtype, count):
    off, nbytes = pr.model.plan.scratch_region(name)
    item = np.dtype(dtype).itemsize
    assert count * item <= nbytes
    return pr.model.scratch[off:off + count * item].cpu().numpy().view(dtype)


def _copy_values(pr, T, H, f16):
    """The 16-bit activation copy as fp64 values [T, H] (f16 copies times 2^row exponent)."""
    Hp = (H + 127) // 128 * 128
    raw = _region(pr, "xq", np.uint16, T * Hp).reshape(T, Hp)[:, :H]
    if not f16:
        return _bf16_values(raw), None
    e = _region(pr, "xs", np.int32, T)
    vals = raw.view(np.float16).astype(np.float64)
    return vals, e


def _check_f16_copy(vals, e, expect):
    """f16 copy with row exponents e: every value equals f16_RNE(expect * 2^-e)
    and the scaled row maxima stay finite in f16."""
    scaled = np.ldexp(expect, -e[:, None])
    assert np.all(np.abs(scaled) < 65520.0)
    np.testing.assert_array_equal(vals, scaled.astype(np.float16).astype(np.float64))
    # exact wherever the scaled round trip is an f16 value (all of them for these rows)
    exact = scaled.astype(np.float16).astype(np.float64) == scaled
    assert exact.mean() > 0.999


MX_GRID = _block_grid(32, 512, shifts=(0, 1, 3, 8, 9, 16, 20))


@pytest.mark.parametrize("decode", [False, True], ids=["grouped_f16", "decode_bf16"])
def test_mxfp8_round_trip_copy_is_exact(decode):
    # NVFP4 weights x MXFP8 activations: the copy of a's MXFP8 round trips
    x = MX_GRID
    H = x.shape[1]
    expect_all = dequant_mxfp8(*quantize_mxfp8(_bf16_values(x)))
    step = 256 if decode else 2048
    for r0 in range(0, len(x), step):
        xb = x[r0:r0 + step]
        T = len(xb)
        print(f"mxfp8 round trip copy decode={decode} rows {r0}..{r0 + T}", flush=True)
        pr = _problem("nvfp4", "mxfp8", H, T, decode)
        _run_quant_stage(pr, xb)
        vals, e = _copy_values(pr, T, H, f16=not decode)
        expect = expect_all[r0:r0 + T]
        if decode:
            np.testing.assert_array_equal(vals, round_to_bf16(expect))
        else:
            _check_f16_copy(vals, e, expect)


def test_mxfp8_codes_and_scales_are_exact():
    # MXFP4 weights x MXFP8 activations: codes and E8M0 scales (grouped path)
    x = MX_GRID
    T, H = x.shape
    codes_ref, scales_ref = quantize_mxfp8(_bf16_values(x))
    pr = _problem("mxfp4", "mxfp8", H, T, decode=False, gated=False)
    _run_quant_stage(pr, x)
    Hp = (H + 127) // 128 * 128
    codes = _region(pr, "xq", np.uint8, T * Hp).reshape(T, Hp)[:, :H]
    scales = _region(pr, "xs", np.uint8, T * (Hp // 32)).reshape(T, Hp // 32)[:, :H // 32]
    np.testing.assert_array_equal(scales, scales_ref)
    # +0 and -0 codes decode alike; compare values, then the signs of nonzero codes
    np.testing.assert_array_equal(codes & 0x7F, codes_ref & 0x7F)
    nz = (codes_ref & 0x7F) != 0
    np.testing.assert_array_equal(codes[nz], codes_ref[nz])


NV_G = [2.0 ** -7, float(np.float32(8.0 / (6 * 448)))]


@pytest.mark.parametrize("g", NV_G, ids=["g_pow2", "g_synth"])
@pytest.mark.parametrize("decode", [False, True], ids=["grouped_f16", "decode_bf16"])
def test_nvfp4_round_trip_copy_is_exact(decode, g):
    # W4A4: the copy of a's NVFP4 round trips (E2M1 * E4M3, without g)
    grid = _block_grid(16, 512, shifts=(0, 2, 5))
    x = np.concatenate([grid, _nv_tie_rows(g, 512)])
    H = x.shape[1]
    codes, scales = quantize_nvfp4(_bf16_values(x), g)
    expect_all = nvfp4_values(codes, scales)
    used = set(np.unique(scales).tolist())
    assert len(used) >= 120, len(used)          # nearly every E4M3 block scale occurs
    step = 256 if decode else 2048
    for r0 in range(0, len(x), step):
        xb = x[r0:r0 + step]
        T = len(xb)
        print(f"nvfp4 round trip copy decode={decode} g={g} rows {r0}..{r0 + T}", flush=True)
        pr = _problem("nvfp4", "nvfp4", H, T, decode, a13=g)
        _run_quant_stage(pr, xb)
        vals, e = _copy_values(pr, T, H, f16=not decode)
        expect = expect_all[r0:r0 + T]
        if decode:
            np.testing.assert_array_equal(vals, expect)     # E2M1 * E4M3 is exact in bf16
        else:
            assert np.all(e == 0)
            np.testing.assert_array_equal(vals, expect)     # and in f16


# ---------------------------------------------------------------- epilogues

def _run_gemm1(pr, T, seed):
    import fp8_moe_amd as fm
    wl = pr.wl
    x = synth.make_x(wl, T, device="cuda", salt=seed)
    ids, tw = synth.make_routing(wl, T, device="cuda", salt=seed)
    b, _ = pr.model.bind(x, ids, tw)
    for st in ("route", "quant_x", "gemm1"):
        fm.run_stage(b, st)
    torch.cuda.synchronize()
    off, nbytes = pr.model.plan.scratch_region("ntiles")
    rows = int(pr.model.scratch[off:off + 16].cpu().numpy().view(np.int32)[1])
    off, nbytes = pr.model.plan.scratch_region("sorted")
    sorted_ids = pr.model.scratch[off:off + 4 * rows].cpu().numpy().view(np.int32)
    return rows, sorted_ids >= 0


EPI = [("mxfp4", "mxfp8", True), ("mxfp4", "mxfp8", False), ("nvfp4", "mxfp8", True), ("nvfp4", "mxfp8", False),
       ("nvfp4", "nvfp4", True), ("nvfp4", "nvfp4", False)]


@pytest.mark.parametrize("wfmt,afmt,gated", EPI)
def test_requantized_h_is_a_fixed_point(wfmt, afmt, gated):
    print(f"epilogue fixed point {wfmt} x {afmt} gated={gated}", flush=True)
    wl = small_workload("epi", 6, 512, 256, 2, gated, wfmt, afmt, x_lognormal=afmt == "mxfp8")
    pr = Problem(wl, 300, gen_device="cpu", decode_max_pairs=-1)
    rows, live = _run_gemm1(pr, 300, seed=5)
    I, Ip = wl.I, (wl.I + 127) // 128 * 128
    if wfmt == "mxfp4":
        codes = _region(pr, "h", np.uint8, rows * Ip).reshape(rows, Ip)[live][:, :I]
        scales = _region(pr, "hs", np.uint8, rows * (Ip // 32)).reshape(rows, Ip // 32)[live][:, :I // 32]
        vals = dequant_mxfp8(codes, scales)
        c2, s2 = quantize_mxfp8(vals)
        np.testing.assert_array_equal(s2, scales)
        np.testing.assert_array_equal(c2 & 0x7F, codes & 0x7F)
        assert np.abs(vals).max() > 0
        return
    h = _bf16_values(_region(pr, "h", np.uint16, rows * Ip).reshape(rows, Ip)[live][:, :I])
    assert np.abs(h).max() > 0
    if afmt == "mxfp8":
        np.testing.assert_array_equal(dequant_mxfp8(*quantize_mxfp8(h)), h)
        return
    # NVFP4: each block of 16 is E2M1 values times one E4M3 scale; with a normal scale
    # (block maximum 6 s) it is a fixed point of the quantizer for any tensor scale g
    blocks = h.reshape(-1, 16)
    amax = np.abs(blocks).max(axis=1)
    e4m3 = e4m3_decode(np.arange(0x7F))
    e2m1 = np.abs(e2m1_decode(np.arange(8)))
    for blk, m in zip(blocks, amax):
        if m == 0:
            continue
        ok = False
        for c in (6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5):
            s = m / c
            if s in e4m3 and np.all(np.isin(np.abs(blk) / s, e2m1)):
                ok = True
                break
        assert ok, blk
    normal = amax >= 6.0 * 2.0 ** -6
    g = 2.0 ** -3
    v = blocks[normal] * g
    np.testing.assert_array_equal(nvfp4_values(*quantize_nvfp4(v, g)) * g, v)
