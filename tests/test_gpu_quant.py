"""MXFP8 row quantizer on the GPU: codes and scales bit-exact with the oracle
over every finite bf16 value in several block arrangements."""
import numpy as np
import pytest
import torch

from oracle import formats as F

pytestmark = pytest.mark.gpu


def _finite_bf16_bits():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (b >> 7) & 0xFF
    return b[exp != 0xFF]


def _run(x_bits_np, stride_pad=0):
    import fp8_moe_amd as fm
    rows, cols = x_bits_np.shape
    buf = np.zeros((rows, cols + stride_pad), dtype=np.uint16)
    buf[:, :cols] = x_bits_np
    xt = torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)[:, :cols]
    codes, scales = fm.mxfp8_quantize_rows(xt)
    torch.cuda.synchronize()
    want_c, want_s = F.quantize_mxfp8(F.bf16_decode(x_bits_np))
    return codes.cpu().numpy(), scales.cpu().numpy(), want_c, want_s


def test_all_bf16_sorted_blocks():
    b = _finite_bf16_bits()
    order = np.argsort(F.bf16_decode(b).__abs__(), kind="stable")
    b = b[order]
    b = np.concatenate([b, np.zeros((-b.size) % 256, np.uint16)])
    c, s, wc, ws = _run(b.reshape(-1, 256))
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


def test_all_bf16_shuffled_blocks_with_stride():
    b = _finite_bf16_bits()
    b = np.random.default_rng(1).permutation(b)
    b = np.concatenate([b, np.zeros((-b.size) % 128, np.uint16)])
    c, s, wc, ws = _run(b.reshape(-1, 128), stride_pad=24)
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


def test_anchored_blocks_cover_every_scale():
    """Blocks [anchor, 31 values within 2^-12 .. 1 of it] for anchors across the
    whole bf16 exponent range: subnormal, normal and saturating E4M3 encodes
    at every shared exponent."""
    rng = np.random.default_rng(2)
    rows = []
    for e in range(-133, 128):
        anchor = np.ldexp(1.0 + rng.integers(0, 128) / 128.0, e)
        vals = anchor * np.ldexp(rng.uniform(0.5, 1.0, 31), -rng.integers(0, 13, 31))
        vals *= rng.choice([-1.0, 1.0], 31)
        rows.append(np.concatenate([[anchor], vals]))
    x = np.array(rows)
    x = np.where(np.isfinite(x), x, 0.0)
    xb = F.bf16_encode(np.clip(x, -3.0e38, 3.0e38))
    c, s, wc, ws = _run(xb.reshape(-1, 32))
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)


def test_random_rows_and_special_blocks():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((257, 2880)) * np.exp(rng.standard_normal((257, 1)))
    x[0] = 0.0
    x[1, :32] = -0.0
    x[2, 5] = 1e-40
    xb = F.bf16_encode(x)
    c, s, wc, ws = _run(xb)
    assert np.array_equal(s, ws)
    assert np.array_equal(c, wc)
    assert np.all(s[0] == 0) and c[1, 0] == 0x80
