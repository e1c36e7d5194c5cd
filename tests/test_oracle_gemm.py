"""Pins of the dense block-scaled GEMM oracle: a scalar brute force (table
decode of every nibble and scale, explicit loops), an identity weight that
returns x exactly, exact doubling with the NVFP4 tensor scale and with every
block scale code raised by one, and the rejection of malformed inputs."""
import numpy as np
import pytest
import torch

from oracle import blockscaled_mm
from test_oracle_ffn import E2M1, E4M3, x_bits


def random_dense(rng, fmt, n, k):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    if fmt == "mxfp4":
        scales = rng.integers(120, 134, size=(n, k // 32), dtype=np.uint8)
        return codes, scales, None
    scales = rng.integers(0x20, 0x60, size=(n, k // 16), dtype=np.uint8)  # finite, non-NaN E4M3
    return codes, scales, np.float32(rng.uniform(0.01, 2.0))


def scalar_mm(xb, codes, scales, fmt, g):
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    m, k = x.shape
    n = codes.shape[0]
    out = np.zeros((m, n))
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for kk in range(k):
                byte = int(codes[j][kk // 2])
                code = byte & 0xF if kk % 2 == 0 else byte >> 4
                if fmt == "mxfp4":
                    wv = E2M1[code] * 2.0 ** (int(scales[j][kk // 32]) - 127)
                else:
                    wv = E2M1[code] * E4M3[int(scales[j][kk // 16])] * float(g)
                acc += float(x[i][kk]) * wv
            out[i][j] = acc
    return out


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_matches_scalar_brute_force(fmt):
    rng = np.random.default_rng(len(fmt))
    m, n, k = 3, 5, 64
    codes, scales, g = random_dense(rng, fmt, n, k)
    xb = x_bits(rng.standard_normal((m, k)).astype(np.float32))
    got = blockscaled_mm(xb, codes, scales, fmt, g)
    want = scalar_mm(xb, codes, scales, fmt, g)
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def test_identity_weight_returns_x():
    # E2M1 code 2 is 1.0 (closed form: e = 1, m = 0), E8M0 code 127 is 2^0
    n = k = 64
    nib = np.zeros((n, k), np.uint8)
    nib[np.arange(n), np.arange(k)] = 2
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((n, k // 32), 127, np.uint8)
    rng = np.random.default_rng(3)
    xb = x_bits(rng.standard_normal((4, k)).astype(np.float32))
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(blockscaled_mm(xb, codes, scales, "mxfp4"), x)


def test_scales_multiply_exactly():
    rng = np.random.default_rng(5)
    m, n, k = 2, 16, 96
    codes, scales, g = random_dense(rng, "nvfp4", n, k)
    xb = x_bits(rng.standard_normal((m, k)).astype(np.float32))
    base = blockscaled_mm(xb, codes, scales, "nvfp4", g)
    assert np.array_equal(blockscaled_mm(xb, codes, scales, "nvfp4", np.float32(2 * g)), 2 * base)
    mcodes, mscales, _ = random_dense(rng, "mxfp4", n, k)
    mbase = blockscaled_mm(xb, mcodes, mscales, "mxfp4")
    assert np.array_equal(blockscaled_mm(xb, mcodes, mscales + 1, "mxfp4"), 2 * mbase)


def test_rejects_malformed_inputs():
    rng = np.random.default_rng(7)
    codes, scales, g = random_dense(rng, "nvfp4", 16, 64)
    xb = x_bits(rng.standard_normal((2, 64)).astype(np.float32))
    with pytest.raises(ValueError):
        blockscaled_mm(xb, codes, scales, "nvfp4", None)
    with pytest.raises(ValueError):
        blockscaled_mm(xb[:, :32], codes, scales, "nvfp4", g)
    with pytest.raises(ValueError):
        blockscaled_mm(xb, codes, scales, "fp8")
    bad = np.full((16, 2), 0xFF, np.uint8)  # E8M0 NaN
    with pytest.raises(ValueError):
        blockscaled_mm(xb, codes, bad, "mxfp4")
