"""Dense block-scaled FP4 GEMM (b12x README "What's in here": gemm.blockscaled,
the dense interface for raw NVFP4 / MXFP4 operands, whose one-shot mm is a
plain function per "Using it").

TEST INFRASTRUCTURE ONLY (see the package docstring).

out[m, n] = sum_k x[m, k] * W[n, k] in fp64, with x the bf16 activation rows
and W the dequantized weight: E2M1(code) * E8M0(scale per 32 along k) for
MXFP4, E2M1(code) * E4M3(scale per 16 along k) * g for NVFP4 (g the fp32
tensor scale).  The pages fix no arithmetic for it; the reading is the same
as the MoE oracle's weight decode (OCP MX v1.0 element formats) followed by
a plain matrix product.
"""
import numpy as np

from .formats import bf16_decode, dequant_mxfp4, dequant_nvfp4


def dequant_weight(codes, scales, weight_format, global_scale=None):
    """W [n, k] in fp64 from packed codes [n, k/2] and scales."""
    if weight_format == "mxfp4":
        return dequant_mxfp4(codes, scales)
    if weight_format == "nvfp4":
        if global_scale is None:
            raise ValueError("NVFP4 weights need their fp32 tensor scale")
        return dequant_nvfp4(codes, scales, global_scale)
    raise ValueError(f"unknown weight format {weight_format!r}")


def blockscaled_mm(x_bits, codes, scales, weight_format, global_scale=None):
    """x_bits: uint16 bf16 bits [m, k]; returns fp64 [m, n] = x . W^T."""
    x = bf16_decode(np.asarray(x_bits, dtype=np.uint16))
    w = dequant_weight(codes, scales, weight_format, global_scale)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and W disagree on k")
    return x @ w.T
