"""CPU oracle for the fused block-scaled-FP4 MoE FFN (b12x ``moe.fused_moe``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``fp8_moe_amd``) never imports, links or calls it, and this package imports
nothing from the product path.

What it computes (plain, slow, fp64, NumPy):

* ``formats``  - E2M1 / E4M3 / E8M0 decoding, FP4 byte unpacking, MXFP4 and
  NVFP4 weight dequantization, bf16 decode and round-to-nearest-even, the
  MXFP8 row quantizer (E4M3 elements, one E8M0 scale per 32) and the NVFP4
  activation quantizer (E2M1 elements, one E4M3 scale per 16, fp32 tensor
  scale).
* ``routing``  - the integer routing stage: expert histogram, prefix scan,
  stable token permutation, per-expert padded row tiles, inverse positions.
* ``ffn``      - the routed-expert FFN: gather, gate/up projection, SiLU-gated,
  SwiGLU-OAI or ReLU^2 activation, down projection and the top-k-weighted
  combine.
* ``gemm``     - the dense block-scaled FP4 GEMM (gemm.blockscaled mm).

Sources are the b12x pages: the README ("What's in here" and "Using it": the
fused_moe op, its W4A16 / dynamic-W4A8 modes, the SiLU / ReLU2 activations and
the MXFP8 row quantizer), the "PCIe DMA wire modes" section (MXFP8 = one E8M0
scale per 32 values) and the vLLM "b12x Linear and MoE Backends" page
("Supported Configurations" and "ModelOpt block codecs": bias-free SiLU or
non-gated ReLU^2 experts, MXFP8 activations by default for MXFP4 MoE).  The
pages fix none of the arithmetic below; every rule is a reading stated in the
function that applies it.  Element formats follow the public OCP MX v1.0 and
OFP8 definitions.
"""
from .formats import (  # noqa: F401
    e2m1_decode, e4m3_decode, e8m0_decode, unpack_fp4, dequant_mxfp4, dequant_nvfp4,
    bf16_decode, round_to_bf16, bf16_encode, quantize_mxfp8, dequant_mxfp8,
    quantize_nvfp4, nvfp4_values, nvfp4_roundtrip,
)
from .routing import route  # noqa: F401
from .ffn import fused_moe, Weights, swiglu_oai  # noqa: F401
from .gemm import blockscaled_mm  # noqa: F401
