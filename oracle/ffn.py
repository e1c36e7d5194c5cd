"""Routed-expert FFN of b12x ``moe.fused_moe`` in fp64 (oracle).

TEST INFRASTRUCTURE ONLY.

What the pages fix (b12x README "What's in here" / "Using it"; vLLM b12x page
"Supported Configurations" and "ModelOpt block codecs"):

* the op is a routed-expert FFN over caller-supplied ``topk_ids`` /
  ``topk_weights``, with expert weights kept packed in MXFP4 or NVFP4;
* activations are BF16 (W4A16: inline weight dequant, no activation-scale
  math), dynamically quantized MXFP8 (W4A8), or NVFP4 with NVFP4 weights
  (W4A4; vLLM b12x page "Supported Configurations": NVFP4 MoE takes the
  checkpoint's activation format);
* experts are bias-free, SiLU-gated or non-gated ReLU^2;
* the output is the top-k-weighted combine of the experts' outputs.

Readings where the pages are silent:

* gated weights ``w13[E, 2I, H]``: rows ``[0, I)`` are the gate projection,
  rows ``[I, 2I)`` the up projection; ``h = silu(gate) * up`` with
  ``silu(z) = z / (1 + exp(-z))``; no clamp, no bias.
* non-gated weights ``w1[E, I, H]``: ``h = max(w1 x, 0)^2``.
* SwiGLU-OAI (named by b12x README "What's in here", defined nowhere on the
  pages): the published definition of the open-weight gpt-oss models, taken
  as the reading.  Gated weights as for SiLU; the gate is clamped from above
  at ``limit``, the up projection to ``[-limit, limit]``, and
  ``h = gate * sigmoid(alpha * gate) * (up + 1)`` with ``alpha = 1.702`` and
  ``limit = 7``; bias-free like the other activations.
* the expert's intermediate ``h`` is rounded to the precision of the down
  projection's operand before it: bf16 (round to nearest even) for BF16
  activations, MXFP8 (per 32 along I, the same rule as the activations) for
  MXFP8 activations, NVFP4 (per 16 along I against the expert's activation
  scale, the same rule as x) for NVFP4 activations.
* NVFP4 activation scales: one fp32 scale for x (x is quantized once, before
  it reaches any expert) and one per expert for h, given with the weights as
  a checkpoint gives its input scales.
* combine: ``out[t] = sum_j w[t, j] * y[t, j]`` in ascending slot order, with
  the weights used as given (no renormalization); a pair whose id lies outside
  ``[0, E)`` contributes nothing; a repeated id counts once per slot.
* ``topk_ids`` are int32 ``[T, k]``, ``topk_weights`` float32 ``[T, k]``.
"""
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .formats import (bf16_decode, dequant_mxfp4, dequant_nvfp4, dequant_mxfp8,
                      nvfp4_roundtrip, quantize_mxfp8, round_to_bf16)


@dataclass
class Weights:
    """Source-format expert weights (the layout a checkpoint provides).

    ``w13_codes`` uint8 [E, N1, H/2] with N1 = 2I (gated) or I (ReLU^2);
    ``w13_scales`` uint8 [E, N1, H/G]; ``w2_codes`` uint8 [E, H, I/2];
    ``w2_scales`` uint8 [E, H, I/G]; G = 32 (MXFP4, E8M0) or 16 (NVFP4,
    E4M3); ``w13_global`` / ``w2_global`` float32 [E] for NVFP4, else None;
    ``a13_global`` (float32 scalar, the scale of x) and ``a2_global``
    (float32 [E], the scale of each expert's h) for NVFP4 activations.
    Each array may also be a mapping expert -> per-expert array (then
    ``num_experts`` is required); only the experts a call touches are read.
    """
    weight_format: str
    gated: bool
    w13_codes: np.ndarray
    w13_scales: np.ndarray
    w2_codes: np.ndarray
    w2_scales: np.ndarray
    w13_global: Optional[np.ndarray] = None
    w2_global: Optional[np.ndarray] = None
    a13_global: Optional[float] = None
    a2_global: Optional[np.ndarray] = None
    num_experts: Optional[int] = None   # required when the arrays are per-expert mappings

    @property
    def E(self):
        return self.num_experts if self.num_experts is not None else len(self.w13_codes)

    def _dequant(self, codes, scales, g):
        if self.weight_format == "mxfp4":
            return dequant_mxfp4(codes, scales)
        if self.weight_format == "nvfp4":
            return dequant_nvfp4(codes, scales, g)
        raise ValueError(f"unknown weight format {self.weight_format!r}")

    def w13(self, e):
        g = None if self.w13_global is None else self.w13_global[e]
        return self._dequant(np.asarray(self.w13_codes[e]), np.asarray(self.w13_scales[e]), g)

    def w2(self, e):
        g = None if self.w2_global is None else self.w2_global[e]
        return self._dequant(np.asarray(self.w2_codes[e]), np.asarray(self.w2_scales[e]), g)


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


OAI_ALPHA = 1.702
OAI_LIMIT = 7.0


def swiglu_oai(gate, up):
    """SwiGLU-OAI of gate and up projections (fp64): the gate clamped from
    above at the limit, up clamped to [-limit, limit], then
    gate * sigmoid(alpha * gate) * (up + 1)."""
    g = np.minimum(gate, OAI_LIMIT)
    u = np.clip(up, -OAI_LIMIT, OAI_LIMIT)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-OAI_ALPHA * g)) * (u + 1.0)


ACTIVATIONS = ("silu", "relu2", "swiglu_oai")


def expert_ffn(xa, w13, w2, gated, intermediate, h_global=None, activation=None):
    """One expert on the rows ``xa`` [m, H]: returns y [m, H] (fp64).
    ``h_global``: the expert's NVFP4 activation scale (intermediate "nvfp4").
    ``activation``: "silu" or "swiglu_oai" (gated weights), "relu2"
    (non-gated); None picks "silu" or "relu2" from ``gated``."""
    if activation is None:
        activation = "silu" if gated else "relu2"
    if activation not in ACTIVATIONS or (activation == "relu2") == gated:
        raise ValueError(f"activation {activation!r} with gated={gated}")
    z = xa @ w13.T
    if gated:
        inter = w13.shape[0] // 2
        if activation == "silu":
            h = _silu(z[:, :inter]) * z[:, inter:]
        else:
            h = swiglu_oai(z[:, :inter], z[:, inter:])
    else:
        h = np.maximum(z, 0.0) ** 2
    if intermediate == "bf16":
        h = round_to_bf16(h)
    elif intermediate == "mxfp8":
        h = dequant_mxfp8(*quantize_mxfp8(h))
    elif intermediate == "nvfp4":
        h = nvfp4_roundtrip(h, h_global)
    elif intermediate != "none":
        raise ValueError(f"unknown intermediate rounding {intermediate!r}")
    return h @ w2.T


def fused_moe(x_bits, topk_ids, topk_weights, weights, act_format="bf16",
              intermediate=None, activation=None):
    """Reference fused MoE.  Returns the fp64 output [T, H] before the final
    bf16 rounding.

    x_bits: uint16 bf16 patterns [T, H]; topk_ids int32 [T, k];
    topk_weights float32 [T, k]; weights: ``Weights``.
    act_format: "bf16" (W4A16), "mxfp8" (W4A8: each row of x is MXFP8
    quantized per 32 along H and the GEMMs see the dequantized values) or
    "nvfp4" (W4A4, NVFP4 weights: x quantized per 16 against
    ``weights.a13_global``, h against ``weights.a2_global[e]``).
    intermediate: rounding of h before the down projection; defaults to the
    activation format ("bf16", "mxfp8" or "nvfp4"; "none" keeps fp64).
    activation: "silu", "relu2" or "swiglu_oai"; None picks "silu" for gated
    weights and "relu2" for non-gated ones.
    """
    x = bf16_decode(x_bits)
    ids = np.asarray(topk_ids).astype(np.int64)
    wts = np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    T, k = ids.shape
    E = weights.E
    if act_format == "bf16":
        xa = x
    elif act_format == "mxfp8":
        xa = dequant_mxfp8(*quantize_mxfp8(x))
    elif act_format == "nvfp4":
        if weights.weight_format != "nvfp4" or weights.a13_global is None or weights.a2_global is None:
            raise ValueError("NVFP4 activations need NVFP4 weights and their activation scales")
        xa = nvfp4_roundtrip(x, weights.a13_global)
    else:
        raise ValueError(f"unknown activation format {act_format!r}")
    if intermediate is None:
        intermediate = act_format

    # y[t, j] for every valid pair, expert by expert (each expert dequantized once)
    y = np.zeros((T, k, x.shape[1]), dtype=np.float64)
    valid = (ids >= 0) & (ids < E)
    for e in np.unique(ids[valid]):
        tt, jj = np.nonzero(ids == e)
        hg = None if weights.a2_global is None else weights.a2_global[e]
        y[tt, jj] = expert_ffn(xa[tt], weights.w13(e), weights.w2(e), weights.gated, intermediate, hg,
                               activation)

    out = np.zeros((T, x.shape[1]), dtype=np.float64)
    for j in range(k):
        out += np.where(valid[:, j:j + 1], wts[:, j:j + 1] * y[:, j], 0.0)
    return out
