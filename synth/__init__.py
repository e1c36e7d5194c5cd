"""Seeded synthetic inputs for the fused-MoE workloads.

Shared by the tests, the benchmark and the smoke check; imported by neither
the oracle nor the product library.  It holds none of the fused-MoE path's
arithmetic: it draws random tensors and encodes the expert weights into the
source FP4 formats a quantized checkpoint would hold (the path itself only
ever decodes weights).  Both the oracle and the GPU path read exactly these
bytes, each with its own decoder.

Workloads (sizes, distributions and routing follow the configurations the
fused_moe path is measured on):

========  ===  =====  =====  =  =====  =======  =======  ======================
name       E     H      I    k  gated  weights  acts     tokens
========  ===  =====  =====  =  =====  =======  =======  ======================
tiny        8    256    128  2  yes    MXFP4    BF16     16
decode    128   2048    768  8  yes    MXFP4    BF16     1, 8, 32
prefill   128   4096   1536  8  yes    NVFP4    BF16     4096
mixed     128   2880   2880  4  no     MXFP4    MXFP8    1, 64, 512, 2048
skew      256   7168   2048  8  yes    NVFP4    BF16     8192
========  ===  =====  =====  =  =====  =======  =======  ======================

Recipe: x ~ N(0, 1) drawn in fp32 and rounded to bf16 (mixed: each token row
first multiplied by exp(N(0, 1)), i.e. LogNormal(0, 1)); weights ~ N(0, 0.02^2)
in fp32, then encoded per expert (MXFP4: E8M0 scale = floor(log2 amax) - 2 per
32 along K, E2M1 round-half-even saturating at 6; NVFP4: fp32 scale
g = amax / (6*448) per expert and matrix, E4M3 block scale per 16 =
RNE(amax_block / (6 g)), E2M1 codes of w / (scale * g)); uniform routing takes
k distinct experts per token uniformly at random; skewed routing draws k
distinct experts per token without replacement with P(e) proportional to
rank(e)^-1.1 over a seeded random ranking (Gumbel top-k); topk_weights are the
softmax of k N(0, 1) logits.  Every tensor has its own torch.Generator seeded
from (workload, tensor, tokens); draws depend on the device (CPU and GPU
generators differ), so a run states the device it generated on.
"""
from dataclasses import dataclass
from typing import Tuple

import torch

BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    E: int
    H: int
    I: int
    k: int
    gated: bool
    weight_format: str   # "mxfp4" | "nvfp4"
    act_format: str      # "bf16" | "mxfp8"
    tokens: Tuple[int, ...]
    routing: str = "uniform"   # "uniform" | "zipf"
    x_lognormal: bool = False

    @property
    def group(self):
        return 32 if self.weight_format == "mxfp4" else 16

    @property
    def n13(self):
        return 2 * self.I if self.gated else self.I

    def weight_bytes_per_expert(self):
        """Packed codes + block scales of one expert (W13/W1 and W2)."""
        elems = self.n13 * self.H + self.H * self.I
        return elems // 2 + elems // self.group


WORKLOADS = {
    "tiny": Workload("tiny", 8, 256, 128, 2, True, "mxfp4", "bf16", (16,)),
    "decode": Workload("decode", 128, 2048, 768, 8, True, "mxfp4", "bf16", (1, 8, 32)),
    "prefill": Workload("prefill", 128, 4096, 1536, 8, True, "nvfp4", "bf16", (4096,)),
    "mixed": Workload("mixed", 128, 2880, 2880, 4, False, "mxfp4", "mxfp8", (1, 64, 512, 2048),
                      x_lognormal=True),
    "skew": Workload("skew", 256, 7168, 2048, 8, True, "nvfp4", "bf16", (8192,), routing="zipf"),
}

_STREAMS = {"x": 1, "w13": 2, "w2": 3, "ids": 4, "weights": 5, "act_scales": 6}


def _gen(wl, stream, tokens, device, salt=0):
    idx = list(WORKLOADS).index(wl.name) if wl.name in WORKLOADS else 7
    seed = (BASE_SEED * 1000003 + idx * 10007 + _STREAMS[stream] * 101 + tokens + salt * 7919) % (2 ** 62)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make_x(wl, T, device="cpu", salt=0):
    """bf16 activations [T, H]; ``salt`` selects another draw of the same shape."""
    g = _gen(wl, "x", T, device, salt)
    x = torch.randn(T, wl.H, generator=g, device=device, dtype=torch.float32)
    if wl.x_lognormal:
        x = x * torch.exp(torch.randn(T, 1, generator=g, device=device, dtype=torch.float32))
    return x.to(torch.bfloat16)


def make_routing(wl, T, device="cpu", salt=0):
    """(topk_ids int32 [T, k], topk_weights float32 [T, k])."""
    g = _gen(wl, "ids", T, device, salt)
    if wl.routing == "uniform":
        scores = torch.rand(T, wl.E, generator=g, device=device)
    elif wl.routing == "zipf":
        perm = torch.randperm(wl.E, generator=g, device=device)
        rank = torch.empty_like(perm)
        rank[perm] = torch.arange(wl.E, device=device)
        logp = -1.1 * torch.log(rank.to(torch.float32) + 1.0)
        u = torch.rand(T, wl.E, generator=g, device=device).clamp_min(1e-20)
        scores = logp[None, :] - torch.log(-torch.log(u))
    else:
        raise ValueError(wl.routing)
    ids = torch.topk(scores, wl.k, dim=1).indices.to(torch.int32)
    gw = _gen(wl, "weights", T, device, salt)
    logits = torch.randn(T, wl.k, generator=gw, device=device, dtype=torch.float32)
    return ids.contiguous(), torch.softmax(logits, dim=1).contiguous()


def _e2m1_codes(q):
    """Nearest E2M1 code (ties to even code, saturating at 6) of fp32 values."""
    a = q.abs()
    mag = ((a > 0.25).to(torch.uint8) + (a >= 0.75).to(torch.uint8) + (a > 1.25).to(torch.uint8)
           + (a >= 1.75).to(torch.uint8) + (a > 2.5).to(torch.uint8) + (a >= 3.5).to(torch.uint8)
           + (a > 5.0).to(torch.uint8))
    return mag | ((q < 0).to(torch.uint8) << 3)


def _pack(codes):
    return codes[..., 0::2] | (codes[..., 1::2] << 4)


def _encode_mxfp4(w):
    n, k = w.shape
    blocks = w.reshape(n, k // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)
    s = torch.clamp(ex.to(torch.int32) - 1 - 2, -127, 127)
    s = torch.where(amax == 0, torch.full_like(s, -127), s)
    q = torch.ldexp(blocks, (-s).to(torch.float32)[..., None])
    codes = _e2m1_codes(q).reshape(n, k)
    return _pack(codes), (s + 127).to(torch.uint8)


def _encode_nvfp4(w):
    n, k = w.shape
    amax = w.abs().amax()
    g = torch.where(amax > 0, amax / (6.0 * 448.0), torch.ones_like(amax)).to(torch.float32)
    blocks = w.reshape(n, k // 16, 16)
    bamax = blocks.abs().amax(dim=-1)
    b = torch.clamp(bamax / (6.0 * g), max=448.0).to(torch.float8_e4m3fn)
    bdec = b.to(torch.float32)
    denom = torch.where(bdec > 0, bdec * g, torch.ones_like(bdec))
    q = torch.where(bdec[..., None] > 0, blocks / denom[..., None], torch.zeros_like(blocks))
    codes = _e2m1_codes(q).reshape(n, k)
    return _pack(codes), b.view(torch.uint8), g


def make_weights(wl, device="cpu", std=0.02):
    """Packed source-format weights as a dict of tensors on ``device``:
    w13_codes [E, N1, H/2], w13_scales [E, N1, H/G], w2_codes [E, H, I/2],
    w2_scales [E, H, I/G], w13_global / w2_global [E] (NVFP4 only), and for NVFP4
    weights the activation scales a13_global [1] and a2_global [E]."""
    out = {}
    for name, (n, k) in (("w13", (wl.n13, wl.H)), ("w2", (wl.H, wl.I))):
        g = _gen(wl, name, 0, device)
        codes = torch.empty(wl.E, n, k // 2, dtype=torch.uint8, device=device)
        scales = torch.empty(wl.E, n, k // wl.group, dtype=torch.uint8, device=device)
        glob = torch.empty(wl.E, dtype=torch.float32, device=device)
        for e in range(wl.E):
            w = torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std
            if wl.weight_format == "mxfp4":
                codes[e], scales[e] = _encode_mxfp4(w)
            else:
                codes[e], scales[e], glob[e] = _encode_nvfp4(w)
        out[name + "_codes"] = codes
        out[name + "_scales"] = scales
        out[name + "_global"] = glob if wl.weight_format == "nvfp4" else None
    if wl.weight_format == "nvfp4":
        # activation scales a checkpoint would carry for NVFP4 activations (its input
        # scales): x ~ N(0, 1) rows, so a block maximum of about 8 maps to the largest
        # block scale; h ~ (std^2 H) times O(1) factors, one scale per expert, spread
        # by a seeded factor in [0.75, 1.25]
        g = _gen(wl, "act_scales", 0, "cpu")
        out["a13_global"] = torch.tensor([8.0 / (6 * 448)], dtype=torch.float32, device=device)
        spread = 0.75 + 0.5 * torch.rand(wl.E, generator=g, dtype=torch.float32)
        out["a2_global"] = (spread * (16.0 * std * std * wl.H / (6 * 448))).to(torch.float32).to(device)
    return out


def make_dense_weight(n, k, weight_format, seed, device="cpu", std=0.02):
    """One packed weight matrix W [n, k] (N(0, std) quantized like the expert
    weights): (codes uint8 [n, k/2], scales uint8 [n, k/G], global fp32 [1] or
    None) on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed((BASE_SEED * 1000003 + 99991 * n + 7919 * k + seed) % (2 ** 62))
    w = torch.randn(n, k, generator=g, device=device, dtype=torch.float32) * std
    if weight_format == "mxfp4":
        codes, scales = _encode_mxfp4(w)
        return codes, scales, None
    codes, scales, glob = _encode_nvfp4(w)
    return codes, scales, torch.tensor([float(glob)], dtype=torch.float32, device=device)


def make_dense_x(m, k, seed, device="cpu"):
    """bf16 activation rows [m, k] for the dense GEMM, N(0, 1)."""
    g = torch.Generator(device=device)
    g.manual_seed((BASE_SEED * 1000003 + 104729 * m + 31 * k + seed + 17) % (2 ** 62))
    return torch.randn(m, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def oracle_weights_kwargs(wdict, experts=None):
    """The weight dict as host NumPy arrays for building the oracle's
    ``Weights``; with ``experts`` given, each array becomes a mapping
    expert -> array holding only those experts."""
    res = {}
    for key, t in wdict.items():
        if t is None:
            res[key] = None
        elif key == "a13_global":  # one value
            res[key] = t.cpu().numpy()[0]
        elif experts is None or t.dim() == 1:
            res[key] = t.cpu().numpy()
        else:
            res[key] = {int(e): t[int(e)].cpu().numpy() for e in experts}
    return res
