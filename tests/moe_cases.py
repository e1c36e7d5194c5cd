"""Shared helpers of the GPU parity tests: build a workload on the device,
run the HIP path through the C ABI, run the oracle on the same bytes and
compare.  Not collected by pytest (no test_ prefix)."""
import numpy as np
import torch

import synth
from oracle import Weights, fused_moe

# parity bar for the bf16 output: normwise relative error and max error
REL_FRO = 5e-3
REL_MAX = 2e-2


def bits(t):
    """bf16 tensor -> uint16 numpy (host)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def compare(gpu_out, ref):
    """(rel_fro, rel_max, ok) of the GPU's bf16 output against the fp64 oracle."""
    o = bf16_to_f64(gpu_out)
    nref = np.linalg.norm(ref)
    if nref == 0:
        return 0.0, 0.0, bool(np.all(o == 0))
    rel_fro = float(np.linalg.norm(o - ref) / nref)
    rel_max = float(np.abs(o - ref).max() / np.abs(ref).max())
    return rel_fro, rel_max, rel_fro <= REL_FRO and rel_max <= REL_MAX


class Problem:
    """A workload instance on the GPU: source weights, prepared weights, plan."""

    def __init__(self, wl, max_tokens, gen_device="cuda", weights=None, decode_max_pairs=0, splitk_max_pairs=0,
                 activation=None):
        import fp8_moe_amd as fm
        self.wl = wl
        self.fm = fm
        self.activation = activation or ("silu" if wl.gated else "relu2")
        self.w = weights if weights is not None else synth.make_weights(wl, device=gen_device)
        self.wd = {k: (None if v is None else v.cuda()) for k, v in self.w.items()}
        self.model = fm.FusedMoE(wl.E, wl.H, wl.I, wl.k, wl.weight_format, wl.act_format,
                                 self.activation, max_tokens, self.wd,
                                 decode_max_pairs=decode_max_pairs, splitk_max_pairs=splitk_max_pairs)

    def run(self, x, ids, tw, out=None):
        binding, out = self.model.bind(x, ids, tw, out)
        self.fm.run(binding)
        return out, binding

    def oracle_weights(self, experts=None):
        kw = synth.oracle_weights_kwargs(self.w, experts)
        return Weights(self.wl.weight_format, self.wl.gated, num_experts=self.wl.E, **kw)

    def oracle(self, x, ids, tw, rows=None):
        """fp64 reference for all tokens, or for the token indices ``rows``."""
        x, ids, tw = x.cpu(), ids.cpu(), tw.cpu()
        if rows is not None:
            x, ids, tw = x[rows], ids[rows], tw[rows]
        ids_np = ids.numpy()
        touched = sorted({int(e) for e in ids_np.reshape(-1) if 0 <= e < self.wl.E})
        w = self.oracle_weights(touched)
        return fused_moe(bits(x), ids_np, tw.numpy(), w, act_format=self.wl.act_format,
                         activation=self.activation)


def small_workload(name, E, H, I, k, gated=True, weight_format="mxfp4", act_format="bf16", routing="uniform",
                   x_lognormal=False):
    return synth.Workload(name, E, H, I, k, gated, weight_format, act_format, (1,), routing, x_lognormal)


def scratch_ints(model, name, count):
    """int32 [count] from one of the plan's scratch regions (after a run)."""
    off, nbytes = model.plan.scratch_region(name)
    assert 4 * count <= nbytes
    return model.scratch[off:off + 4 * count].cpu().numpy().view(np.int32)


def tile_edge_tokens(model, k):
    """Tokens whose pairs sit in the first or the last real row of some GEMM
    tile of the last grouped-path run: comparing their output rows reaches
    every routed expert and every tile (both ends of each)."""
    nt = scratch_ints(model, "ntiles", 4)
    n_tiles, rows = int(nt[0]), int(nt[1])
    tiles = scratch_ints(model, "tiles", 4 * n_tiles).reshape(-1, 4)
    sorted_ids = scratch_ints(model, "sorted", rows)
    tokens = set()
    for e, r0, n, _ in tiles:
        seg = sorted_ids[r0:r0 + n]
        live = np.nonzero(seg >= 0)[0]
        assert len(live) > 0, (e, r0, n)
        tokens.add(int(seg[live[0]]) // k)
        tokens.add(int(seg[live[-1]]) // k)
    return sorted(tokens), n_tiles
