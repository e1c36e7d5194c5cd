"""SwiGLU-OAI experts on the GPU against the fp64 oracle: every weight and
activation format on the split-K decode, decode and grouped paths, with
inputs scaled so that a good share of the gate and up values lie beyond the
clamps, and the gpt-oss layer shape (E=128, H=I=2880, top-4, MXFP4 weights)
with bf16 and MXFP8 activations on sampled rows."""
import numpy as np
import pytest
import torch

import synth
from moe_cases import Problem, compare, small_workload

pytestmark = pytest.mark.gpu

FORMATS = [("mxfp4", "bf16"), ("mxfp4", "mxfp8"), ("nvfp4", "bf16"), ("nvfp4", "mxfp8"), ("nvfp4", "nvfp4")]
# T at k = 4: split-K decode, decode, grouped
TOKENS = [(1, 3), (16, 2), (200, 1)]


@pytest.mark.parametrize("wf,af", FORMATS)
@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_swiglu_oai_all_paths(wf, af, scale):
    import fp8_moe_amd as fm
    wl = small_workload("oai", 16, 256, 192, 4, weight_format=wf, act_format=af)
    pr = Problem(wl, 256, activation="swiglu_oai")
    silu = Problem(wl, 256, weights=pr.w)
    for T, path in TOKENS:
        print(f"oai {wf}/{af} x{scale} T={T}", flush=True)
        x = (synth.make_x(wl, T, device="cuda").float() * scale).to(torch.bfloat16)
        ids, tw = synth.make_routing(wl, T, device="cuda")
        out, b = pr.run(x, ids, tw)
        assert fm.binding_query(b, "path") == path
        torch.cuda.synchronize()
        ref = pr.oracle(x, ids, tw)
        rel_fro, rel_max, ok = compare(out, ref)
        assert ok, (wf, af, scale, T, rel_fro, rel_max)
        # the activation is really another one: SiLU on the same inputs is far off
        other, _ = silu.run(x, ids, tw)
        torch.cuda.synchronize()
        assert compare(other, ref)[0] > 0.05


GPT_OSS = [("bf16", 1), ("bf16", 8), ("bf16", 64), ("bf16", 512), ("mxfp8", 1), ("mxfp8", 64), ("mxfp8", 512)]


@pytest.mark.parametrize("af,T", GPT_OSS)
def test_swiglu_oai_gpt_oss_shape(af, T):
    import fp8_moe_amd as fm
    wl = synth.Workload("gpt_oss", 128, 2880, 2880, 4, True, "mxfp4", af, (T,))
    pr = Problem(wl, 512, activation="swiglu_oai")
    x = (synth.make_x(wl, T, device="cuda").float() * 4.0).to(torch.bfloat16)
    ids, tw = synth.make_routing(wl, T, device="cuda")
    out, b = pr.run(x, ids, tw)
    torch.cuda.synchronize()
    print(f"oai gpt-oss {af} T={T} path {fm.binding_query(b, 'path')}", flush=True)
    rows = sorted({0, T // 2, T - 1})
    ref = pr.oracle(x, ids, tw, rows=rows)
    rel_fro, rel_max, ok = compare(out[rows], ref)
    assert ok, (af, T, rel_fro, rel_max)
    assert np.abs(ref).max() > 0
