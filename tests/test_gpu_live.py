"""A binding at capacity for a live token count (b12x_moe_bind_live): one
graph, captured once, serves token counts on every path of the plan (split-K
decode, decode, grouped) with the count written to device memory between
replays.  Each replay's output rows agree with the oracle and are identical,
bit for bit, to an ordinary binding of the same T on the same inputs (the same
kernels run); rows past the live count are never written."""
import pytest
import torch

import synth
from moe_cases import Problem, compare, small_workload

pytestmark = pytest.mark.gpu

CAP = 4096
# (weights, activations, gated, activation): bf16 activations with the fused decode
# kernel; MXFP8 activations with the quantization stage and the two-launch decode
CASES = [("mxfp4", "bf16", True, "silu"), ("nvfp4", "mxfp8", False, "relu2"), ("mxfp4", "bf16", True, "swiglu_oai")]
# T*k with k = 4: 4 and 28 (split-K), 160 (decode), 1200 and 16384 (grouped)
TS = [1, 7, 40, 300, 4096, 7]


@pytest.mark.parametrize("wfmt,afmt,gated,act", CASES, ids=[f"{c[0]}_{c[1]}_{c[3]}" for c in CASES])
def test_one_graph_serves_every_token_count(wfmt, afmt, gated, act):
    import fp8_moe_amd as fm
    wl = small_workload("live", 16, 256, 128, 4, gated=gated, weight_format=wfmt, act_format=afmt)
    print(f"live binding {wfmt} x {afmt} {act}", flush=True)
    pr = Problem(wl, CAP, activation=act)
    model = pr.model
    full_x = synth.make_x(wl, CAP, device="cuda", salt=7)
    full_ids, full_tw = synth.make_routing(wl, CAP, device="cuda", salt=7)
    x = torch.zeros_like(full_x)
    ids = torch.zeros_like(full_ids)
    tw = torch.zeros_like(full_tw)
    out = torch.empty(CAP, wl.H, dtype=torch.bfloat16, device="cuda")
    t_live = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = fm.bind_live(model.plan, model.scratch, model.experts, x, ids, tw, out, t_live)
    assert fm.binding_query(b, "path") == 4 and fm.binding_query(b, "T") == CAP
    with pytest.raises(fm.B12xUnsupported):
        fm.run_stage(b, "decode1")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fm.run(b, stream=s)
    torch.cuda.synchronize()
    sentinel = torch.tensor(0x7F7F, dtype=torch.int16).view(torch.bfloat16).item()
    ref_out = torch.empty(CAP, wl.H, dtype=torch.bfloat16, device="cuda")
    for T in TS:
        print(f"  T={T}", flush=True)
        x.copy_(full_x)
        ids.copy_(full_ids)
        tw.copy_(full_tw)
        out.fill_(sentinel)
        t_live.fill_(T)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # ordinary binding of the same T on the same inputs
        ordinary = fm.bind(model.plan, model.scratch, model.experts, x[:T], ids[:T], tw[:T], ref_out[:T])
        fm.run(ordinary)
        torch.cuda.synchronize()
        assert torch.equal(out[:T].view(torch.int16), ref_out[:T].view(torch.int16)), T
        assert (out[T:].view(torch.int16) == 0x7F7F).all(), T
        rows = None if T <= 300 else list(range(0, T, 97))
        ref = pr.oracle(x[:T], ids[:T], tw[:T], rows)
        got = out[:T] if rows is None else out[:T][rows]
        rel_fro, rel_max, ok = compare(got, ref)
        assert ok, (T, rel_fro, rel_max)


def test_live_count_out_of_range_writes_nothing():
    import fp8_moe_amd as fm
    wl = small_workload("live_oor", 8, 256, 128, 2)
    pr = Problem(wl, 64)
    model = pr.model
    x = synth.make_x(wl, 64, device="cuda")
    ids, tw = synth.make_routing(wl, 64, device="cuda")
    out = torch.zeros(64, wl.H, dtype=torch.bfloat16, device="cuda")
    t_live = torch.zeros(1, dtype=torch.int32, device="cuda")
    b = fm.bind_live(model.plan, model.scratch, model.experts, x, ids, tw, out, t_live)
    for bad in (0, -3, 65):
        t_live.fill_(bad)
        fm.run(b)
        torch.cuda.synchronize()
        assert (out.view(torch.int16) == 0).all(), bad
    t_live.fill_(64)
    fm.run(b)
    torch.cuda.synchronize()
    rel_fro, rel_max, ok = compare(out, pr.oracle(x, ids, tw))
    assert ok, (rel_fro, rel_max)
