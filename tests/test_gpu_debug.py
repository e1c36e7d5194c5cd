"""The library's debug aids on the GPU: a scratch filled with 0xFF bytes
before priming (B12X_DEBUG_SCRATCH_FILL=1) changes no result of any path, so
no kernel reads scratch that the same call did not write; per-stage timing
(B12X_TIMING=1) prints one line per stage of an eager run and stays out of
a captured graph."""
import re

import pytest
import torch

import synth
from moe_cases import Problem, small_workload

pytestmark = pytest.mark.gpu

# (weight format, activation format, gated): every fused-decode, two-kernel
# decode and grouped-path variant; T = 1, 16, 200 at k = 4 take the split-K
# decode, decode and grouped paths
FORMATS = [("mxfp4", "bf16", True), ("mxfp4", "mxfp8", False), ("nvfp4", "bf16", True), ("nvfp4", "nvfp4", True)]
TOKENS = [(1, 3), (16, 2), (200, 1)]


@pytest.mark.parametrize("wf,af,gated", FORMATS)
def test_scratch_fill_changes_no_result(monkeypatch, wf, af, gated):
    import fp8_moe_amd as fm
    wl = small_workload("fill", 16, 256, 192, 4, gated=gated, weight_format=wf, act_format=af)
    pr = Problem(wl, 256)
    filled = torch.empty_like(pr.model.scratch)
    monkeypatch.setenv("B12X_DEBUG_SCRATCH_FILL", "1")
    fm.prime(pr.model.plan, filled)
    monkeypatch.delenv("B12X_DEBUG_SCRATCH_FILL")
    torch.cuda.synchronize()
    # the fill reached every region the paths read and write
    for name in fm.REGIONS:
        off, nbytes = pr.model.plan.scratch_region(name)
        assert bool((filled[off:off + nbytes] == 255).all()), name
    for T, path in TOKENS:
        print(f"fill {wf}/{af} T={T}", flush=True)
        x = synth.make_x(wl, T, device="cuda")
        ids, tw = synth.make_routing(wl, T, device="cuda")
        ref, rb = pr.run(x, ids, tw)
        assert fm.binding_query(rb, "path") == path
        out = torch.full_like(ref, float("nan"))
        b = fm.bind(pr.model.plan, filled, pr.model.experts, x, ids, tw, out)
        for _ in range(2):
            fm.run(b)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), (wf, af, T)


def test_timing_prints_every_stage(monkeypatch, capfd):
    import fp8_moe_amd as fm
    wl = small_workload("timing", 16, 256, 192, 4, weight_format="nvfp4", act_format="nvfp4")
    pr = Problem(wl, 256)
    for T, path in TOKENS:
        x = synth.make_x(wl, T, device="cuda")
        ids, tw = synth.make_routing(wl, T, device="cuda")
        ref, _ = pr.run(x, ids, tw)
        monkeypatch.setenv("B12X_TIMING", "1")
        b, out = pr.model.bind(x, ids, tw)
        monkeypatch.delenv("B12X_TIMING")
        capfd.readouterr()
        fm.run(b)
        torch.cuda.synchronize()
        lines = [ln for ln in capfd.readouterr().err.splitlines() if ln.startswith("b12x_moe_run:")]
        assert len(lines) == fm.binding_query(b, "num_stages"), lines
        for ln in lines:
            m = re.match(r"b12x_moe_run: path (\d) T (\d+) +(\w+) +([0-9.]+) us$", ln)
            assert m and int(m.group(1)) == path and int(m.group(2)) == T, ln
            assert float(m.group(4)) > 0
        assert torch.equal(out, ref)
        # captured: no event, no wait, no line; every replay gives the eager result
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fm.run(b, s)
        torch.cuda.synchronize()
        assert "b12x_moe_run:" not in capfd.readouterr().err
        for _ in range(3):
            out.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref)
        del g


@pytest.mark.parametrize("wf,af,gated", FORMATS[:2])
def test_forced_fallback_on_a_filled_scratch_with_a_live_count(monkeypatch, wf, af, gated):
    """Everything at once: a scratch filled with 0xFF bytes before priming, a
    binding at capacity with the token count in device memory, and (bf16
    activations) fused-decode waits forced to run out so that every down part
    computes its gate/up groups itself.  Each token count gives the ordinary
    binding's output bit for bit."""
    import fp8_moe_amd as fm
    wl = small_workload("all", 16, 256, 192, 4, gated=gated, weight_format=wf, act_format=af)
    pr = Problem(wl, 256)
    filled = torch.empty_like(pr.model.scratch)
    monkeypatch.setenv("B12X_DEBUG_SCRATCH_FILL", "1")
    fm.prime(pr.model.plan, filled)
    monkeypatch.delenv("B12X_DEBUG_SCRATCH_FILL")
    cap = 256
    x = torch.zeros(cap, wl.H, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(cap, wl.k, dtype=torch.int32, device="cuda")
    tw = torch.zeros(cap, wl.k, dtype=torch.float32, device="cuda")
    out = torch.empty(cap, wl.H, dtype=torch.bfloat16, device="cuda")
    t_live = torch.zeros(1, dtype=torch.int32, device="cuda")
    monkeypatch.setenv("B12X_DEBUG_FORCE_GIVEUP", "1")
    b = fm.bind_live(pr.model.plan, filled, pr.model.experts, x, ids, tw, out, t_live)
    monkeypatch.delenv("B12X_DEBUG_FORCE_GIVEUP")
    for T in (1, 16, 200, 16):
        print(f"all-at-once {wf}/{af} T={T}", flush=True)
        xs = synth.make_x(wl, T, device="cuda", salt=T)
        ids_s, tw_s = synth.make_routing(wl, T, device="cuda", salt=T)
        x[:T].copy_(xs)
        ids[:T].copy_(ids_s)
        tw[:T].copy_(tw_s)
        t_live.fill_(T)
        fm.run(b)
        ref, _ = pr.run(xs, ids_s, tw_s)
        torch.cuda.synchronize()
        assert torch.equal(out[:T], ref), (wf, af, T)


def test_two_scratch_buffers_give_the_same_bits():
    """No state outside the scratch: two bindings of one plan over two scratch
    buffers, run alternately on the same inputs, agree bit for bit on every path."""
    import fp8_moe_amd as fm
    wl = small_workload("two", 16, 256, 192, 4)
    pr = Problem(wl, 256)
    other = fm.alloc_scratch(pr.model.plan)
    for T in (1, 16, 200):
        x = synth.make_x(wl, T, device="cuda")
        ids, tw = synth.make_routing(wl, T, device="cuda")
        a = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
        c = torch.empty_like(a)
        ba = fm.bind(pr.model.plan, pr.model.scratch, pr.model.experts, x, ids, tw, a)
        bc = fm.bind(pr.model.plan, other, pr.model.experts, x, ids, tw, c)
        for _ in range(2):
            fm.run(ba)
            fm.run(bc)
        torch.cuda.synchronize()
        assert torch.equal(a, c), T
