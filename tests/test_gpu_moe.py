"""End-to-end parity of the fused MoE on the GPU against the fp64 oracle:
every workload at its full size (sampled tokens where the oracle would take
too long), small shapes with ragged tiles and ragged K, edge cases, run-to-run
determinism, token-permutation invariance and graph replay."""
import numpy as np
import pytest
import torch

import synth
from moe_cases import Problem, compare, small_workload, tile_edge_tokens

pytestmark = pytest.mark.gpu

_PROBLEMS = {}


def problem(name, max_tokens):
    key = (name, max_tokens)
    if key not in _PROBLEMS:
        _PROBLEMS.clear()
        torch.cuda.empty_cache()
        _PROBLEMS[key] = Problem(synth.WORKLOADS[name], max_tokens)
    return _PROBLEMS[key]


def _inputs(wl, T):
    x = synth.make_x(wl, T, device="cuda")
    ids, tw = synth.make_routing(wl, T, device="cuda")
    return x, ids, tw


# (workload, T, rows): "all" compares every output row; "tiles" every token that
# owns the first or the last row of some GEMM tile (so every routed expert and
# every tile of the grouped path is reached)
FULL = [
    ("tiny", 16, "all"),
    # decode T=4: contiguous shares; T=8: short deals; T=16 and 32: several rounds
    ("decode", 1, "all"), ("decode", 4, "all"), ("decode", 8, "all"), ("decode", 16, "all"),
    ("decode", 32, "all"),
    ("mixed", 1, "all"), ("mixed", 64, "all"), ("mixed", 512, "all"), ("mixed", 2048, "tiles"),
    ("prefill", 4096, "tiles"),
    ("skew", 8192, "tiles"),
]


@pytest.mark.parametrize("name,T,rows", FULL)
def test_workload_parity(name, T, rows):
    print(f"parity {name} T={T} rows={rows}", flush=True)
    wl = synth.WORKLOADS[name]
    pr = problem(name, max(wl.tokens))
    x, ids, tw = _inputs(wl, T)
    out, b = pr.run(x, ids, tw)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    sel = None
    if rows == "tiles":
        import fp8_moe_amd as fm
        assert fm.binding_query(b, "path") == 1
        sel, n_tiles = tile_edge_tokens(pr.model, wl.k)
        print(f"  {len(sel)} tokens cover both ends of {n_tiles} tiles", flush=True)
    ref = pr.oracle(x, ids, tw, sel)
    got = out if sel is None else out[sel]
    rel_fro, rel_max, ok = compare(got, ref)
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    assert ok, (rel_fro, rel_max)


@pytest.mark.parametrize("afmt", ["mxfp8", "nvfp4"])
def test_prefill_layer_quantized_activations(afmt):
    """The prefill layer's NVFP4 experts (E=128, H=4096, I=1536, top-8,
    T=4096) with MXFP8 or NVFP4 activations, the shapes the benchmark times:
    every token owning an end of a GEMM tile against the oracle."""
    import dataclasses
    import fp8_moe_amd as fm
    print(f"prefill layer x {afmt}", flush=True)
    wl = dataclasses.replace(synth.WORKLOADS["prefill"], act_format=afmt)
    _PROBLEMS.clear()
    torch.cuda.empty_cache()
    pr = Problem(wl, 4096)
    x, ids, tw = _inputs(wl, 4096)
    out, b = pr.run(x, ids, tw)
    torch.cuda.synchronize()
    assert fm.binding_query(b, "path") == 1
    sel, n_tiles = tile_edge_tokens(pr.model, wl.k)
    print(f"  {len(sel)} tokens cover both ends of {n_tiles} tiles", flush=True)
    ref = pr.oracle(x, ids, tw, sel)
    rel_fro, rel_max, ok = compare(out[sel], ref)
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    del pr
    assert ok, (rel_fro, rel_max)


SMALL = [
    # name, E, H, I, k, gated, wfmt, afmt, T
    ("multi_tile", 2, 256, 128, 1, True, "mxfp4", "bf16", 300),
    ("ragged_k_gated", 4, 160, 96, 2, True, "mxfp4", "bf16", 40),
    ("ragged_k_nv", 4, 160, 96, 2, True, "nvfp4", "bf16", 40),
    ("ragged_k_a8", 4, 160, 96, 2, False, "mxfp4", "mxfp8", 40),
    ("a8_multi_tile", 3, 288, 224, 2, False, "mxfp4", "mxfp8", 400),
    ("nv_relu2", 5, 256, 192, 3, False, "nvfp4", "bf16", 77),
    ("mx_relu2", 5, 256, 192, 3, False, "mxfp4", "bf16", 77),
    ("a8_gated", 6, 256, 128, 2, True, "mxfp4", "mxfp8", 50),
    # NVFP4 weights x MXFP8 activations (bf16 round trips), grouped path
    ("nv_a8_gated", 4, 256, 128, 2, True, "nvfp4", "mxfp8", 200),
    ("nv_a8_relu2_ragged", 5, 160, 96, 3, False, "nvfp4", "mxfp8", 120),
    ("nv_a8_mid", 16, 1024, 512, 4, True, "nvfp4", "mxfp8", 256),
    # NVFP4 weights x NVFP4 activations (W4A4), grouped path
    ("nv_a4_gated", 4, 256, 128, 2, True, "nvfp4", "nvfp4", 200),
    ("nv_a4_relu2_ragged", 5, 160, 96, 3, False, "nvfp4", "nvfp4", 120),
    ("nv_a4_mid", 16, 1024, 512, 4, True, "nvfp4", "nvfp4", 256),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shapes(case):
    name, E, H, I, k, gated, wfmt, afmt, T = case
    print(f"small {case}", flush=True)
    wl = small_workload(name, E, H, I, k, gated, wfmt, afmt, x_lognormal=afmt == "mxfp8")
    pr = Problem(wl, T, gen_device="cpu")
    x, ids, tw = _inputs(wl, T)
    out, _ = pr.run(x, ids, tw)
    torch.cuda.synchronize()
    rel_fro, rel_max, ok = compare(out, pr.oracle(x, ids, tw))
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    assert ok, (rel_fro, rel_max)


def test_bad_and_duplicate_ids_and_strided_io():
    wl = small_workload("edge", 8, 256, 128, 3)
    pr = Problem(wl, 64, gen_device="cpu")
    x, ids, tw = _inputs(wl, 64)
    ids = ids.clone()
    ids[0, 1] = -1
    ids[1, 2] = 8
    ids[2, 0] = 10 ** 6
    ids[3, :] = 5
    ids[4, 1] = ids[4, 0]
    xs = torch.zeros(64, 256 + 40, dtype=torch.bfloat16, device="cuda")
    xs[:, :256] = x
    outs = torch.full((64, 256 + 24), 7.0, dtype=torch.bfloat16, device="cuda")
    pr.run(xs[:, :256], ids, tw, outs[:, :256])
    torch.cuda.synchronize()
    rel_fro, rel_max, ok = compare(outs[:, :256], pr.oracle(x, ids, tw))
    assert ok, (rel_fro, rel_max)
    assert torch.all(outs[:, 256:] == 7.0)           # nothing written past H


def test_zero_tokens_is_a_noop():
    import fp8_moe_amd as fm
    wl = small_workload("empty", 4, 256, 128, 2)
    pr = Problem(wl, 8, gen_device="cpu")
    x = torch.empty(0, 256, dtype=torch.bfloat16, device="cuda")
    ids = torch.empty(0, 2, dtype=torch.int32, device="cuda")
    tw = torch.empty(0, 2, dtype=torch.float32, device="cuda")
    b, out = pr.model.bind(x, ids, tw)
    fm.run(b)
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


def test_capacity_error():
    import fp8_moe_amd as fm
    wl = small_workload("cap", 4, 256, 128, 2)
    pr = Problem(wl, 8, gen_device="cpu")
    x, ids, tw = _inputs(wl, 9)
    with pytest.raises(fm.B12xError) as e:
        pr.model.bind(x, ids, tw)
    assert e.value.status == 3


@pytest.mark.parametrize("name", ["tiny", "mixed"])
def test_deterministic_and_permutation_invariant(name):
    wl = synth.WORKLOADS[name] if name == "tiny" else small_workload("perm", 16, 288, 224, 4, False, "mxfp4",
                                                                      "mxfp8", x_lognormal=True)
    T = 96
    pr = Problem(wl, T, gen_device="cpu")
    x, ids, tw = _inputs(wl, T)
    a, _ = pr.run(x, ids, tw)
    a = a.clone()
    b, _ = pr.run(x, ids, tw)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(5)).cuda()
    c, _ = pr.run(x[perm].contiguous(), ids[perm].contiguous(), tw[perm].contiguous())
    assert torch.equal(a[perm].view(torch.int16), c.view(torch.int16))


@pytest.mark.parametrize("T", [1, 8])
def test_graph_replay_matches_eager(T):
    import fp8_moe_amd as fm
    wl = synth.WORKLOADS["decode"]
    pr = problem("decode", 32)
    x, ids, tw = _inputs(wl, T)
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
    b, _ = pr.model.bind(x, ids, tw, out)
    fm.run(b)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fm.run(b, stream=s)
    for i in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        _ = (x.float() * 2).sum()      # unrelated eager work between replays


@pytest.mark.parametrize("afmt,T", [("nvfp4", 8), ("nvfp4", 20), ("nvfp4", 200), ("mxfp8", 8), ("mxfp8", 20),
                                    ("mxfp8", 200)])
def test_graph_replay_matches_eager_quantized(afmt, T):
    """Graph replay of the paths with activation quantization (NVFP4 weights
    with NVFP4 or MXFP8 activations): split-K decode (T=8), two-phase decode
    (T=20) and grouped (T=200), bit-identical to the eager run on every replay."""
    import fp8_moe_amd as fm
    print(f"graph replay {afmt} T={T}", flush=True)
    wl = small_workload(f"graph_{afmt}", 16, 512, 256, 4, True, "nvfp4", afmt)
    pr = Problem(wl, 256, gen_device="cpu")
    x, ids, tw = _inputs(wl, T)
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
    b, _ = pr.model.bind(x, ids, tw, out)
    assert fm.binding_query(b, "path") == (3 if T * wl.k <= 32 else 2 if T * wl.k <= 256 else 1)
    fm.run(b)
    torch.cuda.synchronize()
    eager = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fm.run(b, stream=s)
    for i in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        _ = (x.float() * 2).sum()      # unrelated eager work between replays
    rel_fro, rel_max, ok = compare(out, pr.oracle(x, ids, tw))
    assert ok, (rel_fro, rel_max)


def test_decode_binding_reused_with_new_inputs():
    """One decode binding run again and again while its inputs change in place
    (x, then the routing): every output matches the oracle for the inputs of
    its own call, in eager runs and in replays of one captured graph.  The
    fused decode kernel's down phase waits for flags tagged with its own
    launch's number, so it never consumes the h rows of an earlier call."""
    import fp8_moe_amd as fm
    wl = synth.WORKLOADS["decode"]
    pr = problem("decode", 32)
    T = 8
    x, ids, tw = _inputs(wl, T)
    b, out = pr.model.bind(x, ids, tw)
    assert fm.binding_query(b, "path") == 2
    variants = []
    for salt in range(1, 4):
        xs = synth.make_x(wl, T, device="cuda", salt=100 + salt)
        ids_s, tw_s = synth.make_routing(wl, T, device="cuda", salt=100 + salt)
        variants.append((xs, ids_s, tw_s))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fm.run(b, stream=s)
    for i, (xs, ids_s, tw_s) in enumerate(variants * 2):
        x.copy_(xs)
        ids.copy_(ids_s)
        tw.copy_(tw_s)
        out.fill_(0)
        torch.cuda.synchronize()
        if i < len(variants):
            fm.run(b)
        else:
            g.replay()
        torch.cuda.synchronize()
        rel_fro, rel_max, ok = compare(out, pr.oracle(x, ids, tw))
        assert ok, (i, rel_fro, rel_max)


def test_fused_decode_stage_run_twice_with_new_inputs():
    """The fused decode kernel run twice without the combine in between (a
    stage-by-stage caller), the inputs changed between the two: every launch
    tags its flags with a tag of its own, so the second launch's down phase
    waits for its own gate/up results, and the combine gives the oracle's
    output for the second inputs."""
    import fp8_moe_amd as fm
    wl = synth.WORKLOADS["decode"]
    pr = problem("decode", 32)
    T = 8
    x, ids, tw = _inputs(wl, T)
    b, out = pr.model.bind(x, ids, tw)
    assert fm.binding_query(b, "path") == 2 and fm.binding_query(b, "num_stages") == 2
    fm.run(b)
    for salt in (201, 202):
        fm.run_stage(b, "decode1")
        x.copy_(synth.make_x(wl, T, device="cuda", salt=salt))
        ids_s, tw_s = synth.make_routing(wl, T, device="cuda", salt=salt)
        ids.copy_(ids_s)
        tw.copy_(tw_s)
        out.fill_(0)
        fm.run_stage(b, "decode1")
        fm.run_stage(b, "combine")
        torch.cuda.synchronize()
        rel_fro, rel_max, ok = compare(out, pr.oracle(x, ids, tw))
        assert ok, (salt, rel_fro, rel_max)


def test_fused_decode_wait_runs_out_and_computes_the_missing_groups(monkeypatch):
    """The fused decode kernel's bounded wait, forced from the host to run out
    (the test hook makes every wait expect a tag that no flag holds, with a
    few polls; all kernels still run to their end): every down part then
    computes its expert's gate/up groups itself, which is what a workgroup
    does when the groups' producer is not resident.  The output is
    bit-identical to an ordinary call's, eager and replayed from a graph, and
    an ordinary binding over the same scratch is unaffected afterwards."""
    import fp8_moe_amd as fm
    wl = synth.WORKLOADS["decode"]
    pr = problem("decode", 32)
    for T in (8, 32):  # (T = 1 runs the split-K kernel, which has no waits)
        x, ids, tw = _inputs(wl, T)
        good, ref = pr.model.bind(x, ids, tw)
        assert fm.binding_query(good, "path") == 2 and fm.binding_query(good, "num_stages") == 2
        fm.run(good)
        monkeypatch.setenv("B12X_DEBUG_FORCE_GIVEUP", "1")
        forced, out = pr.model.bind(x, ids, tw)
        monkeypatch.delenv("B12X_DEBUG_FORCE_GIVEUP")
        for _ in range(2):
            out.fill_(0)
            fm.run(forced)
            torch.cuda.synchronize()
            assert torch.equal(out, ref), T
        s = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                fm.run(forced, s)
        torch.cuda.synchronize()
        for _ in range(3):
            out.fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref), T
        del g
        again = torch.zeros_like(ref)
        b2, _ = pr.model.bind(x, ids, tw, again)
        fm.run(b2)
        torch.cuda.synchronize()
        assert torch.equal(again, ref), T
        rel_fro, rel_max, ok = compare(ref, pr.oracle(x, ids, tw))
        assert ok, (T, rel_fro, rel_max)


def test_fused_decode_needs_a_primed_scratch():
    """A scratch that b12x_moe_prime never zeroed (filled with 0x01 bytes here:
    its launch counter is not a multiple of the launch step) makes the fused
    decode call write NaN rows, not a result that may be stale.  Primed, the
    same scratch gives the output of a freshly allocated one, bit for bit."""
    import fp8_moe_amd as fm
    wl = synth.WORKLOADS["decode"]
    pr = problem("decode", 32)
    T = 8
    x, ids, tw = _inputs(wl, T)
    ref_b, ref_out = pr.model.bind(x, ids, tw)
    fm.run(ref_b)
    raw = torch.full_like(pr.model.scratch, 1)
    out = torch.zeros_like(ref_out)
    b = fm.bind(pr.model.plan, raw, pr.model.experts, x, ids, tw, out)
    assert fm.binding_query(b, "path") == 2 and fm.binding_query(b, "num_stages") == 2
    fm.run(b)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    fm.prime(pr.model.plan, raw)
    for _ in range(2):
        out.fill_(0)
        fm.run(b)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)


# decode path (T*k <= 256) against the grouped path and the oracle on the same inputs
DECODE = [
    ("tiny", 16), ("decode", 1), ("decode", 8), ("decode", 32), ("mixed", 1), ("mixed", 64),
]


@pytest.mark.parametrize("name,T", DECODE)
def test_decode_and_grouped_paths_agree(name, T):
    import fp8_moe_amd as fm
    print(f"paths {name} T={T}", flush=True)
    wl = synth.WORKLOADS[name]
    pr = problem(name, max(wl.tokens))
    grouped = fm.FusedMoE(wl.E, wl.H, wl.I, wl.k, wl.weight_format, wl.act_format,
                          "silu" if wl.gated else "relu2", T, pr.wd, decode_max_pairs=-1)
    x, ids, tw = _inputs(wl, T)
    b_dec, out_dec = pr.model.bind(x, ids, tw)
    b_grp, out_grp = grouped.bind(x, ids, tw)
    assert fm.binding_query(b_dec, "path") in (2, 3) and fm.binding_query(b_grp, "path") == 1
    fm.run(b_dec)
    fm.run(b_grp)
    torch.cuda.synchronize()
    rows = None
    ref = pr.oracle(x, ids, tw, rows)
    for out in (out_dec, out_grp):
        got = out if rows is None else out[rows]
        rel_fro, rel_max, ok = compare(got, ref)
        assert ok, (rel_fro, rel_max)
    d = (out_dec.float() - out_grp.float()).abs().max().item()
    assert d <= 2e-2 * out_grp.float().abs().max().item()


DECODE_EDGE = [
    # name, E, H, I, k, gated, wfmt, afmt, T, ids kind
    ("one_expert_many_rows", 8, 256, 128, 8, True, "mxfp4", "bf16", 32, "one_expert"),
    ("all_dropped", 8, 256, 128, 2, True, "mxfp4", "bf16", 5, "all_bad"),
    ("some_dropped_dups", 16, 256, 128, 4, True, "nvfp4", "bf16", 20, "bad_dups"),
    ("a8_one_expert", 8, 288, 224, 4, False, "mxfp4", "mxfp8", 40, "one_expert"),
    ("a8_gated", 8, 256, 128, 2, True, "mxfp4", "mxfp8", 30, "uniform"),
    ("nv_relu2_ragged", 8, 160, 96, 3, False, "nvfp4", "bf16", 50, "uniform"),
    ("k1", 4, 256, 128, 1, True, "mxfp4", "bf16", 1, "uniform"),
    # bf16 shapes outside the fused gate/up + down kernel: 5 K fragments per wave,
    # and 68 gate/up groups per expert
    ("nv_a8_gated_decode", 8, 256, 128, 2, True, "nvfp4", "mxfp8", 10, "uniform"),
    ("nv_a8_relu2_decode", 8, 288, 224, 4, False, "nvfp4", "mxfp8", 30, "one_expert"),
    ("nv_a4_gated_decode", 8, 256, 128, 2, True, "nvfp4", "nvfp4", 10, "uniform"),
    ("nv_a4_relu2_decode", 8, 288, 224, 4, False, "nvfp4", "nvfp4", 30, "one_expert"),
    ("nv_a4_dups_dropped", 16, 256, 128, 4, True, "nvfp4", "nvfp4", 20, "bad_dups"),
    ("separate_long_k", 8, 2304, 128, 2, True, "mxfp4", "bf16", 6, "uniform"),
    ("separate_many_groups", 8, 256, 1088, 2, True, "nvfp4", "bf16", 5, "uniform"),
    # split-K decode (T*k <= 32): two 16-row blocks of one expert, ragged K, every
    # activation format, K fragments in two rounds per wave, dropped and duplicate ids
    ("sk_one_expert_two_blocks", 8, 256, 128, 8, True, "mxfp4", "bf16", 4, "one_expert"),
    ("sk_ragged_k", 8, 160, 96, 3, False, "nvfp4", "bf16", 8, "uniform"),
    ("sk_a8_relu2", 8, 288, 224, 4, False, "mxfp4", "mxfp8", 6, "uniform"),
    ("sk_a8_gated_dups", 8, 256, 128, 4, True, "mxfp4", "mxfp8", 8, "bad_dups"),
    ("sk_nv_a8", 8, 256, 128, 2, True, "nvfp4", "mxfp8", 10, "uniform"),
    ("sk_nv_a4_relu2", 8, 288, 224, 4, False, "nvfp4", "nvfp4", 8, "one_expert"),
    ("sk_long_k", 8, 2304, 128, 2, True, "mxfp4", "bf16", 6, "uniform"),
    ("sk_k1", 4, 256, 128, 1, True, "nvfp4", "bf16", 1, "uniform"),
]


@pytest.mark.parametrize("splitk", [True, False], ids=["splitk", "two_phase"])
@pytest.mark.parametrize("case", DECODE_EDGE, ids=[c[0] for c in DECODE_EDGE])
def test_decode_edge_cases(case, splitk):
    import fp8_moe_amd as fm
    name, E, H, I, k, gated, wfmt, afmt, T, kind = case
    print(f"decode edge {case} splitk={splitk}", flush=True)
    wl = small_workload(name, E, H, I, k, gated, wfmt, afmt, x_lognormal=afmt == "mxfp8")
    pr = Problem(wl, T, gen_device="cpu", splitk_max_pairs=0 if splitk else -1)
    x, ids, tw = _inputs(wl, T)
    ids = ids.clone()
    if kind == "one_expert":
        ids[:] = E - 1
    elif kind == "all_bad":
        ids[:] = -1
        ids[0, 0] = E
    elif kind == "bad_dups":
        ids[0, 1] = -5
        ids[1, :] = 3
        ids[2, 2] = E + 7
    b, out = pr.model.bind(x, ids, tw)
    sk = splitk and T * k <= 32 and H <= 4096
    assert fm.binding_query(b, "path") == (3 if sk else 2)
    fused = afmt == "bf16" and not name.startswith("separate") and not name.startswith("sk_long")
    expect_stages = 2 if sk else (2 if fused else 3 + (afmt != "bf16"))
    assert fm.binding_query(b, "num_stages") == expect_stages
    out.fill_(1.0)
    fm.run(b)
    torch.cuda.synchronize()
    ref = pr.oracle(x, ids, tw)
    rel_fro, rel_max, ok = compare(out, ref)
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    assert ok, (rel_fro, rel_max)
    if kind == "all_bad":
        assert torch.all(out == 0)


@pytest.mark.parametrize("T,rows", [(8, None), (32, None)])
def test_w4a4_at_prefill_shape(T, rows):
    """NVFP4 activations on the prefill layer's NVFP4 weights (E=128, H=4096,
    I=1536, top-8) on the decode path, every row (T=4096 is covered with the
    MXFP8 activations in test_prefill_layer_quantized_activations)."""
    import dataclasses
    print(f"w4a4 prefill shape T={T} rows={rows}", flush=True)
    wl = dataclasses.replace(synth.WORKLOADS["prefill"], act_format="nvfp4")
    _PROBLEMS.clear()
    torch.cuda.empty_cache()
    pr = Problem(wl, 4096)
    x, ids, tw = _inputs(wl, T)
    out, b = pr.run(x, ids, tw)
    torch.cuda.synchronize()
    import fp8_moe_amd as fm
    assert fm.binding_query(b, "path") == (2 if T * wl.k <= 256 else 1)
    ref = pr.oracle(x, ids, tw, rows)
    got = out if rows is None else out[rows]
    rel_fro, rel_max, ok = compare(got, ref)
    print(f"  rel_fro={rel_fro:.3e} rel_max={rel_max:.3e}", flush=True)
    del pr
    assert ok, (rel_fro, rel_max)


def test_nvfp4_rows_of_extreme_magnitude():
    """NVFP4 x bf16 on the grouped path: rows scaled far up and down, a zero
    row and a row mixing large and tiny values, compared row by row (each row
    on its own scale) with the fp64 oracle.  (The per-tensor NVFP4 scale
    multiplies the fp32 accumulators, so intermediates must stay finite
    before it: row scales up to 2^40 here.)"""
    import fp8_moe_amd as fm
    wl = small_workload("nv_range", 4, 256, 128, 2, True, "nvfp4", "bf16")
    T = 40
    pr = Problem(wl, T, gen_device="cpu", decode_max_pairs=-1)
    x, ids, tw = _inputs(wl, T)
    scale = torch.ones(T, 1, dtype=torch.float32)
    scale[0], scale[1], scale[2], scale[3] = 2.0 ** 40, 2.0 ** -50, 2.0 ** 25, 2.0 ** -30
    xs = (x.float().cpu() * scale)
    xs[4] = 0.0
    xs[5, ::2] *= 2.0 ** -40                     # half the row 2^40 smaller than the rest
    x = xs.to(torch.bfloat16).cuda()
    b, out = pr.model.bind(x, ids, tw)
    assert fm.binding_query(b, "path") == 1
    fm.run(b)
    torch.cuda.synchronize()
    ref = pr.oracle(x, ids, tw)
    got = out.detach().cpu().to(torch.float64).numpy()
    assert np.all(np.isfinite(got))
    assert np.all(got[4] == 0.0)
    for t in range(T):
        if t == 4:
            continue
        n = np.linalg.norm(ref[t])
        assert n > 0, t
        rel = np.linalg.norm(got[t] - ref[t]) / n
        assert rel <= 5e-3, (t, rel)
