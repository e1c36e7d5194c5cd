"""The allocation-free call b12x_moe_run_noalloc (for callers that cannot
allocate device memory): on the GPU its output is bit-identical to
b12x_moe_bind + b12x_moe_run on the same inputs, over two calls in a row on
the library's static scratch, the second with a smaller batch; on the host,
its refusals (wrong path, partial rows beyond the static array)."""
import ctypes

import pytest
import torch


def _noalloc_status(p, ex, T, a_stride, a_ptr=0x10000, out_ptr=0x9000000, ids_ptr=0x200000, tw_ptr=0x300000):
    import fp8_moe_amd as fm
    return fm.lib().b12x_moe_run_noalloc(p.handle, ctypes.byref(ex), ctypes.c_void_p(a_ptr), T, a_stride,
                                         ctypes.c_void_p(ids_ptr), ctypes.c_void_p(tw_ptr),
                                         ctypes.c_void_p(out_ptr), a_stride, None)


def test_noalloc_refusals_on_host():
    # every refusal below is decided before any HIP call
    import fp8_moe_amd as fm
    wp = fm.plan_weights(128, 2048, 768, True, "mxfp4")
    ex = fm.Experts(wp, ctypes.c_void_p(0x7000000), wp.prepared_bytes)
    p = fm.plan(wp, 8, 64)
    assert _noalloc_status(p, ex, 5, 2048) == 2                  # 40 pairs: not the split-K path
    assert _noalloc_status(p, ex, 65, 2048) == 3                 # beyond max_tokens
    assert _noalloc_status(p, ex, 4, 2048, a_ptr=0x10008) == 5   # misaligned a
    assert _noalloc_status(p, ex, 0, 2048, a_ptr=0, out_ptr=0, ids_ptr=0, tw_ptr=0) == 0   # T = 0: no work
    big = fm.plan_weights(8, 4096, 4096, True, "mxfp4")          # 4 MB of partial rows per pair... x 8
    exb = fm.Experts(big, ctypes.c_void_p(0x7000000), big.prepared_bytes)
    pb = fm.plan(big, 8, 4)
    need = 8 * (4096 // 32) * ((4096 // 16 + 3) // 4 * 64 + 64) * 4
    assert need > fm.NOALLOC_SCRATCH_BYTES
    assert _noalloc_status(pb, exb, 1, 4096) == 3                # partial rows beyond the static array


CASES = [("tiny", "silu", (16, 5)), ("decode", "silu", (4, 1)), ("mixed", "relu2", (3, 1)),
         ("decode", "swiglu_oai", (4, 1))]


@pytest.mark.gpu
@pytest.mark.parametrize("name,act,Ts", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_noalloc_matches_bind_run(name, act, Ts):
    import fp8_moe_amd as fm
    import synth
    wl = synth.WORKLOADS[name]
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    ex = fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"],
                            w["w13_global"], w["w2_global"])
    del w
    plan = fm.plan(wp, wl.k, max(Ts), wl.act_format, act)
    scratch = fm.alloc_scratch(plan)
    for i, T in enumerate(Ts):
        print(f"noalloc case {name} T={T}", flush=True)
        x = synth.make_x(wl, T, device="cuda", salt=i)
        ids, tw = synth.make_routing(wl, T, device="cuda", salt=i)
        ref = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
        b = fm.bind(plan, scratch, ex, x, ids, tw, ref)
        assert fm.binding_query(b, "path") == 3
        fm.run(b)
        out = torch.full((T, wl.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        fm.run_noalloc(plan, ex, x, ids, tw, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"{name} T={T}"
        assert torch.isfinite(out.float()).all()
