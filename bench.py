"""Benchmark of the fused block-scaled-FP4 MoE on one MI355X.

Headline workload: decode, MXFP4 weights x BF16 activations (W4A16),
E=128, H=2048, I=768, top_k=8, SiLU-gated, one batch each of T = 1, 8 and 32
tokens per step.  Metric: weight GB/s = touched-expert weight bytes (packed
FP4 codes + block scales of every expert the batch routes to) / time.

Method: C prepared copies of the weights (more than the 256 MB Infinity
Cache holds) and S input sets rotate, so each call streams cold weights;
S steps are captured in one graph and replayed (no host launch overhead in
the timed region); timing with events around K steps after W warmup steps.
The dominant kernel (the decode path's fused gate/up + down kernel) is also
timed for the roofline object, in the sequence it runs in: graphs of (fused
kernel, combine) less graphs of the combines alone; its HBM traffic comes from
the committed counter record in profiles/ when that record matches the kernel
sources.  Extra lines report
prefill (NVFP4, T=4096) TFLOP/s with bf16, MXFP8 and NVFP4 activations, the
dense block-scaled GEMM (4096^3), and under "configs" every configuration
(tiny T=16, decode T=1/8/32, mixed MXFP4 x MXFP8 ReLU^2 T=1/64/512/2048,
prefill T=4096, large skewed T=8192): time per call, its roofline fraction
(HBM on touched-expert weight bytes, or the bf16 MFMA peak), and the CPU
oracle timed on a bounded sample of the same inputs.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
       python bench.py --decode-t T [--steps K]   (one T only, for counter and trace runs)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
N_WEIGHT_COPIES = 5            # 5 x 323 MB > 256 MB Infinity Cache
N_SETS = 10                    # input sets per graph (also the steps per replay)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---- measurement probes (libb12x_probes.so, include/b12x_probes.h): the achieved
# ceilings that the MoE kernels' rates are read against
class ProbeError(RuntimeError):
    pass


_PROBES = None


def _probes():
    global _PROBES
    if _PROBES is None:
        import ctypes
        path = os.path.join(ROOT, "fp8_moe_amd", "libb12x_probes.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built; run `python fp8_moe_amd/build.py`")
        lib = ctypes.CDLL(path)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.b12x_probe_stream_read.restype = i32
        lib.b12x_probe_stream_read.argtypes = [vp, ctypes.c_uint64, vp, i32, vp]
        lib.b12x_probe_mfma.restype = i32
        lib.b12x_probe_mfma.argtypes = [vp, i32, i32, i32, vp]
        _PROBES = lib
    return _PROBES


def _probe_stream(stream):
    import ctypes
    import torch
    return ctypes.c_void_p((stream if stream is not None else torch.cuda.current_stream()).cuda_stream)


def probe_stream_read(src, sink, workgroups, stream=None):
    """Stream `src` (contiguous device tensor, a multiple of 16 bytes) through
    `workgroups` workgroups; sink: 32-bit tensor of workgroups * 256 elements."""
    import ctypes
    if sink.numel() < workgroups * 256:
        raise ValueError("sink needs workgroups*256 elements")
    st = _probes().b12x_probe_stream_read(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                          ctypes.c_void_p(sink.data_ptr()), workgroups, _probe_stream(stream))
    if st:
        raise ProbeError(f"stream-read probe: status {st}")


def probe_mfma(sink, workgroups, iterations, f16=False, stream=None):
    """16 * iterations 16x16x32 MFMAs per wave, four waves per workgroup; sink:
    float32 tensor of workgroups * 256 elements."""
    import ctypes
    import torch
    if sink.dtype != torch.float32 or sink.numel() < workgroups * 256:
        raise ValueError("sink must be float32 with workgroups*256 elements")
    st = _probes().b12x_probe_mfma(ctypes.c_void_p(sink.data_ptr()), workgroups, iterations, int(bool(f16)),
                                   _probe_stream(stream))
    if st:
        raise ProbeError(f"MFMA probe: status {st}")


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def touched_experts(ids, E):
    ids = ids.reshape(-1).tolist()
    return len({e for e in ids if 0 <= e < E})


def build_decode(fm, synth, torch, only_t=None):
    wl = synth.WORKLOADS["decode"]
    Ts = wl.tokens
    if only_t is not None and only_t not in Ts:
        raise SystemExit(f"--decode-t must be one of {Ts}")
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    copies = [fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"])
              for _ in range(N_WEIGHT_COPIES)]
    plan = fm.plan(wp, wl.k, max(Ts), wl.act_format, "silu")
    scratch = fm.alloc_scratch(plan)
    per_expert = wl.weight_bytes_per_expert()
    w13_per_expert = wl.n13 * wl.H // 2 + wl.n13 * wl.H // wl.group
    sets = {}
    for T in Ts:
        if only_t is not None and T != only_t:
            continue
        rows = []
        for s in range(N_SETS):
            x = synth.make_x(wl, T, device="cuda", salt=s)
            ids, tw = synth.make_routing(wl, T, device="cuda", salt=s)
            out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
            copy = copies[(s * len(Ts) + Ts.index(T)) % N_WEIGHT_COPIES]   # reuse distance: 5 calls
            b = fm.bind(plan, scratch, copy, x, ids, tw, out)
            n_e = touched_experts(ids.cpu(), wl.E)
            rows.append(dict(x=x, ids=ids, tw=tw, out=out, binding=b, experts=n_e, bytes=n_e * per_expert,
                             w13_bytes=n_e * w13_per_expert))
        sets[T] = rows
    return wl, w, plan, scratch, copies, sets


def bench_decode_t(fm, synth, torch, stream, T, reps):
    """The decode workload at one T: the 10 input sets of the headline step (rotating
    weight copies) captured in one graph and replayed `reps` times."""
    wl, _, _, _, _, sets = build_decode(fm, synth, torch, only_t=T)
    bl = [row["binding"] for row in sets[T]]
    for b in bl:
        fm.run(b, stream=stream)
    g = capture(torch, fm, bl, stream)
    g.replay()
    sec = time_graph(torch, g, stream, reps) / (reps * len(bl))
    nb = sum(row["bytes"] for row in sets[T]) / len(bl)
    kind, d, extra = time_decode_kernel(torch, fm, bl, stream)
    return {"decode_T": T, "calls": reps * len(bl), "us_per_call": sec * 1e6, "weight_GBs": nb / sec / 1e9,
            "w13_bytes_per_call": sum(row["w13_bytes"] for row in sets[T]) / len(bl),
            "kernel": kind, "kernel_launch_us": round(d * 1e6, 3), **extra}


def capture(torch, fm, bindings, stream):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for b in bindings:
            fm.run(b, stream=stream)
    return g


def time_graph(torch, g, stream, reps):
    e0, e1 = _events()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3  # seconds


def time_graph_samples(torch, g, stream, reps):
    """Per-replay durations (s) of `reps` back-to-back replays, from one event
    recorded between consecutive replays."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        ev[0].record(stream)
        for i in range(reps):
            g.replay()
            ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) / 1e3 for i in range(reps)]


def percentile(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def measure_ceilings(fm, torch, stream):
    """Achieved ceilings of this device: the best rate of a plain streaming read
    of 1 GiB (over a few grid sizes) and the sustained rate of an MFMA register
    loop (bf16 and f16, two workgroups of four waves per CU)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    best = 0.0
    for per_cu in (4, 8, 16):
        wg = cus * per_cu
        sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
        per = (nbytes // 16) // wg
        read = wg * (per // 1024) * 1024 * 16
        for _ in range(2):
            probe_stream_read(src, sink, wg, stream=stream)
        e0, e1 = _events()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(10):
                probe_stream_read(src, sink, wg, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, read * 10 / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del src
    out = {"stream_read_GBs": round(best, 1)}
    wg, iters = cus * 2, 4000
    sink = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    for name, f16 in (("mfma_bf16_TFLOPs", False), ("mfma_f16_TFLOPs", True)):
        probe_mfma(sink, wg, 10, f16=f16, stream=stream)
        e0, e1 = _events()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(3):
                probe_mfma(sink, wg, iters, f16=f16, stream=stream)
            e1.record(stream)
        torch.cuda.synchronize()
        flops = 3.0 * wg * 4 * 16 * 16384 * iters
        out[name] = round(flops / (e0.elapsed_time(e1) / 1e3) / 1e12, 1)
    return out


def measure_sized_reads(fm, torch, stream, sizes):
    """What a plain streaming read achieves at the decode kernel's own sizes:
    for each name -> bytes, a graph of 10 probe launches that each read a
    different slice of a 1 GiB buffer (so consecutive launches find nothing in
    the caches, like the decode bench's rotating weight copies), timed like the
    kernel (graph replays between two events, divided per launch).  The probe's
    workgroups read whole 16 KB chunks, so each launch reads the largest such
    multiple not above the size; the best of a few grid sizes is kept."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    total = 1 << 30
    src = torch.ones(total // 4, dtype=torch.int32, device="cuda")
    out = {}
    for name, size in sizes.items():
        best = None
        for per_cu in (1, 2, 3, 4):
            wg = cus * per_cu
            chunks = int(size) // (wg * 16384)
            if chunks == 0:
                continue
            read = wg * chunks * 16384
            n_slices = max(1, total // read)
            sink = torch.empty(wg * 256, dtype=torch.int32, device="cuda")
            views = [src[(i % n_slices) * read // 4:(i % n_slices + 1) * read // 4] for i in range(10)]
            for v in views[:2]:
                probe_stream_read(v, sink, wg, stream=stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for v in views:
                    probe_stream_read(v, sink, wg, stream=stream)
            g.replay()
            sec = time_graph(torch, g, stream, 20) / (20 * len(views))
            rate = read / sec / 1e9
            if best is None or rate > best["GBs"]:
                best = {"bytes": read, "us": round(sec * 1e6, 3), "GBs": round(rate, 1), "workgroups": wg}
        out[name] = best
    del src
    return out


def time_stage_graph(torch, fm, bindings, stages, stream, reps=10):
    """Mean duration (s) per binding of the given stages' kernels: a graph of
    those stages for every binding, replayed `reps` times between two events
    on `stream`.  Every binding ran in full beforehand (inputs of any stage
    are in place)."""
    for b in bindings:
        fm.run(b, stream=stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for b in bindings:
            for stage in stages:
                fm.run_stage(b, stage, stream=stream)
    g.replay()
    return time_graph(torch, g, stream, reps) / (reps * len(bindings))


def time_decode_kernel(torch, fm, bl, stream):
    """The decode path's main kernel and its mean launch duration (s) over the
    bindings `bl` (one T): (kind, seconds, per-T fields).

    The split-K kernel and the fused gate/up + down kernel are timed alone:
    a graph of that one kernel for every binding (each fused launch has a tag
    of its own, so every launch waits for its own gate/up groups).  Without
    either (unfused decode or grouped path) the gate/up kernel alone."""
    path = fm.binding_query(bl[0], "path")
    fused = path == 2 and fm.binding_query(bl[0], "num_stages") == 2
    extra = {"path": {3: "decode, split-K", 2: "decode, fused" if fused else "decode"}.get(path, "grouped")}
    if path == 3 or fused:
        d = time_stage_graph(torch, fm, bl, ["decode1"], stream)
        extra["decode_kernel_us"] = d * 1e6
        return ("splitk" if path == 3 else "fused"), d, extra
    st1, st2 = ("decode1", "decode2") if path == 2 else ("gemm1", "gemm2")
    d = time_stage_graph(torch, fm, bl, [st1], stream)
    extra["gate_up_kernel_us"] = d * 1e6
    extra["down_kernel_us"] = time_stage_graph(torch, fm, bl, [st2], stream) * 1e6
    return "gate_up", d, extra


def time_stage_launches(torch, fm, bindings, stage, stream, repeats=3):
    """Mean duration (s) of one stage's kernel, event pair around each launch.
    The stages before it ran for every binding beforehand (valid routing)."""
    for b in bindings:
        fm.run(b, stream=stream)
    pairs = []
    with torch.cuda.stream(stream):
        for _ in range(repeats):
            for b in bindings:
                e0, e1 = _events()
                e0.record(stream)
                fm.run_stage(b, stage, stream=stream)
                e1.record(stream)
                pairs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / len(pairs) / 1e3


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
TRAFFIC_SOURCES = ["fp8_moe_amd/csrc/decode.hip", "fp8_moe_amd/csrc/decode_common.h",
                   "fp8_moe_amd/csrc/device_common.h", "fp8_moe_amd/csrc/internal.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` (its name up to the template arguments) from the
    committed counter record (FETCH_SIZE and WRITE_SIZE, calibrated on a plain copy
    kernel), or None when the record is missing, is for another kernel or was taken on
    different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    if rec.get("kernel", "").split("<")[0] != kernel.split("<")[0]:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, w_host, sets_host, budget_s=12.0):
    """The fp64 oracle on the host: decode T=1 calls until ~budget_s seconds."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import Weights, fused_moe
    cores = len(os.sched_getaffinity(0))
    weights = Weights(wl.weight_format, wl.gated, **w_host)
    done_bytes, calls = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=cores):
        while True:
            xb, ids, tw, nbytes = sets_host[calls % len(sets_host)]
            fused_moe(xb, ids, tw, weights, act_format=wl.act_format)
            done_bytes += nbytes
            calls += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    dt = time.perf_counter() - t0
    flops_per_call = 6.0 * wl.H * wl.I * 1 * wl.k  # T = 1
    return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "tokens_per_s": calls / dt, "gflops": flops_per_call * calls / dt / 1e9,
            "sample": f"{calls} decode T=1 calls (E=128, H=2048, I=768, top_k=8, MXFP4 W4A16), "
                      f"{dt:.1f} s; weight bytes of touched experts / wall time; BLAS limited to {cores} threads, "
                      f"elementwise NumPy single-threaded",
            "seconds_per_call": dt / calls}


def bench_prefill(fm, synth, torch, stream, reps=20, act_format=None):
    wl = synth.WORKLOADS["prefill"]
    if act_format is not None:  # the same experts with another activation format
        import dataclasses
        wl = dataclasses.replace(wl, act_format=act_format)
    T = wl.tokens[0]
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    ex = fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"],
                            w["w13_global"], w["w2_global"], a13_global=w.get("a13_global"),
                            a2_global=w.get("a2_global"))
    del w
    plan = fm.plan(wp, wl.k, T, wl.act_format, "silu")
    scratch = fm.alloc_scratch(plan)
    x = synth.make_x(wl, T, device="cuda")
    ids, tw = synth.make_routing(wl, T, device="cuda")
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
    b = fm.bind(plan, scratch, ex, x, ids, tw, out)
    for _ in range(2):
        fm.run(b, stream=stream)
    g = capture(torch, fm, [b], stream)
    g.replay()
    samples = time_graph_samples(torch, g, stream, reps)
    sec = sum(samples) / reps
    flops = 6.0 * wl.H * wl.I * T * wl.k
    stages = {st: time_stage_launches(torch, fm, [b], st, stream, repeats=3) * 1e6
              for st in ("route", "quant_x", "gemm1", "gemm2", "combine")}
    return {"T": T, "us": sec * 1e6, "us_p10_p50_p90": [round(percentile(samples, q) * 1e6, 1) for q in (0.1, 0.5, 0.9)],
            "runs": reps, "tflops": flops / sec / 1e12,
            "frac_bf16_peak": flops / sec / 1e12 / BF16_PEAK_TFLOPS, "stage_us": stages,
            "gemm1_tflops": 4.0 * wl.H * wl.I * T * wl.k / (stages["gemm1"] * 1e-6) / 1e12,
            "gemm2_tflops": 2.0 * wl.H * wl.I * T * wl.k / (stages["gemm2"] * 1e-6) / 1e12}


def bench_dense_mm(fm, synth, torch, stream, m=4096, n=4096, k=4096, reps=20):
    """Dense block-scaled GEMM (gemm.blockscaled mm) at m x n x k, NVFP4 and MXFP4
    weights, bf16 activations: TFLOP/s over a graph of `reps` calls."""
    res = {"shape": [m, n, k]}
    x = synth.make_dense_x(m, k, seed=0, device="cuda")
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    for fmt in ("nvfp4", "mxfp4"):
        codes, scales, glob = synth.make_dense_weight(n, k, fmt, seed=0, device="cuda")
        wp = fm.gemm_pack_weight(codes, scales, fmt)
        for _ in range(2):
            fm.gemm_mm(x, wp, n, fmt, glob, out=out, stream=stream)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            fm.gemm_mm(x, wp, n, fmt, glob, out=out, stream=stream)
        g.replay()
        samples = time_graph_samples(torch, g, stream, reps)
        sec = sorted(samples)[len(samples) // 2]
        tf = 2.0 * m * n * k / sec / 1e12
        res[fmt] = {"us_p50": round(sec * 1e6, 1), "tflops": round(tf, 1),
                    "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
    return res


def cpu_sample(wl, w_dev, x, ids, tw, max_experts=None, reps=1, seed=0):
    """The fp64 oracle on the host for one call's inputs (device tensors).  With
    max_experts, only the pairs of that many touched experts (a fixed-seed random
    draw) are computed and the time is scaled by touched / sampled experts (the
    oracle's cost is per expert: one dequantization plus the expert's rows).
    Returns seconds per call (median of `reps`) and what was run."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import Weights, fused_moe
    import synth
    import torch
    cores = len(os.sched_getaffinity(0))
    ids_h, tw_h = ids.cpu().numpy(), tw.cpu().numpy()
    touched = sorted({int(e) for e in ids_h.reshape(-1) if 0 <= e < wl.E})
    sample = touched
    if max_experts is not None and len(touched) > max_experts:
        rng = np.random.default_rng(seed)
        sample = sorted(int(e) for e in rng.choice(touched, size=max_experts, replace=False))
    ids_s = np.where(np.isin(ids_h, sample), ids_h, -1).astype(np.int32)
    weights = Weights(wl.weight_format, wl.gated, num_experts=wl.E, **synth.oracle_weights_kwargs(w_dev, sample))
    xb = x.cpu().view(torch.int16).numpy().view(np.uint16)
    times = []
    with threadpool_limits(limits=cores):
        for _ in range(reps):
            t0 = time.perf_counter()
            fused_moe(xb, ids_s, tw_h, weights, act_format=wl.act_format)
            times.append(time.perf_counter() - t0)
    med = sorted(times)[len(times) // 2]
    sec = med * len(touched) / len(sample)
    T = ids_h.shape[0]
    what = (f"T={T}: all {len(touched)} touched experts, median of {reps}" if len(sample) == len(touched) else
            f"T={T}: the pairs of {len(sample)} of {len(touched)} touched experts ({med:.2f} s), "
            f"scaled by {len(touched)}/{len(sample)}")
    return {"seconds_per_call": round(sec, 4), "tokens_per_s": round(T / sec, 2),
            "gflops": round(6.0 * wl.H * wl.I * T * wl.k / sec / 1e9, 3) if wl.gated else
                      round(4.0 * wl.H * wl.I * T * wl.k / sec / 1e9, 3),
            "cores": cores, "kind": "oracle", "sample": what}


def hbm_roofline(nbytes, sec):
    ach = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "scope": "whole call, touched-expert weight bytes"}


def mfma_roofline(flops, sec):
    ach = flops / sec / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / BF16_PEAK_TFLOPS, 4), "scope": "whole call, bf16 dense peak"}


def bench_mixed(fm, synth, torch, stream, reps=20, cpu=True):
    """Mixed batch (MXFP4 weights x MXFP8 activations, ReLU^2, E=128, H=I=2880,
    top_k=4) at each of its batch sizes: time per call over graphs of several
    input sets (two weight copies rotate), HBM roofline on touched-expert bytes."""
    wl = synth.WORKLOADS["mixed"]
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    copies = [fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"])
              for _ in range(2)]   # 2 x 1.13 GB
    res = {}
    for T in wl.tokens:
        plan = fm.plan(wp, wl.k, T, wl.act_format, "relu2")
        scratch = fm.alloc_scratch(plan)
        n_sets = 4 if T <= 64 else 2
        bs, nbytes, nexp = [], 0, 0
        for s in range(n_sets):
            x = synth.make_x(wl, T, device="cuda", salt=s)
            ids, tw = synth.make_routing(wl, T, device="cuda", salt=s)
            out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
            bs.append((fm.bind(plan, scratch, copies[s % 2], x, ids, tw, out), x, ids, tw, out))
            ne = touched_experts(ids.cpu(), wl.E)
            nexp += ne
            nbytes += ne * wl.weight_bytes_per_expert()
        g = capture(torch, fm, [t[0] for t in bs], stream)
        g.replay()
        sec = time_graph(torch, g, stream, reps) / (reps * n_sets)
        path = fm.binding_query(bs[0][0], "path")
        r = {"us": round(sec * 1e6, 3), "touched_experts": nexp / n_sets,
             "path": {3: "decode, split-K", 2: "decode"}.get(path, "grouped"),
             "roofline": hbm_roofline(nbytes / n_sets, sec)}
        if cpu:
            _, x, ids, tw, _ = bs[0]
            r["cpu_baseline"] = cpu_sample(wl, w, x, ids, tw, max_experts=None if T == 1 else 4,
                                           reps=3 if T == 1 else 1)
        res[f"T{T}"] = r
        del bs, g, scratch, plan
    del copies, w
    torch.cuda.empty_cache()
    return res


def bench_gemm_config(fm, synth, torch, stream, name, reps=10, cpu=True):
    """A prefill-sized config (one batch): time per call, bf16 MFMA roofline on the
    FFN FLOPs, stage times, and the oracle on a sample of its experts."""
    wl = synth.WORKLOADS[name]
    T = wl.tokens[0]
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    ex = fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"],
                            w["w13_global"], w["w2_global"])
    plan = fm.plan(wp, wl.k, T, wl.act_format, "silu")
    scratch = fm.alloc_scratch(plan)
    x = synth.make_x(wl, T, device="cuda")
    ids, tw = synth.make_routing(wl, T, device="cuda")
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
    b = fm.bind(plan, scratch, ex, x, ids, tw, out)
    for _ in range(2):
        fm.run(b, stream=stream)
    g = capture(torch, fm, [b], stream)
    g.replay()
    samples = time_graph_samples(torch, g, stream, reps)
    sec = sorted(samples)[len(samples) // 2]
    flops = 6.0 * wl.H * wl.I * T * wl.k
    stages = {st: round(time_stage_launches(torch, fm, [b], st, stream, repeats=2) * 1e6, 1)
              for st in ("route", "quant_x", "gemm1", "gemm2", "combine")}
    r = {"T": T, "us_p50": round(sec * 1e6, 1), "tflops": round(flops / sec / 1e12, 1),
         "roofline": mfma_roofline(flops, sec), "stage_us": stages,
         "weight_GB": round(wl.E * wl.weight_bytes_per_expert() / 1e9, 3)}
    if cpu:
        r["cpu_baseline"] = cpu_sample(wl, w, x, ids, tw, max_experts=4, reps=1)
    del g, b, scratch, plan, ex, w
    torch.cuda.empty_cache()
    return r


def bench_tiny(fm, synth, torch, stream, reps=50, cpu=True):
    """Tiny reference config (E=8, H=256, I=128, top_k=2, T=16): launch-bound, time
    per call over a graph of 10 calls; the oracle: median of 3 calls."""
    wl = synth.WORKLOADS["tiny"]
    T = wl.tokens[0]
    w = synth.make_weights(wl, device="cuda")
    wp = fm.plan_weights(wl.E, wl.H, wl.I, wl.gated, wl.weight_format)
    ex = fm.prepare_weights(wp, w["w13_codes"], w["w13_scales"], w["w2_codes"], w["w2_scales"])
    plan = fm.plan(wp, wl.k, T, wl.act_format, "silu")
    scratch = fm.alloc_scratch(plan)
    x = synth.make_x(wl, T, device="cuda")
    ids, tw = synth.make_routing(wl, T, device="cuda")
    out = torch.empty(T, wl.H, dtype=torch.bfloat16, device="cuda")
    b = fm.bind(plan, scratch, ex, x, ids, tw, out)
    g = capture(torch, fm, [b] * 10, stream)
    g.replay()
    sec = time_graph(torch, g, stream, reps) / (reps * 10)
    r = {"T": T, "us": round(sec * 1e6, 3), "path": {3: "decode, split-K", 2: "decode"}.get(
        fm.binding_query(b, "path"), "grouped"), "note": "launch-bound; correctness config"}
    if cpu:
        r["cpu_baseline"] = cpu_sample(wl, w, x, ids, tw, reps=3)
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the prefill and W4A8 lines")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--prefill-only", action="store_true", help="only the prefill line (kernel tuning)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="five plain 1 GiB device copies (the reference for the HBM byte counters)")
    ap.add_argument("--decode-t", type=int, default=0,
                    help="only the decode workload at this T (one of 1, 8, 32), --steps graph replays of its "
                         "10 input sets (for counter and trace runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the fused MoE here is a "
              f"single-GPU build and a multi-GPU figure is not produced.", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_moe_amd as fm
    import synth
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()

    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill(fm, synth, torch, stream)}))
        return
    if args.copy_calibration:
        # a plain device copy of exactly 1 GiB per dispatch (counter calibration)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "dispatches": 5}))
        return
    if args.decode_t:
        print(json.dumps(bench_decode_t(fm, synth, torch, stream, args.decode_t, max(args.steps, 1))))
        return
    log("building decode workload")
    wl, w, plan, scratch, copies, sets = build_decode(fm, synth, torch)
    Ts = wl.tokens
    # cpu baseline inputs (host copies) before the source weights go
    w_host = synth.oracle_weights_kwargs(w) if not args.no_cpu else None
    sets_host = [(row["x"].cpu().view(torch.int16).numpy().view("uint16"), row["ids"].cpu().numpy(),
                  row["tw"].cpu().numpy(), row["bytes"]) for row in sets[1]]
    del w

    # warm everything once eagerly (first launches, lazy module loads)
    for T in Ts:
        for row in sets[T]:
            fm.run(row["binding"], stream=stream)
    torch.cuda.synchronize()

    # one graph = N_SETS steps (a step = one call at each T); a second graph holds
    # the remainder so that exactly --steps steps are timed
    step_bindings = [sets[T][s]["binding"] for s in range(N_SETS) for T in Ts]
    g_all = capture(torch, fm, step_bindings, stream)

    def run_steps(n):
        full, rem = divmod(n, N_SETS)
        g_rem = capture(torch, fm, step_bindings[:rem * len(Ts)], stream) if rem else None
        e0, e1 = _events()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(full):
                g_all.replay()
            if g_rem is not None:
                g_rem.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3

    log("timing decode steps")
    run_steps(max(args.warmup, 1))
    steps = args.steps
    elapsed = run_steps(steps)
    ms_per_step = elapsed / steps * 1e3
    bytes_per_step = sum(row["bytes"] for T in Ts for row in sets[T]) / N_SETS
    value = bytes_per_step / (ms_per_step / 1e3) / 1e9

    # per-T breakdown (graph of the N_SETS calls at one T)
    per_t = {}
    for T in Ts:
        g = capture(torch, fm, [row["binding"] for row in sets[T]], stream)
        g.replay()
        reps = max(20, steps // N_SETS)  # >= 200 calls
        samples = [t / N_SETS for t in time_graph_samples(torch, g, stream, reps)]
        sec = sum(samples) / reps
        nb = sum(row["bytes"] for row in sets[T]) / N_SETS
        ne = sum(row["experts"] for row in sets[T]) / N_SETS
        per_t[f"T{T}"] = {"us": sec * 1e6, "touched_experts": ne, "weight_MB": nb / 1e6,
                          "weight_GBs": nb / sec / 1e9, "frac_hbm": nb / sec / 1e9 / HBM_PEAK_GBS,
                          "tflops": 6.0 * wl.H * wl.I * T * wl.k / sec / 1e12,
                          "us_p10_p50_p90": [round(percentile(samples, q) * 1e6, 2) for q in (0.1, 0.5, 0.9)],
                          "calls": reps * N_SETS}

    durs, kbytes, kinds = [], [], []
    for T in Ts:
        bl = [row["binding"] for row in sets[T]]
        kind, d, extra = time_decode_kernel(torch, fm, bl, stream)
        nb = sum(row["w13_bytes" if kind == "gate_up" else "bytes"] for row in sets[T]) / N_SETS
        per_t[f"T{T}"].update(extra)
        durs.append(d)
        kbytes.append(nb)
        kinds.append(kind)
        per_t[f"T{T}"]["kernel_GBs"] = round(nb / d / 1e9, 1)
        per_t[f"T{T}"]["kernel_frac_hbm"] = round(nb / d / 1e9 / HBM_PEAK_GBS, 4)
    names = {"fused": "decode_fused_kernel<MXFP4, SILU> (gate/up + down, decode path)",
             "splitk": "decode_sk_kernel<MXFP4, BF16, SILU> (split-K decode)",
             "gate_up": "decode_kernel<MXFP4, BF16, SILU> (gate/up, decode path)"}

    def roofline_of(kind):
        sel = [i for i, k in enumerate(kinds) if k == kind]
        avg_dur = sum(durs[i] for i in sel) / len(sel)
        avg_bytes = sum(kbytes[i] for i in sel) / len(sel)
        ach = avg_bytes / avg_dur / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic(names[kind].split(" ")[0]),
                "kernel": names[kind], "avg_launch_us": round(avg_dur * 1e6, 3),
                "algorithmic_bytes_per_launch": round(avg_bytes),
                "per_T_launch_us": {f"T{Ts[i]}": round(durs[i] * 1e6, 3) for i in sel}}, ach

    # the dominant kernel: the one with the most time per step
    by_kind = {}
    for k, d in zip(kinds, durs):
        by_kind[k] = by_kind.get(k, 0.0) + d
    dominant = max(by_kind, key=by_kind.get)
    roofline, achieved = roofline_of(dominant)
    others = {k: roofline_of(k)[0] for k in by_kind if k != dominant}

    result = {
        "metric": "fused-MoE weight GB/s (decode T=1,8,32; MXFP4 W4A16)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode: MXFP4 W4A16, E=128, H=2048, I=768, top_k=8, SiLU-gated, "
                               "one batch each of T=1, 8, 32 per step, cold weights (5 rotating copies)",
                   "global_batch": sum(Ts), "seq_len": 1, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "other_decode_kernels": others,
        "per_T": per_t,
    }
    log("achieved ceilings")
    ceil = measure_ceilings(fm, torch, stream)
    ceil["decode_kernel_frac_of_stream_read"] = round(achieved / ceil["stream_read_GBs"], 4)
    # the same bytes per launch as the decode kernel at each T, streamed by the probe
    sized = measure_sized_reads(fm, torch, stream, {f"T{T}": b for T, b in zip(Ts, kbytes)})
    for T, d, b in zip(Ts, durs, kbytes):
        r = sized[f"T{T}"]
        if r is not None:
            r["decode_kernel_GBs"] = round(b / d / 1e9, 1)
            r["decode_kernel_frac"] = round(b / d / 1e9 / r["GBs"], 4)
    ceil["stream_read_at_decode_sizes"] = sized
    result["ceilings"] = ceil
    if not args.no_extra:
        log("prefill line")
        result["prefill"] = bench_prefill(fm, synth, torch, stream)
        ceil["prefill_frac_of_mfma_f16"] = round(result["prefill"]["tflops"] / ceil["mfma_f16_TFLOPs"], 4)
        log("prefill line, NVFP4 x MXFP8")
        pa8 = bench_prefill(fm, synth, torch, stream, act_format="mxfp8")
        result["prefill_w4a8_nvfp4"] = {k: pa8[k] for k in ("T", "us", "us_p10_p50_p90", "tflops", "frac_bf16_peak",
                                                            "stage_us")}
        log("prefill line, NVFP4 x NVFP4")
        pa4 = bench_prefill(fm, synth, torch, stream, act_format="nvfp4")
        result["prefill_w4a4_nvfp4"] = {k: pa4[k] for k in ("T", "us", "us_p10_p50_p90", "tflops", "frac_bf16_peak",
                                                            "stage_us")}
        log("dense mm line")
        result["dense_mm"] = bench_dense_mm(fm, synth, torch, stream)
    if not args.no_cpu:
        log("cpu oracle baseline")
        result["cpu_baseline"] = cpu_baseline(wl, w_host, sets_host)
    if not args.no_extra:
        # every configuration: time per call, its roofline fraction, the oracle beside it
        cpu = not args.no_cpu
        configs = {}
        log("config: tiny")
        configs["tiny"] = bench_tiny(fm, synth, torch, stream, cpu=cpu)
        configs["decode"] = {f"T{T}": {"us": round(per_t[f"T{T}"]["us"], 3), "path": per_t[f"T{T}"]["path"],
                                       "roofline": hbm_roofline(per_t[f"T{T}"]["weight_MB"] * 1e6,
                                                                per_t[f"T{T}"]["us"] * 1e-6)} for T in Ts}
        if cpu:
            row = sets[1][0]
            configs["decode"]["T1"]["cpu_baseline"] = {
                **{k: result["cpu_baseline"][k] for k in ("cores", "kind")},
                "seconds_per_call": round(result["cpu_baseline"]["seconds_per_call"], 4),
                "sample": "the decode line's baseline: " + result["cpu_baseline"]["sample"]}
        log("config: mixed")
        configs["mixed"] = bench_mixed(fm, synth, torch, stream, cpu=cpu)
        log("config: prefill")
        configs["prefill"] = bench_gemm_config(fm, synth, torch, stream, "prefill", cpu=cpu)
        log("config: skew")
        configs["skew"] = bench_gemm_config(fm, synth, torch, stream, "skew", reps=5, cpu=cpu)
        result["configs"] = configs
    print(json.dumps(result))


if __name__ == "__main__":
    main()
