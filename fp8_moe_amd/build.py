"""Build ``libb12x_moe.so`` (all HIP kernels + the C ABI) and the benchmark
harness's ``libb12x_probes.so`` (measurement probes) for gfx950 in-tree.

Usage: ``python fp8_moe_amd/build.py`` (or ``build()`` from Python).  Always
recompiles every source; objects go to ``fp8_moe_amd/_build/``.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libb12x_moe.so")
PROBES_OUT = os.path.join(HERE, "libb12x_probes.so")
BUILD = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["gemm_inst_silu_f16.hip", "gemm_inst_relu2_f16.hip", "gemm_inst_silu.hip", "gemm_inst_relu2.hip",
           "gemm_inst_down.hip", "decode.hip", "decode_sk.hip", "api.cpp", "pack.hip", "route.hip", "quant.hip", "gemm.hip",
           "combine.hip", "debug.hip"]
PROBE_SOURCES = ["probes.hip"]

# -packed-fp32-ops: keep hipcc from emitting packed fp32 VALU ops.
# -pragma-unroll-threshold: loops marked `#pragma unroll` are unrolled whatever
# their size.  Under LLVM's default limit the grouped GEMM's W4A4 epilogue (the
# exact NVFP4 requantization of h, once per element of the tile) stayed a loop,
# which indexed the accumulator array at run time and moved it to scratch
# memory, inside the K loop too.
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-pragma-unroll-threshold=1000000",
         "-I" + os.path.join(os.path.dirname(HERE), "include")]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    return obj, errs


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    sources = SOURCES + PROBE_SOURCES
    jobs = min(len(sources), max(1, int(os.environ.get("MAX_JOBS", str(os.cpu_count() or 8)))))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = dict(zip(sources, ex.map(_compile, sources)))
    for _, errs in results.values():
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], OUT)
    _link([results[s][0] for s in PROBE_SOURCES], PROBES_OUT)
    return OUT


# Host-sanitized variant of the MoE library for the CPU sanitizer run: api.cpp (the
# host runtime: planning, validation, binding, dispatch) built with AddressSanitizer
# and UndefinedBehaviorSanitizer on its host pass only, linked with the ordinary
# kernel objects of build().  Load it with the sanitizer runtime preloaded
# (HOSTSAN_RUNTIME) and B12X_MOE_LIB pointing at it.
HOSTSAN_OUT = os.path.join(BUILD, "libb12x_moe_hostsan.so")
HOSTSAN_RUNTIME = "/opt/rocm/llvm/lib/clang/{}/lib/linux/libclang_rt.asan-x86_64.so"


def hostsan_runtime():
    base = "/opt/rocm/llvm/lib/clang"
    for v in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
        path = HOSTSAN_RUNTIME.format(v)
        if os.path.exists(path):
            return path
    return None


def build_hostsan():
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: {missing[0]} is missing")
    api_o = os.path.join(BUILD, "api.cpp.hostsan.o")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g"]
    res = subprocess.run([HIPCC, "-x", "hip", *flags, *san, "-c", os.path.join(CSRC, "api.cpp"), "-o", api_o],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for api.cpp (host-sanitized):\n" + res.stderr)
    tmp = HOSTSAN_OUT + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan", *san, api_o, *objs,
                          "-o", tmp], capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed (host-sanitized):\n" + res.stderr)
    os.replace(tmp, HOSTSAN_OUT)
    return HOSTSAN_OUT


if __name__ == "__main__":
    print(build(verbose=True))
    if len(sys.argv) > 1 and sys.argv[1] == "--hostsan":
        print(build_hostsan())
