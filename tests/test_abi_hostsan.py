"""The host runtime of the C ABI (planning, validation, binding, the
allocation-free call's refusals) under AddressSanitizer and
UndefinedBehaviorSanitizer: api.cpp is rebuilt with both sanitizers on its
host pass and the host-side ABI tests run in a child process against that
library, with the sanitizer runtime preloaded.  Any report fails the child
(UBSan does not recover; ASan aborts on the first error).  CPU only."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("_b12x_build", os.path.join(ROOT, "fp8_moe_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_abi_host_paths_under_asan_and_ubsan():
    b = _build_module()
    runtime = b.hostsan_runtime()
    if runtime is None:
        pytest.skip("no AddressSanitizer runtime in this ROCm toolchain")
    if not all(os.path.exists(os.path.join(b.BUILD, s + ".o")) for s in b.SOURCES):
        pytest.skip("the kernel objects of the ordinary build are missing (run fp8_moe_amd/build.py)")
    lib = b.build_hostsan()
    env = dict(os.environ, LD_PRELOAD=runtime, B12X_MOE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py"), os.path.join(ROOT, "tests", "test_zz_no_alloc.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, res.stderr[-3000:]
    assert " passed" in res.stdout
