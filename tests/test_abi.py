"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and its host-side planning and binding validation behave as the
header documents (no device work is launched by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(header="b12x_moe.h"):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(b12x_\w+)\s*\(", text)))


def test_probe_library_is_separate():
    # the harness's measurement probes live in their own library, not in the MoE ABI
    import fp8_moe_amd as fm
    names = _declared_functions("b12x_probes.h")
    assert names == ["b12x_probe_mfma", "b12x_probe_stream_read"]
    probes = ctypes.CDLL(os.path.join(ROOT, "fp8_moe_amd", "libb12x_probes.so"))
    for n in names:
        assert hasattr(probes, n), n
        assert not hasattr(ctypes.CDLL(fm.LIB_PATH), n), n


def test_library_exports_every_declared_function():
    import fp8_moe_amd as fm
    names = _declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(fm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fm.EXPORTED)


def test_weight_plan_sizes():
    import fp8_moe_amd as fm
    wp = fm.plan_weights(128, 2048, 768, True, "mxfp4")
    codes13 = 128 * 1536 * 2048 // 2
    codes2 = 128 * 2048 * 768 // 2
    assert wp.w13_scales_off - wp.w13_codes_off == codes13
    assert wp.w2_scales_off - wp.w2_codes_off == codes2
    assert wp.prepared_bytes >= codes13 + codes2 + (codes13 + codes2) // 16
    assert wp.alignment == 256 and all(o % 256 == 0 for o in (wp.w13_scales_off, wp.w2_codes_off, wp.w2_scales_off))
    nv = fm.plan_weights(8, 160, 96, False, "nvfp4")       # K = 160 pads to two 128-K fragments
    assert nv.w13_scales_off - nv.w13_codes_off == 8 * (96 // 16) * 2 * 1024


@pytest.mark.parametrize("E,H,I,fmt,err", [(8, 100, 128, "mxfp4", 2), (8, 256, 48, "nvfp4", 2),
                                           (0, 256, 128, "mxfp4", 1), (2000, 256, 128, "mxfp4", 2)])
def test_weight_plan_rejects(E, H, I, fmt, err):
    import fp8_moe_amd as fm
    with pytest.raises(fm.B12xError) as e:
        fm.plan_weights(E, H, I, True, fmt)
    assert e.value.status == err


def test_support_matrix():
    import fp8_moe_amd as fm
    mx_g = fm.plan_weights(8, 256, 128, True, "mxfp4")
    mx_r = fm.plan_weights(8, 256, 128, False, "mxfp4")
    nv_g = fm.plan_weights(8, 256, 128, True, "nvfp4")
    assert fm.is_supported(mx_g, 2, 16, "bf16", "silu")
    assert fm.is_supported(mx_g, 2, 16, "mxfp8", "silu")
    assert fm.is_supported(mx_r, 2, 16, "mxfp8", "relu2")
    assert fm.is_supported(nv_g, 2, 16, "bf16", "silu")
    assert fm.is_supported(nv_g, 2, 16, "mxfp8", "silu")          # NVFP4 x MXFP8 through bf16 round trips
    assert fm.is_supported(nv_g, 2, 16, "nvfp4", "silu")          # NVFP4 x NVFP4 (W4A4)
    assert not fm.is_supported(mx_g, 2, 16, "nvfp4", "silu")      # NVFP4 activations need NVFP4 weights
    assert not fm.is_supported(mx_g, 2, 16, "bf16", "relu2")      # gated weights need SiLU or SwiGLU-OAI
    for af in ("bf16", "mxfp8"):
        assert fm.is_supported(mx_g, 2, 16, af, "swiglu_oai")
        assert fm.is_supported(nv_g, 2, 16, af, "swiglu_oai")
        assert not fm.is_supported(mx_r, 2, 16, af, "swiglu_oai")  # SwiGLU-OAI needs gated weights
    assert fm.is_supported(nv_g, 2, 16, "nvfp4", "swiglu_oai")
    assert not fm.is_supported(mx_g, 0, 16, "bf16", "silu")


def test_scratch_grows_with_capacity_only():
    import fp8_moe_amd as fm
    wp = fm.plan_weights(128, 2048, 768, True, "mxfp4")
    small = fm.plan(wp, 8, 32).scratch_specs()[0].bytes
    big = fm.plan(wp, 8, 4096).scratch_specs()[0].bytes
    assert 0 < small < big
    p = fm.plan(wp, 8, 32)
    for name in fm.REGIONS:
        off, n = p.scratch_region(name)
        assert off % 256 == 0 and off + n <= p.scratch_specs()[0].bytes


class _FakeTensor:
    """Stand-in device tensor for binding validation (bind never touches memory)."""

    def __init__(self, ptr, shape, stride0, dtype, numel=0):
        self.ptr, self.shape, self._s0, self.dtype, self._n = ptr, shape, stride0, dtype, numel

    def data_ptr(self):
        return self.ptr

    def stride(self, i):
        return self._s0

    def numel(self):
        return self._n

    def is_contiguous(self):
        return True


def _bind_status(p, ex, T, a_ptr=0x10000, a_stride=256, out_ptr=0x9000000, scratch_ptr=0x4000000, scratch_bytes=None,
                 ids_ptr=0x200000, tw_ptr=0x300000):
    import fp8_moe_amd as fm
    if scratch_bytes is None:
        scratch_bytes = p.scratch_specs()[0].bytes
    b = fm.Binding()
    return fm.lib().b12x_moe_bind(p.handle, ctypes.c_void_p(scratch_ptr), scratch_bytes, ctypes.byref(ex),
                                  ctypes.c_void_p(a_ptr), T, a_stride, ctypes.c_void_p(ids_ptr),
                                  ctypes.c_void_p(tw_ptr), ctypes.c_void_p(out_ptr), a_stride, ctypes.byref(b)), b


def test_prime_validation_on_host():
    """b12x_moe_prime checks its arguments before it enqueues anything; a
    plan without a decode path has nothing to prime."""
    import fp8_moe_amd as fm
    wp = fm.plan_weights(8, 256, 128, True, "mxfp4")
    p = fm.plan(wp, 2, 16)
    nbytes = p.scratch_specs()[0].bytes
    prime = fm.lib().b12x_moe_prime
    assert prime(p.handle, None, nbytes, None) == 1                          # NULL scratch
    assert prime(p.handle, ctypes.c_void_p(0x4000080), nbytes, None) == 5    # misaligned
    assert prime(p.handle, ctypes.c_void_p(0x4000000), nbytes - 1, None) == 4   # too small
    grouped_only = fm.plan(wp, 2, 16, decode_max_pairs=-1)
    assert prime(grouped_only.handle, ctypes.c_void_p(0x4000000), grouped_only.scratch_specs()[0].bytes, None) == 0


def test_freeze_refuses_unresolved_paths():
    """b12x_moe_freeze: a binding of a path that no binding of the plan used
    before is refused (status 8); paths used before keep binding."""
    import fp8_moe_amd as fm
    wp = fm.plan_weights(8, 256, 128, True, "mxfp4")
    p = fm.plan(wp, 2, 512)   # T*k: <= 32 split-K, <= 256 decode, beyond grouped
    ex = fm.Experts(wp, ctypes.c_void_p(0x7000000), wp.prepared_bytes)
    assert _bind_status(p, ex, 1)[0] == 0
    assert fm.binding_query(_bind_status(p, ex, 1)[1], "path") == 3
    assert _bind_status(p, ex, 300)[0] == 0                                  # grouped, resolved
    assert fm.lib().b12x_moe_freeze(p.handle) == 0
    assert _bind_status(p, ex, 16)[0] == 0                                   # split-K again
    assert _bind_status(p, ex, 400)[0] == 0                                  # grouped again
    assert _bind_status(p, ex, 64)[0] == 8                                   # decode: never resolved
    b = fm.Binding()
    live = fm.lib().b12x_moe_bind_live(p.handle, ctypes.c_void_p(0x4000000), p.scratch_specs()[0].bytes,
                                       ctypes.byref(ex), ctypes.c_void_p(0x10000), 256, ctypes.c_void_p(0x200000),
                                       ctypes.c_void_p(0x300000), ctypes.c_void_p(0x9000000), 256,
                                       ctypes.c_void_p(0x500000), ctypes.byref(b))
    assert live == 8                                                         # live: never resolved
    assert fm.lib().b12x_moe_freeze(None) == 1


def test_bind_live_validation_on_host():
    import fp8_moe_amd as fm
    wp = fm.plan_weights(8, 256, 128, True, "mxfp4")
    p = fm.plan(wp, 2, 64)
    ex = fm.Experts(wp, ctypes.c_void_p(0x7000000), wp.prepared_bytes)
    nbytes = p.scratch_specs()[0].bytes

    def live(t_ptr, out_ptr=0x9000000):
        b = fm.Binding()
        st = fm.lib().b12x_moe_bind_live(p.handle, ctypes.c_void_p(0x4000000), nbytes, ctypes.byref(ex),
                                         ctypes.c_void_p(0x10000), 256, ctypes.c_void_p(0x200000),
                                         ctypes.c_void_p(0x300000), ctypes.c_void_p(out_ptr), 256,
                                         ctypes.c_void_p(t_ptr) if t_ptr else None, ctypes.byref(b))
        return st, b
    st, b = live(0x500000)
    assert st == 0
    assert fm.binding_query(b, "path") == 4 and fm.binding_query(b, "T") == 64
    assert fm.binding_query(b, "num_stages") == 0
    assert fm.lib().b12x_moe_run_stage(ctypes.byref(b), 6, None) == 2      # whole calls only
    assert live(0)[0] == 1                                                   # no live count
    assert live(0x500002)[0] == 5                                            # misaligned count
    assert live(0x500000, out_ptr=0x10000 + 512)[0] == 1                     # out aliases a (at capacity)


def test_bind_validation_on_host():
    import fp8_moe_amd as fm
    wp = fm.plan_weights(8, 256, 128, True, "mxfp4")
    p = fm.plan(wp, 2, 16)
    ex = fm.Experts(wp, ctypes.c_void_p(0x7000000), wp.prepared_bytes)
    st, b = _bind_status(p, ex, 16)
    assert st == 0
    assert fm.binding_query(b, "T") == 16 and fm.binding_query(b, "tile_rows") % fm.binding_query(b, "row_pad") == 0
    assert _bind_status(p, ex, 17)[0] == 3                                   # capacity
    assert _bind_status(p, ex, 16, a_ptr=0x10008)[0] == 5                    # misaligned a
    assert _bind_status(p, ex, 16, scratch_ptr=0x4000080)[0] == 5            # misaligned scratch
    assert _bind_status(p, ex, 16, scratch_bytes=1024)[0] == 4               # scratch too small
    assert _bind_status(p, ex, 16, out_ptr=0x10000 + 512)[0] == 1            # out aliases a
    assert _bind_status(p, ex, 16, a_stride=100)[0] == 1                     # stride < H
    assert _bind_status(p, ex, 0, a_ptr=0, out_ptr=0, ids_ptr=0, tw_ptr=0)[0] == 0   # T = 0 needs no buffers
    other = fm.plan_weights(8, 256, 128, True, "nvfp4")
    ex2 = fm.Experts(other, ctypes.c_void_p(0x7000000), other.prepared_bytes)
    assert _bind_status(p, ex2, 16)[0] == 6                                  # layout mismatch
    assert fm.lib().b12x_moe_run(None, None) == 1
    # NVFP4 activations need the activation scales among the prepared weights
    p4 = fm.plan(other, 2, 16, "nvfp4")
    assert _bind_status(p4, ex2, 16)[0] == 1
    ex3 = fm.Experts(other, ctypes.c_void_p(0x7000000), other.prepared_bytes, 1)
    assert _bind_status(p4, ex3, 16)[0] == 0


def test_status_strings():
    import fp8_moe_amd as fm
    for s in range(8):
        assert fm.lib().b12x_status_string(s)
    assert fm.lib().b12x_status_string(99) == b"unknown status"


def test_path_selection_at_bind():
    import fp8_moe_amd as fm
    wp = fm.plan_weights(128, 2048, 768, True, "mxfp4")
    ex = fm.Experts(wp, ctypes.c_void_p(0x7000000), wp.prepared_bytes)
    p = fm.plan(wp, 8, 64)
    assert fm.binding_query(_bind_status(p, ex, 4, a_stride=2048)[1], "path") == 3      # 32 pairs: split-K decode
    assert fm.binding_query(_bind_status(p, ex, 5, a_stride=2048)[1], "path") == 2      # 40 pairs: decode
    assert fm.binding_query(_bind_status(p, ex, 32, a_stride=2048)[1], "path") == 2     # 256 pairs: decode
    assert fm.binding_query(_bind_status(p, ex, 33, a_stride=2048)[1], "path") == 1     # 264 pairs: grouped
    nosk = fm.plan(wp, 8, 64, splitk_max_pairs=-1)
    assert fm.binding_query(_bind_status(nosk, ex, 1, a_stride=2048)[1], "path") == 2
    wider = fm.plan(wp, 8, 64, splitk_max_pairs=64)
    assert fm.binding_query(_bind_status(wider, ex, 8, a_stride=2048)[1], "path") == 3
    assert fm.binding_query(_bind_status(wider, ex, 9, a_stride=2048)[1], "path") == 2
    never = fm.plan(wp, 8, 64, decode_max_pairs=-1)
    assert fm.binding_query(_bind_status(never, ex, 1, a_stride=2048)[1], "path") == 1
    small = fm.plan(wp, 8, 64, decode_max_pairs=64, splitk_max_pairs=-1)
    assert fm.binding_query(_bind_status(small, ex, 8, a_stride=2048)[1], "path") == 2
    assert fm.binding_query(_bind_status(small, ex, 9, a_stride=2048)[1], "path") == 1
    wide = fm.plan_weights(8, 7168, 256, True, "nvfp4")                                   # K too long per wave
    exw = fm.Experts(wide, ctypes.c_void_p(0x7000000), wide.prepared_bytes)
    pw = fm.plan(wide, 8, 4)
    assert fm.binding_query(_bind_status(pw, exw, 1, a_stride=7168)[1], "path") == 1
