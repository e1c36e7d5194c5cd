"""Python binding of ``libb12x_moe.so`` (the C ABI in ``include/b12x_moe.h``).

Argument marshalling only: every step of the fused MoE runs in the library's
HIP kernels.  PyTorch provides device memory and streams.  The call sequence
mirrors b12x's fused_moe (README "Using it"):

    wplan   = plan_weights(E, H, I, gated, "mxfp4")
    experts = prepare_weights(wplan, w13_codes, w13_scales, w2_codes, w2_scales, ...)
    plan    = plan(wplan, top_k, max_tokens, act_format="bf16", activation="silu")
    spec    = plan.scratch_specs()[0]
    scratch = torch.empty(spec.bytes, dtype=torch.uint8, device="cuda")
    binding = bind(plan, scratch, experts, x, topk_ids, topk_weights, out)
    run(binding)

The library must be built (``python fp8_moe_amd/build.py``); importing this
module fails loudly when it is missing.  There is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# B12X_MOE_LIB: another build of the same library (the host-sanitized one for the sanitizer run)
LIB_PATH = os.environ.get("B12X_MOE_LIB") or os.path.join(_HERE, "libb12x_moe.so")

WEIGHT_FORMATS = {"mxfp4": 1, "nvfp4": 2}
ACT_FORMATS = {"bf16": 1, "mxfp8": 2, "nvfp4": 3}
ACTIVATIONS = {"silu": 1, "relu2": 2, "swiglu_oai": 3}
STAGES = {"route": 1, "quant_x": 2, "gemm1": 3, "gemm2": 4, "combine": 5, "decode1": 6, "decode2": 7}
NOALLOC_SCRATCH_BYTES = 16 << 20   # B12X_NOALLOC_SCRATCH_BYTES: the static scratch of run_noalloc
QUERIES = {"path": 1, "tile_rows": 2, "row_pad": 3, "T": 4, "num_stages": 5}
REGIONS = {"counts": 1, "offsets": 2, "padded_offsets": 3, "sorted": 4, "pos": 5, "tiles": 6, "ntiles": 7,
           "xq": 9, "xs": 10, "h": 11, "hs": 12, "y": 13}

STATUS_NAMES = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "SCRATCH_TOO_SMALL",
                5: "MISALIGNED", 6: "LAYOUT_MISMATCH", 7: "HIP", 8: "FROZEN"}


class B12xError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class B12xUnsupported(B12xError):
    pass


class WeightDesc(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("num_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("gated", ctypes.c_int32), ("weight_format", ctypes.c_int32)]


class WeightPlan(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("layout_id", ctypes.c_uint32), ("desc", WeightDesc),
                ("prepared_bytes", ctypes.c_uint64), ("alignment", ctypes.c_uint64),
                ("w13_codes_off", ctypes.c_uint64), ("w13_scales_off", ctypes.c_uint64),
                ("w13_global_off", ctypes.c_uint64), ("w2_codes_off", ctypes.c_uint64),
                ("w2_scales_off", ctypes.c_uint64), ("w2_global_off", ctypes.c_uint64),
                ("a13_global_off", ctypes.c_uint64), ("a2_global_off", ctypes.c_uint64)]


class WeightSrc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w13_codes", "w13_scales", "w13_global", "w2_codes", "w2_scales", "w2_global", "a13_global",
                 "a2_global")]


class Experts(ctypes.Structure):
    _fields_ = [("plan", WeightPlan), ("base", ctypes.c_void_p), ("bytes", ctypes.c_uint64),
                ("act_scales", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Caps(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("top_k", ctypes.c_int32), ("weights", WeightPlan),
                ("act_format", ctypes.c_int32), ("activation", ctypes.c_int32), ("decode_max_pairs", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("splitk_max_pairs", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ScratchSpec(ctypes.Structure):
    _fields_ = [("bytes", ctypes.c_uint64), ("alignment", ctypes.c_uint64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Binding(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_uint64 * 64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python fp8_moe_amd/build.py` (there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int32
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    i64 = ctypes.c_int64
    sig = {
        "b12x_moe_plan_weights": (st, [P(WeightDesc), P(WeightPlan)]),
        "b12x_moe_prepare_weights": (st, [P(WeightPlan), P(WeightSrc), vp, ctypes.c_uint64, vp, P(Experts)]),
        "b12x_moe_is_supported": (ctypes.c_int32, [P(Caps)]),
        "b12x_moe_plan": (st, [P(Caps), P(vp)]),
        "b12x_moe_plan_destroy": (None, [vp]),
        "b12x_moe_scratch_specs": (st, [vp, P(ScratchSpec), ctypes.c_int32, P(ctypes.c_int32)]),
        "b12x_moe_prime": (st, [vp, vp, ctypes.c_uint64, vp]),
        "b12x_moe_bind": (st, [vp, vp, ctypes.c_uint64, P(Experts), vp, i64, i64, vp, vp, vp, i64, P(Binding)]),
        "b12x_moe_bind_live": (st, [vp, vp, ctypes.c_uint64, P(Experts), vp, i64, vp, vp, vp, i64, vp, P(Binding)]),
        "b12x_moe_freeze": (st, [vp]),
        "b12x_moe_run": (st, [P(Binding), vp]),
        "b12x_moe_run_stage": (st, [P(Binding), ctypes.c_int32, vp]),
        "b12x_moe_run_noalloc": (st, [vp, P(Experts), vp, i64, i64, vp, vp, vp, i64, vp]),
        "b12x_moe_binding_query": (st, [P(Binding), ctypes.c_int32, P(i64)]),
        "b12x_moe_scratch_region": (st, [vp, ctypes.c_int32, P(ctypes.c_uint64), P(ctypes.c_uint64)]),
        "b12x_mxfp8_quantize_rows": (st, [vp, i64, i64, i64, vp, vp, vp]),
        "b12x_gemm_packed_bytes": (st, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P(ctypes.c_uint64)]),
        "b12x_gemm_pack_weight": (st, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, ctypes.c_uint64, vp]),
        "b12x_gemm_mm": (st, [vp, i64, i64, vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, i64, vp]),
        "b12x_status_string": (ctypes.c_char_p, [st]),
        "b12x_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()
EXPORTED = ("b12x_moe_plan_weights", "b12x_moe_prepare_weights", "b12x_moe_is_supported", "b12x_moe_plan",
            "b12x_moe_plan_destroy", "b12x_moe_scratch_specs", "b12x_moe_prime", "b12x_moe_bind",
            "b12x_moe_bind_live", "b12x_moe_freeze", "b12x_moe_run",
            "b12x_moe_run_stage", "b12x_moe_run_noalloc", "b12x_moe_binding_query", "b12x_moe_scratch_region",
            "b12x_mxfp8_quantize_rows", "b12x_gemm_packed_bytes", "b12x_gemm_pack_weight", "b12x_gemm_mm",
            "b12x_status_string",
            "b12x_last_error")


def lib():
    return _lib


def _check(status):
    if status != 0:
        msg = _lib.b12x_last_error().decode(errors="replace")
        cls = B12xUnsupported if status == 2 else B12xError
        raise cls(status, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------- weights

def plan_weights(num_experts, hidden, inter, gated, weight_format):
    d = WeightDesc(ctypes.sizeof(WeightDesc), num_experts, hidden, inter, int(bool(gated)),
                   WEIGHT_FORMATS[weight_format])
    wp = WeightPlan()
    _check(_lib.b12x_moe_plan_weights(ctypes.byref(d), ctypes.byref(wp)))
    return wp


class PreparedExperts:
    """Prepared weights: the caller-owned device buffer and its descriptor."""

    def __init__(self, experts, buffer):
        self.experts = experts
        self.buffer = buffer


def prepare_weights(wplan, w13_codes, w13_scales, w2_codes, w2_scales, w13_global=None, w2_global=None,
                    out=None, stream=None, a13_global=None, a2_global=None):
    """Pack source FP4 weights (device tensors, layouts as in the header).
    a13_global (f32 [1]) / a2_global (f32 [E]): NVFP4 activation scales of x
    and of each expert's h, needed for NVFP4 activations."""
    dev = w13_codes.device
    opt = (w13_global, w2_global, a13_global, a2_global)
    tensors = [w13_codes, w13_scales, w2_codes, w2_scales] + [t for t in opt if t is not None]
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("source weights must be contiguous device tensors")
    if out is None:
        out = torch.empty(wplan.prepared_bytes, dtype=torch.uint8, device=dev)
    def p(t):
        return None if t is None else t.data_ptr()

    src = WeightSrc(w13_codes.data_ptr(), w13_scales.data_ptr(), p(w13_global), w2_codes.data_ptr(),
                    w2_scales.data_ptr(), p(w2_global), p(a13_global), p(a2_global))
    ex = Experts()
    _check(_lib.b12x_moe_prepare_weights(ctypes.byref(wplan), ctypes.byref(src), _ptr(out), out.numel(),
                                         _stream(stream), ctypes.byref(ex)))
    return PreparedExperts(ex, out)


# ---------------------------------------------------------------- op plan

def make_caps(wplan, top_k, max_tokens, act_format="bf16", activation="silu", decode_max_pairs=0,
              splitk_max_pairs=0):
    """decode_max_pairs: largest T*k routed to the decode path (0: library
    default, negative: always use the grouped path); splitk_max_pairs: largest
    T*k that runs the split-K decode kernel (0: default, negative: never)."""
    return Caps(ctypes.sizeof(Caps), top_k, wplan, ACT_FORMATS[act_format], ACTIVATIONS[activation],
                decode_max_pairs, max_tokens, splitk_max_pairs, 0)


def is_supported(wplan, top_k, max_tokens, act_format="bf16", activation="silu"):
    caps = make_caps(wplan, top_k, max_tokens, act_format, activation)
    return bool(_lib.b12x_moe_is_supported(ctypes.byref(caps)))


class Plan:
    def __init__(self, handle, caps):
        self._h = handle
        self.caps = caps
        self._destroy = _lib.b12x_moe_plan_destroy

    @property
    def handle(self):
        return self._h

    def scratch_specs(self):
        n = ctypes.c_int32(0)
        specs = (ScratchSpec * 4)()
        _check(_lib.b12x_moe_scratch_specs(self._h, specs, 4, ctypes.byref(n)))
        return [specs[i] for i in range(n.value)]

    def scratch_region(self, name):
        off, nbytes = ctypes.c_uint64(0), ctypes.c_uint64(0)
        _check(_lib.b12x_moe_scratch_region(self._h, REGIONS[name], ctypes.byref(off), ctypes.byref(nbytes)))
        return off.value, nbytes.value

    def __del__(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None


def plan(wplan, top_k, max_tokens, act_format="bf16", activation="silu", decode_max_pairs=0, splitk_max_pairs=0):
    caps = make_caps(wplan, top_k, max_tokens, act_format, activation, decode_max_pairs, splitk_max_pairs)
    h = ctypes.c_void_p()
    _check(_lib.b12x_moe_plan(ctypes.byref(caps), ctypes.byref(h)))
    return Plan(h, caps)


def alloc_scratch(p, device="cuda", stream=None):
    """A scratch buffer for plan p, primed (b12x_moe_prime) on `stream`."""
    spec = p.scratch_specs()[0]
    scratch = torch.empty(spec.bytes, dtype=torch.uint8, device=device)
    prime(p, scratch, stream)
    return scratch


def prime(p, scratch, stream=None):
    """b12x_moe_prime: zero the decode synchronization region of a scratch
    buffer (once per buffer, before its first run)."""
    _check(_lib.b12x_moe_prime(p.handle, _ptr(scratch), scratch.numel(), _stream(stream)))


def bind(p, scratch, experts, a, topk_ids, topk_weights, out):
    """a, out: bf16 [T, H] (row stride a.stride(0)); topk_ids int32 [T, k];
    topk_weights float32 [T, k]; scratch: uint8 device tensor."""
    T = a.shape[0]
    for t, dt in ((a, torch.bfloat16), (out, torch.bfloat16), (topk_ids, torch.int32),
                  (topk_weights, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"expected {dt}, got {t.dtype}")
    if topk_ids.shape != topk_weights.shape or topk_ids.shape[0] != T or out.shape[0] != T:
        raise ValueError("shape mismatch between a, out, topk_ids and topk_weights")
    if not (topk_ids.is_contiguous() and topk_weights.is_contiguous()):
        raise ValueError("topk_ids / topk_weights must be contiguous")
    b = Binding()
    _check(_lib.b12x_moe_bind(p.handle, _ptr(scratch), scratch.numel(), ctypes.byref(experts.experts), _ptr(a), T,
                              a.stride(0), _ptr(topk_ids), _ptr(topk_weights), _ptr(out), out.stride(0),
                              ctypes.byref(b)))
    return b


def bind_live(p, scratch, experts, a, topk_ids, topk_weights, out, t_live):
    """b12x_moe_bind_live: a, out bf16 [max_tokens, H]; topk_ids int32 and
    topk_weights float32 [max_tokens, k]; t_live: int32 device tensor of one
    element, the token count each run reads when its kernels run."""
    for t, dt in ((a, torch.bfloat16), (out, torch.bfloat16), (topk_ids, torch.int32),
                  (topk_weights, torch.float32), (t_live, torch.int32)):
        if t.dtype != dt:
            raise TypeError(f"expected {dt}, got {t.dtype}")
    cap = p.caps.max_tokens
    if (a.shape[0] < cap or out.shape[0] < cap or topk_ids.shape[0] < cap or topk_weights.shape != topk_ids.shape
            or t_live.numel() != 1):
        raise ValueError("a, out, topk_ids and topk_weights need max_tokens rows; t_live one element")
    if not (topk_ids.is_contiguous() and topk_weights.is_contiguous()):
        raise ValueError("topk_ids / topk_weights must be contiguous")
    b = Binding()
    _check(_lib.b12x_moe_bind_live(p.handle, _ptr(scratch), scratch.numel(), ctypes.byref(experts.experts), _ptr(a),
                                   a.stride(0), _ptr(topk_ids), _ptr(topk_weights), _ptr(out), out.stride(0),
                                   _ptr(t_live), ctypes.byref(b)))
    return b


def freeze(p):
    """b12x_moe_freeze: bindings of paths not used before now fail."""
    _check(_lib.b12x_moe_freeze(p.handle))


def run(binding, stream=None):
    _check(_lib.b12x_moe_run(ctypes.byref(binding), _stream(stream)))


def run_noalloc(p, experts, a, topk_ids, topk_weights, out, stream=None):
    """b12x_moe_run_noalloc: bind + run on the library's static scratch (split-K
    decode path only); same arguments as bind() without the scratch."""
    T = a.shape[0]
    for t, dt in ((a, torch.bfloat16), (out, torch.bfloat16), (topk_ids, torch.int32),
                  (topk_weights, torch.float32)):
        if t.dtype != dt:
            raise TypeError(f"expected {dt}, got {t.dtype}")
    if topk_ids.shape != topk_weights.shape or topk_ids.shape[0] != T or out.shape[0] != T:
        raise ValueError("shape mismatch between a, out, topk_ids and topk_weights")
    if not (topk_ids.is_contiguous() and topk_weights.is_contiguous()):
        raise ValueError("topk_ids / topk_weights must be contiguous")
    _check(_lib.b12x_moe_run_noalloc(p.handle, ctypes.byref(experts.experts), _ptr(a), T, a.stride(0),
                                     _ptr(topk_ids), _ptr(topk_weights), _ptr(out), out.stride(0), _stream(stream)))


def run_stage(binding, stage, stream=None):
    _check(_lib.b12x_moe_run_stage(ctypes.byref(binding), STAGES[stage], _stream(stream)))


def binding_query(binding, what):
    v = ctypes.c_int64(0)
    _check(_lib.b12x_moe_binding_query(ctypes.byref(binding), QUERIES[what], ctypes.byref(v)))
    return v.value


def mxfp8_quantize_rows(x, codes=None, scales=None, stream=None):
    """bf16 [rows, cols] -> (uint8 codes [rows, cols], uint8 E8M0 scales [rows, cols/32])."""
    rows, cols = x.shape
    if x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be bf16 with unit column stride")
    if codes is None:
        codes = torch.empty(rows, cols, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device)
    _check(_lib.b12x_mxfp8_quantize_rows(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales),
                                         _stream(stream)))
    return codes, scales


_WFMT = {"mxfp4": 1, "nvfp4": 2}


def gemm_pack_weight(codes, scales, weight_format, stream=None):
    """Dense block-scaled weight W [n, k] (uint8 codes [n, k/2], uint8 scales
    [n, k/32] or [n, k/16]) -> packed uint8 device tensor for gemm_mm."""
    n, k = codes.shape[0], codes.shape[1] * 2
    nb = ctypes.c_uint64()
    _check(_lib.b12x_gemm_packed_bytes(n, k, _WFMT[weight_format], ctypes.byref(nb)))
    dst = torch.empty(nb.value, dtype=torch.uint8, device=codes.device)
    _check(_lib.b12x_gemm_pack_weight(n, k, _WFMT[weight_format], _ptr(codes), _ptr(scales), _ptr(dst), nb.value,
                                      _stream(stream)))
    return dst


def gemm_mm(x, w_packed, n, weight_format, global_scale=None, out=None, stream=None):
    """out[m, n] = bf16(x[m, :] . W[n, :]): x bf16 [m, k] with unit column stride,
    w_packed from gemm_pack_weight, global_scale a 1-element float32 device
    tensor (NVFP4)."""
    m, k = x.shape
    if x.dtype != torch.bfloat16 or x.stride(1) != 1:
        raise ValueError("x must be bf16 with unit column stride")
    if out is None:
        out = torch.empty(m, n, dtype=torch.bfloat16, device=x.device)
    _check(_lib.b12x_gemm_mm(_ptr(x), m, x.stride(0), _ptr(w_packed), n, k, _WFMT[weight_format], _ptr(global_scale),
                             _ptr(out), out.stride(0), _stream(stream)))
    return out


class FusedMoE:
    """Convenience holder for one prepared model layer: weights plan,
    prepared experts and an op plan at a given capacity."""

    def __init__(self, E, H, I, top_k, weight_format, act_format, activation, max_tokens, weights, stream=None,
                 decode_max_pairs=0, splitk_max_pairs=0):
        gated = activation != "relu2"
        self.wplan = plan_weights(E, H, I, gated, weight_format)
        self.experts = prepare_weights(self.wplan, weights["w13_codes"], weights["w13_scales"],
                                       weights["w2_codes"], weights["w2_scales"], weights.get("w13_global"),
                                       weights.get("w2_global"), stream=stream,
                                       a13_global=weights.get("a13_global"), a2_global=weights.get("a2_global"))
        self.plan = plan(self.wplan, top_k, max_tokens, act_format, activation, decode_max_pairs, splitk_max_pairs)
        self.scratch = alloc_scratch(self.plan, weights["w13_codes"].device)
        self.H = H

    def bind(self, a, topk_ids, topk_weights, out=None):
        if out is None:
            out = torch.empty(a.shape[0], self.H, dtype=torch.bfloat16, device=a.device)
        return bind(self.plan, self.scratch, self.experts, a, topk_ids, topk_weights, out), out

    def __call__(self, a, topk_ids, topk_weights, out=None, stream=None):
        b, out = self.bind(a, topk_ids, topk_weights, out)
        run(b, stream)
        return out
