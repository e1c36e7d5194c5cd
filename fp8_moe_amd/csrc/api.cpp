// Host runtime and C ABI of the fused MoE: weight planning, op planning,
// scratch layout, binding validation and launch sequencing.  Plan, scratch
// and bind logic touch no device; only prepare_weights, run, run_stage and
// quantize_rows enqueue kernels.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>

#include "internal.h"

using namespace b12x;

namespace {

thread_local char g_err[512];

b12x_status fail(b12x_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
b12x_status fail(b12x_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

b12x_status hip_fail(int err, const char* what) {
  return fail(B12X_ERR_HIP, "%s: HIP error %d (%s)", what, err, hip_error_name(err));
}

uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool aligned(const void* p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

b12x_status check_desc(const b12x_moe_weight_desc* d) {
  if (!d) return fail(B12X_ERR_INVALID_ARGUMENT, "weight desc is NULL");
  if (d->struct_size != sizeof(b12x_moe_weight_desc))
    return fail(B12X_ERR_INVALID_ARGUMENT, "weight desc struct_size %u != %zu", d->struct_size,
                sizeof(b12x_moe_weight_desc));
  if (d->weight_format != B12X_WEIGHT_MXFP4 && d->weight_format != B12X_WEIGHT_NVFP4)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown weight format %d", d->weight_format);
  if (d->gated != 0 && d->gated != 1) return fail(B12X_ERR_INVALID_ARGUMENT, "gated must be 0 or 1");
  if (d->num_experts < 1 || d->hidden < 1 || d->inter < 1)
    return fail(B12X_ERR_INVALID_ARGUMENT, "E, H and I must be positive");
  if (d->num_experts > kMaxExperts)
    return fail(B12X_ERR_UNSUPPORTED, "E = %d exceeds %d experts", d->num_experts, kMaxExperts);
  // whole scale blocks along both contractions, whole 16-row fragments along both outputs
  if (d->hidden % 32 || d->inter % 32)
    return fail(B12X_ERR_UNSUPPORTED, "H (%d) and I (%d) must be multiples of 32", d->hidden, d->inter);
  if ((int64_t)d->hidden * d->inter * d->num_experts > (int64_t)1 << 40)
    return fail(B12X_ERR_UNSUPPORTED, "weights larger than 2^40 elements");
  // one expert's packed matrix (K padded to 128) must stay below 1 GiB
  const int64_t n13 = (int64_t)(d->gated ? 2 : 1) * d->inter;
  if (n13 * (int64_t)align_up(d->hidden, kFragK) / 2 >= kMaxBufferBytes ||
      (int64_t)d->hidden * (int64_t)align_up(d->inter, kFragK) / 2 >= kMaxBufferBytes)
    return fail(B12X_ERR_UNSUPPORTED, "one expert's packed weights exceed 1 GiB");
  return B12X_OK;
}

b12x_status check_caps(const b12x_moe_caps* c) {
  if (!c) return fail(B12X_ERR_INVALID_ARGUMENT, "caps is NULL");
  if (c->struct_size != sizeof(b12x_moe_caps))
    return fail(B12X_ERR_INVALID_ARGUMENT, "caps struct_size %u != %zu", c->struct_size, sizeof(b12x_moe_caps));
  if (c->weights.struct_size != sizeof(b12x_moe_weight_plan) || c->weights.layout_id != kLayoutId)
    return fail(B12X_ERR_INVALID_ARGUMENT, "caps.weights is not a plan from b12x_moe_plan_weights");
  b12x_status st = check_desc(&c->weights.desc);
  if (st) return st;
  if (c->top_k < 1 || c->top_k > 64) return fail(B12X_ERR_UNSUPPORTED, "top_k %d outside [1, 64]", c->top_k);
  if (c->max_tokens < 1) return fail(B12X_ERR_INVALID_ARGUMENT, "max_tokens must be >= 1");
  if (c->max_tokens * c->top_k > ((int64_t)1 << 30))
    return fail(B12X_ERR_UNSUPPORTED, "max_tokens * top_k exceeds 2^30 pairs");
  if (c->act_format != B12X_ACT_BF16 && c->act_format != B12X_ACT_MXFP8 && c->act_format != B12X_ACT_NVFP4)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown activation format %d", c->act_format);
  if (c->act_format == B12X_ACT_NVFP4 && c->weights.desc.weight_format != B12X_WEIGHT_NVFP4)
    return fail(B12X_ERR_UNSUPPORTED, "NVFP4 activations run with NVFP4 weights only");
  if (c->activation != B12X_ACTIVATION_SILU_GATED && c->activation != B12X_ACTIVATION_RELU2 &&
      c->activation != B12X_ACTIVATION_SWIGLU_OAI)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown activation %d", c->activation);
  if ((c->activation != B12X_ACTIVATION_RELU2) != (c->weights.desc.gated == 1))
    return fail(B12X_ERR_UNSUPPORTED,
                "SiLU-gated and SwiGLU-OAI experts need gated weights and ReLU^2 needs non-gated ones");
  return B12X_OK;
}

}  // namespace

extern "C" {

const char* b12x_status_string(b12x_status s) {
  switch (s) {
    case B12X_OK: return "ok";
    case B12X_ERR_INVALID_ARGUMENT: return "invalid argument";
    case B12X_ERR_UNSUPPORTED: return "unsupported";
    case B12X_ERR_CAPACITY: return "capacity exceeded";
    case B12X_ERR_SCRATCH_TOO_SMALL: return "scratch too small";
    case B12X_ERR_MISALIGNED: return "misaligned";
    case B12X_ERR_LAYOUT_MISMATCH: return "layout mismatch";
    case B12X_ERR_HIP: return "HIP error";
    case B12X_ERR_FROZEN: return "kernel resolution frozen";
    default: return "unknown status";
  }
}

const char* b12x_last_error(void) { return g_err; }

b12x_status b12x_moe_plan_weights(const b12x_moe_weight_desc* d, b12x_moe_weight_plan* out) {
  b12x_status st = check_desc(d);
  if (st) return st;
  if (!out) return fail(B12X_ERR_INVALID_ARGUMENT, "out is NULL");
  MatrixLayout l13 = make_matrix_layout((int64_t)(d->gated ? 2 : 1) * d->inter, d->hidden, d->weight_format);
  MatrixLayout l2 = make_matrix_layout(d->hidden, d->inter, d->weight_format);
  const uint64_t E = (uint64_t)d->num_experts;
  memset(out, 0, sizeof(*out));
  out->struct_size = sizeof(b12x_moe_weight_plan);
  out->layout_id = kLayoutId;
  out->desc = *d;
  out->alignment = 256;
  uint64_t off = 0;
  out->w13_codes_off = off;  off = align_up(off + E * l13.codes_per_expert, 256);
  out->w13_scales_off = off; off = align_up(off + E * l13.scales_per_expert, 256);
  out->w2_codes_off = off;   off = align_up(off + E * l2.codes_per_expert, 256);
  out->w2_scales_off = off;  off = align_up(off + E * l2.scales_per_expert, 256);
  out->w13_global_off = off; off = align_up(off + E * 4, 256);
  out->w2_global_off = off;  off = align_up(off + E * 4, 256);
  out->a13_global_off = off; off = align_up(off + 4, 256);
  out->a2_global_off = off;  off = align_up(off + E * 4, 256);
  out->prepared_bytes = off;
  return B12X_OK;
}

b12x_status b12x_moe_prepare_weights(const b12x_moe_weight_plan* wp, const b12x_moe_weight_src* src, void* dst,
                                     uint64_t dst_bytes, void* stream, b12x_moe_experts* out) {
  if (!wp || !src || !dst || !out) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL argument");
  if (wp->struct_size != sizeof(b12x_moe_weight_plan) || wp->layout_id != kLayoutId)
    return fail(B12X_ERR_INVALID_ARGUMENT, "not a weight plan from b12x_moe_plan_weights");
  b12x_status st = check_desc(&wp->desc);
  if (st) return st;
  if (dst_bytes < wp->prepared_bytes)
    return fail(B12X_ERR_SCRATCH_TOO_SMALL, "prepared buffer %llu < %llu bytes", (unsigned long long)dst_bytes,
                (unsigned long long)wp->prepared_bytes);
  if (!aligned(dst, wp->alignment)) return fail(B12X_ERR_MISALIGNED, "prepared buffer not %llu-byte aligned",
                                                (unsigned long long)wp->alignment);
  const b12x_moe_weight_desc& d = wp->desc;
  const bool nv = d.weight_format == B12X_WEIGHT_NVFP4;
  if (!src->w13_codes || !src->w13_scales || !src->w2_codes || !src->w2_scales)
    return fail(B12X_ERR_INVALID_ARGUMENT, "NULL source weight pointer");
  if (nv && (!src->w13_global || !src->w2_global))
    return fail(B12X_ERR_INVALID_ARGUMENT, "NVFP4 weights need both per-expert fp32 scales");
  if ((src->a13_global || src->a2_global) && (!nv || !src->a13_global || !src->a2_global))
    return fail(B12X_ERR_INVALID_ARGUMENT, "activation scales: both a13_global and a2_global, NVFP4 weights only");
  if (!aligned(src->w13_codes, 16) || !aligned(src->w2_codes, 16))
    return fail(B12X_ERR_MISALIGNED, "source codes must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)dst;
  PackArgs a;
  a.wfmt = d.weight_format;
  a.E = d.num_experts;
  a.l = make_matrix_layout((int64_t)(d.gated ? 2 : 1) * d.inter, d.hidden, d.weight_format);
  a.src_codes = (const uint8_t*)src->w13_codes;
  a.src_scales = (const uint8_t*)src->w13_scales;
  a.dst_codes = base + wp->w13_codes_off;
  a.dst_scales = base + wp->w13_scales_off;
  a.gated_interleave = d.gated;
  int err = launch_pack(a, s);
  if (err) return hip_fail(err, "pack w13");
  a.l = make_matrix_layout(d.hidden, d.inter, d.weight_format);
  a.src_codes = (const uint8_t*)src->w2_codes;
  a.src_scales = (const uint8_t*)src->w2_scales;
  a.dst_codes = base + wp->w2_codes_off;
  a.dst_scales = base + wp->w2_scales_off;
  a.gated_interleave = 0;
  err = launch_pack(a, s);
  if (err) return hip_fail(err, "pack w2");
  if (nv) {
    err = launch_copy_f32(src->w13_global, (float*)(base + wp->w13_global_off), d.num_experts, s);
    if (!err) err = launch_copy_f32(src->w2_global, (float*)(base + wp->w2_global_off), d.num_experts, s);
    if (err) return hip_fail(err, "copy global scales");
  }
  const bool act_scales = nv && src->a13_global && src->a2_global;
  if (act_scales) {
    err = launch_copy_f32(src->a13_global, (float*)(base + wp->a13_global_off), 1, s);
    if (!err) err = launch_copy_f32(src->a2_global, (float*)(base + wp->a2_global_off), d.num_experts, s);
    if (err) return hip_fail(err, "copy activation scales");
  }
  out->plan = *wp;
  out->base = dst;
  out->bytes = dst_bytes;
  out->act_scales = act_scales ? 1 : 0;
  out->reserved = 0;
  return B12X_OK;
}

int32_t b12x_moe_is_supported(const b12x_moe_caps* caps) { return check_caps(caps) == B12X_OK ? 1 : 0; }

b12x_status b12x_moe_plan(const b12x_moe_caps* caps, b12x_moe_plan_t* out) {
  b12x_status st = check_caps(caps);
  if (st) return st;
  if (!out) return fail(B12X_ERR_INVALID_ARGUMENT, "out is NULL");
  b12x_moe_plan_impl* p = new (std::nothrow) b12x_moe_plan_impl();
  if (!p) return fail(B12X_ERR_INVALID_ARGUMENT, "host allocation failed");
  const b12x_moe_weight_desc& d = caps->weights.desc;
  p->caps = *caps;
  p->E = d.num_experts;
  p->H = d.hidden;
  p->I = d.inter;
  p->k = caps->top_k;
  p->gated = d.gated;
  p->wfmt = d.weight_format;
  p->afmt = caps->act_format;
  p->act = caps->activation;
  p->max_tokens = caps->max_tokens;
  p->l13 = make_matrix_layout((int64_t)(d.gated ? 2 : 1) * d.inter, d.hidden, d.weight_format);
  p->l2 = make_matrix_layout(d.hidden, d.inter, d.weight_format);
  p->Hp = align_up(p->H, kFragK);
  p->Ip = align_up(p->I, kFragK);
  p->max_pairs = p->max_tokens * p->k;
  p->max_rows = p->max_pairs + (int64_t)p->E * (kRowPad - 1);
  p->max_rows = (int64_t)align_up(p->max_rows, kRowPad);
  p->max_tiles = (p->max_rows + kTileRows - 1) / kTileRows + p->E;
  p->max_chunks = (p->max_pairs + kRouteChunk - 1) / kRouteChunk;
  // decode path: every wave keeps its K fragments in registers (<= 8 of them)
  const bool decode_ok = (p->l13.kf + 3) / 4 <= kDecodeMaxKPerWave && (p->l2.kf + 3) / 4 <= kDecodeMaxKPerWave;
  int dmax = caps->decode_max_pairs == 0 ? kDecodePairs : caps->decode_max_pairs;
  if (dmax > kDecodePairs) dmax = kDecodePairs;
  p->decode_max_pairs = (decode_ok && dmax > 0) ? dmax : 0;
  int smax = caps->splitk_max_pairs == 0 ? kSplitKPairs : caps->splitk_max_pairs;
  if (smax > kSplitKMaxPairs) smax = kSplitKMaxPairs;
  const bool splitk_ok = p->H <= kSplitKMaxH;
  if (smax > p->decode_max_pairs) smax = p->decode_max_pairs;  // a part of the decode path
  p->splitk_max_pairs = (splitk_ok && smax > 0) ? smax : 0;
  const bool a8 = a8_native(p->wfmt, p->afmt);
  // NVFP4 weights with bf16 activations: the grouped path's GEMM1 reads a
  // scaled f16 copy of a (2 bytes per element) and one exponent per row.
  // NVFP4 weights with MXFP8 (NVFP4) activations: both paths read a copy of
  // a's MXFP8 (NVFP4) round trips, f16 with row exponents on the grouped path.
  const bool x16 = p->wfmt == B12X_WEIGHT_NVFP4 && p->afmt == B12X_ACT_BF16;
  const bool xrt = a8_bf16(p->wfmt, p->afmt) || a4_nv(p->afmt);
  uint64_t len[R_COUNT_] = {0};
  len[R_COUNTS] = 4ull * p->E;
  len[R_OFFSETS] = 4ull * (p->E + 1);
  len[R_POFF] = 4ull * (p->E + 1);
  len[R_SORTED] = 4ull * p->max_rows;
  len[R_POS] = 4ull * p->max_pairs;
  len[R_TILES] = 16ull * p->max_tiles;
  len[R_NTILES] = 16;
  len[R_CHUNK] = 4ull * p->max_chunks * p->E;
  len[R_XQ] = a8 ? (uint64_t)p->max_tokens * p->Hp : (x16 || xrt ? 2ull * p->max_tokens * p->Hp : 0);
  len[R_XS] = a8 ? (uint64_t)p->max_tokens * (p->Hp / 32) : (x16 || xrt ? 4ull * p->max_tokens : 0);
  len[R_H] = (uint64_t)p->max_rows * p->Ip * (a8 ? 1 : 2);
  len[R_HS] = a8 ? (uint64_t)p->max_rows * (p->Ip / 32) : 0;
  {  // y: bf16 rows in routing order (grouped path), fp32 rows by pair id (decode path), or
     // fp32 partial rows by (pair, 32-column slice of h) (split-K decode)
    const uint64_t grouped = 2ull * p->max_rows * p->H, decode = 4ull * p->decode_max_pairs * p->H;
    const uint64_t splitk = 4ull * p->splitk_max_pairs * (p->I / 32) * ((p->H / 16 + 3) / 4 * 64 + kSplitKRowPad);
    len[R_Y] = grouped > decode ? grouped : decode;
    if (splitk > len[R_Y]) len[R_Y] = splitk;
  }
  {  // decode path: launch counter and one flag per (touched expert slot, gate/up group of 2 fragments)
    const int64_t slots = p->decode_max_pairs < p->E ? p->decode_max_pairs : p->E;
    len[R_DSYNC] = p->decode_max_pairs > 0 ? kDecodeFlagsOffset + 8ull * slots * ((p->l13.nf + 1) / 2) : 0;
  }
  uint64_t off = 0;
  for (int r = 1; r < R_COUNT_; ++r) {
    p->off[r] = off;
    p->len[r] = len[r];
    off = align_up(off + len[r], 256);
  }
  p->scratch_bytes = off;
  if (len[R_XQ] >= (uint64_t)kMaxBufferBytes || len[R_H] >= (uint64_t)kMaxBufferBytes ||
      4ull * p->splitk_max_pairs * (p->I / 32) * ((p->H / 16 + 3) / 4 * 64 + kSplitKRowPad) >= (uint64_t)kMaxBufferBytes) {
    delete p;
    return fail(B12X_ERR_UNSUPPORTED, "max_tokens too large: activation buffers would exceed 1 GiB");
  }
  *out = p;
  return B12X_OK;
}

void b12x_moe_plan_destroy(b12x_moe_plan_t plan) { delete plan; }

b12x_status b12x_moe_scratch_specs(b12x_moe_plan_t p, b12x_scratch_spec* specs, int32_t cap, int32_t* n) {
  if (!p || !n) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL argument");
  if (cap > 0 && !specs) return fail(B12X_ERR_INVALID_ARGUMENT, "specs is NULL");
  *n = 1;
  if (cap >= 1) {
    specs[0].bytes = p->scratch_bytes;
    specs[0].alignment = 256;
    specs[0].dtype = 0;
    specs[0].reserved = 0;
  }
  return B12X_OK;
}

b12x_status b12x_moe_prime(b12x_moe_plan_t p, void* scratch, uint64_t scratch_bytes, void* stream) {
  if (!p || !scratch) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL plan or scratch");
  if (!aligned(scratch, 256)) return fail(B12X_ERR_MISALIGNED, "scratch must be 256-byte aligned");
  if (scratch_bytes < p->scratch_bytes)
    return fail(B12X_ERR_SCRATCH_TOO_SMALL, "scratch %llu < %llu bytes", (unsigned long long)scratch_bytes,
                (unsigned long long)p->scratch_bytes);
  // debug aid (B12X_DEBUG_SCRATCH_FILL=1): every byte of the plan's scratch set to 0xFF before the
  // synchronization region is zeroed, so a kernel that reads scratch it has not written reads NaNs and
  // out-of-range codes instead of stale values that happen to be right
  const char* fill = getenv("B12X_DEBUG_SCRATCH_FILL");
  if (fill && fill[0] == '1') {
    const int err = launch_fill_words(scratch, p->scratch_bytes, ~0ull, (hipStream_t)stream);
    if (err) return hip_fail(err, "kernel launch");
  }
  if (!p->len[R_DSYNC]) return B12X_OK;
  const int err = launch_decode_prime((uint8_t*)scratch + p->off[R_DSYNC], p->len[R_DSYNC], (hipStream_t)stream);
  if (err) return hip_fail(err, "kernel launch");
  return B12X_OK;
}

b12x_status b12x_moe_scratch_region(b12x_moe_plan_t p, int32_t region, uint64_t* offset, uint64_t* bytes) {
  if (!p || !offset || !bytes) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL argument");
  if (region < R_COUNTS || region > R_Y || region == R_CHUNK)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown region %d", region);
  *offset = p->off[region];
  *bytes = p->len[region];
  return B12X_OK;
}

}  // extern "C"

// The binding of b12x_moe_bind; with no_scratch (the allocation-free call) the
// scratch arguments are ignored and the scratch pointers left null.
static b12x_status make_binding(b12x_moe_plan_t p, void* scratch, uint64_t scratch_bytes, bool no_scratch,
                                const b12x_moe_experts* ex, const void* a, int64_t T, int64_t a_stride,
                                const int32_t* ids, const float* tw, void* out, int64_t out_stride, BindingImpl& b,
                                const int32_t* t_live = nullptr) {
  if (!p || !ex) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL plan or experts");
  if (T < 0) return fail(B12X_ERR_INVALID_ARGUMENT, "T < 0");
  if (T > p->max_tokens)
    return fail(B12X_ERR_CAPACITY, "T = %lld exceeds max_tokens = %lld", (long long)T, (long long)p->max_tokens);
  if (memcmp(&ex->plan, &p->caps.weights, sizeof(b12x_moe_weight_plan)) != 0)
    return fail(B12X_ERR_LAYOUT_MISMATCH, "prepared weights follow a different weight plan");
  if (!ex->base || ex->bytes < ex->plan.prepared_bytes)
    return fail(B12X_ERR_LAYOUT_MISMATCH, "prepared weight buffer missing or too small");
  if (a4_nv(p->afmt) && !ex->act_scales)
    return fail(B12X_ERR_INVALID_ARGUMENT, "NVFP4 activations need the activation scales (a13_global, a2_global)");
  if (T > 0) {
    if (!a || !ids || !tw || !out || (!scratch && !no_scratch)) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL device pointer");
    if (a_stride < p->H || out_stride < p->H) return fail(B12X_ERR_INVALID_ARGUMENT, "row stride smaller than H");
    if (a_stride % 8 || out_stride % 8) return fail(B12X_ERR_MISALIGNED, "row strides must be multiples of 8");
    if (!aligned(a, 16) || !aligned(out, 16) || !aligned(ids, 16) || !aligned(tw, 16))
      return fail(B12X_ERR_MISALIGNED, "a, out, topk_ids and topk_weights must be 16-byte aligned");
    if (!no_scratch && !aligned(scratch, 256)) return fail(B12X_ERR_MISALIGNED, "scratch must be 256-byte aligned");
    if (!no_scratch && scratch_bytes < p->scratch_bytes)
      return fail(B12X_ERR_SCRATCH_TOO_SMALL, "scratch %llu < %llu bytes", (unsigned long long)scratch_bytes,
                  (unsigned long long)p->scratch_bytes);
    const char* ab = (const char*)a;
    const char* ob = (const char*)out;
    const int64_t abytes = ((T - 1) * a_stride + p->H) * 2, obytes = ((T - 1) * out_stride + p->H) * 2;
    if (ab < ob + obytes && ob < ab + abytes) return fail(B12X_ERR_INVALID_ARGUMENT, "out aliases a");
    if (abytes >= kMaxBufferBytes) return fail(B12X_ERR_UNSUPPORTED, "a spans 1 GiB or more");
  }
  memset(&b, 0, sizeof(b));
  b.magic = kBindingMagic;
  b.path = (T > 0 && T * p->k <= p->decode_max_pairs) ? 2 : 1;
  if (T > 0 && T * p->k <= p->splitk_max_pairs) b.path = 3;
  if (t_live) b.path = 4;
  // kernel resolution: a path first bound after b12x_moe_freeze is refused
  const uint32_t bit = 1u << b.path;
  if (!(p->resolved.load() & bit)) {
    if (p->frozen.load())
      return fail(B12X_ERR_FROZEN, "kernel resolution is frozen and this binding needs the %s path, not resolved before",
                  b.path == 4 ? "live-token" : b.path == 3 ? "split-K decode" : b.path == 2 ? "decode" : "grouped");
    p->resolved.fetch_or(bit);
  }
  b.t_live = t_live;
  b.splitk_max = p->splitk_max_pairs;
  b.decode_max = p->decode_max_pairs;
  b.E = p->E; b.H = p->H; b.I = p->I; b.k = p->k;
  b.gated = p->gated; b.wfmt = p->wfmt; b.afmt = p->afmt; b.act = p->act;
  b.oai = p->act == B12X_ACTIVATION_SWIGLU_OAI;
  // grouped path, NVFP4 weights: GEMM1 reads a scaled f16 copy of a (of its MXFP8 or NVFP4 round trips with
  // MXFP8 or NVFP4 activations)
  b.a_f16 = b.path == 1 && p->wfmt == B12X_WEIGHT_NVFP4;
  // test hook of the fused decode kernel's bounded waits (B12X_DEBUG_FORCE_GIVEUP=1 at bind)
  const char* fg = getenv("B12X_DEBUG_FORCE_GIVEUP");
  b.force_giveup = fg && fg[0] == '1';
  const char* tm = getenv("B12X_TIMING");
  b.timing = tm && tm[0] == '1';
  b.T = T; b.a_stride = a_stride; b.out_stride = out_stride;
  b.Hp = p->Hp; b.Ip = p->Ip; b.max_rows = p->max_rows; b.max_tiles = p->max_tiles;
  b.nf13 = p->l13.nf; b.kf13 = p->l13.kf; b.kfs13 = p->l13.kfs;
  b.nf2 = p->l2.nf; b.kf2 = p->l2.kf; b.kfs2 = p->l2.kfs;
  b.a = (const uint16_t*)a; b.ids = ids; b.tw = tw; b.out = (uint16_t*)out;
  const uint8_t* wb = (const uint8_t*)ex->base;
  const b12x_moe_weight_plan& wp = ex->plan;
  b.w13_codes = wb + wp.w13_codes_off;
  b.w13_scales = wb + wp.w13_scales_off;
  b.w2_codes = wb + wp.w2_codes_off;
  b.w2_scales = wb + wp.w2_scales_off;
  const bool nv = p->wfmt == B12X_WEIGHT_NVFP4;
  b.w13_global = nv ? (const float*)(wb + wp.w13_global_off) : nullptr;
  b.w2_global = nv ? (const float*)(wb + wp.w2_global_off) : nullptr;
  b.a13_global = a4_nv(p->afmt) ? (const float*)(wb + wp.a13_global_off) : nullptr;
  b.a2_global = a4_nv(p->afmt) ? (const float*)(wb + wp.a2_global_off) : nullptr;
  if (no_scratch) return B12X_OK;
  uint8_t* sb = (uint8_t*)scratch;
  b.counts = (int32_t*)(sb + p->off[R_COUNTS]);
  b.offsets = (int32_t*)(sb + p->off[R_OFFSETS]);
  b.poff = (int32_t*)(sb + p->off[R_POFF]);
  b.sorted = (int32_t*)(sb + p->off[R_SORTED]);
  b.pos = (int32_t*)(sb + p->off[R_POS]);
  b.tiles = (int32_t*)(sb + p->off[R_TILES]);
  b.ntiles = (int32_t*)(sb + p->off[R_NTILES]);
  b.chunk = (int32_t*)(sb + p->off[R_CHUNK]);
  b.xq = p->len[R_XQ] ? sb + p->off[R_XQ] : nullptr;
  b.xs = p->len[R_XS] ? sb + p->off[R_XS] : nullptr;
  b.h = sb + p->off[R_H];
  b.hs = p->len[R_HS] ? sb + p->off[R_HS] : nullptr;
  b.y = (float*)(sb + p->off[R_Y]);
  b.y16 = (uint16_t*)(sb + p->off[R_Y]);
  b.dsync = p->len[R_DSYNC] ? sb + p->off[R_DSYNC] : nullptr;
  return B12X_OK;
}

extern "C" {

b12x_status b12x_moe_bind(b12x_moe_plan_t p, void* scratch, uint64_t scratch_bytes, const b12x_moe_experts* ex,
                          const void* a, int64_t T, int64_t a_stride, const int32_t* ids, const float* tw, void* out,
                          int64_t out_stride, b12x_moe_binding* binding) {
  if (!binding) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL binding");
  BindingImpl b;
  const b12x_status st = make_binding(p, scratch, scratch_bytes, false, ex, a, T, a_stride, ids, tw, out, out_stride, b);
  if (st) return st;
  memset(binding, 0, sizeof(*binding));
  memcpy(binding, &b, sizeof(b));
  return B12X_OK;
}

b12x_status b12x_moe_bind_live(b12x_moe_plan_t p, void* scratch, uint64_t scratch_bytes, const b12x_moe_experts* ex,
                               const void* a, int64_t a_stride, const int32_t* ids, const float* tw, void* out,
                               int64_t out_stride, const int32_t* t_live, b12x_moe_binding* binding) {
  if (!binding) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL binding");
  if (!p) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL plan");
  if (!t_live) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL live token count");
  if (!aligned(t_live, 4)) return fail(B12X_ERR_MISALIGNED, "the live token count must be 4-byte aligned");
  if (p->max_tokens < 1) return fail(B12X_ERR_CAPACITY, "a live binding needs max_tokens >= 1");
  BindingImpl b;
  const b12x_status st = make_binding(p, scratch, scratch_bytes, false, ex, a, p->max_tokens, a_stride, ids, tw, out,
                                      out_stride, b, t_live);
  if (st) return st;
  memset(binding, 0, sizeof(*binding));
  memcpy(binding, &b, sizeof(b));
  return B12X_OK;
}

b12x_status b12x_moe_freeze(b12x_moe_plan_t p) {
  if (!p) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL plan");
  p->frozen.store(1);
  return B12X_OK;
}

static b12x_status get_binding(const b12x_moe_binding* binding, BindingImpl* b) {
  if (!binding) return fail(B12X_ERR_INVALID_ARGUMENT, "binding is NULL");
  memcpy(b, binding, sizeof(*b));
  if (b->magic != kBindingMagic) return fail(B12X_ERR_INVALID_ARGUMENT, "not a binding from b12x_moe_bind");
  return B12X_OK;
}

static bool stage_in_path(const BindingImpl& b, int stage) {
  if (b.path == 4) return false;  // a live binding runs whole calls only
  if (b.path == 3) return stage == B12X_STAGE_DECODE1 || stage == B12X_STAGE_COMBINE;
  if (stage == B12X_STAGE_QUANT_X) return b.afmt != B12X_ACT_BF16 || b.a_f16;
  if (b.path == 2)
    return stage == B12X_STAGE_DECODE1 || stage == B12X_STAGE_COMBINE ||
           (stage == B12X_STAGE_DECODE2 && !decode_fused(b));
  return stage >= B12X_STAGE_ROUTE && stage <= B12X_STAGE_COMBINE;
}

static b12x_status run_stage(const BindingImpl& b, int stage, hipStream_t s) {
  if (stage < B12X_STAGE_ROUTE || stage > B12X_STAGE_DECODE2)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown stage %d", stage);
  if (!stage_in_path(b, stage))
    return fail(B12X_ERR_UNSUPPORTED, "stage %d is not part of this binding's path (%s)", stage,
                b.path == 3 ? "split-K decode" : b.path == 2 ? "decode" : "grouped");
  int err = 0;
  switch (stage) {
    case B12X_STAGE_ROUTE: err = launch_route(b, s); break;
    case B12X_STAGE_QUANT_X:
      if (a4_nv(b.afmt))  // exact NVFP4 round trips: f16 (grouped path, row exponents 0) or bf16
        err = launch_nv_roundtrip_rows(b.a, b.live(), b.H, b.a_stride, b.a13_global, (uint16_t*)b.xq, b.Hp,
                                       (int32_t*)b.xs, b.a_f16, s);
      else if (b.a_f16)
        err = launch_f16_rows(b.a, b.live(), b.H, b.a_stride, (uint16_t*)b.xq, b.Hp, (int32_t*)b.xs,
                              a8_bf16(b.wfmt, b.afmt), s);
      else if (a8_bf16(b.wfmt, b.afmt))
        err = launch_mx_roundtrip_rows(b.a, b.live(), b.H, b.a_stride, (uint16_t*)b.xq, b.Hp, s);
      else err = launch_quant_rows(b.a, b.live(), b.H, b.a_stride, b.xq, b.Hp, b.xs, b.Hp / 32, s);
      break;
    case B12X_STAGE_GEMM1: err = launch_gemm1(b, s); break;
    case B12X_STAGE_GEMM2: err = launch_gemm2(b, s); break;
    case B12X_STAGE_COMBINE:
      err = b.path == 3 ? launch_decode_sk_combine(b, s) : b.path == 2 ? launch_decode_combine(b, s) : launch_combine(b, s);
      break;
    case B12X_STAGE_DECODE1: err = b.path == 3 ? launch_decode_sk(b, s) : launch_decode1(b, s); break;
    case B12X_STAGE_DECODE2: err = launch_decode2(b, s); break;
  }
  if (err) return hip_fail(err, "kernel launch");
  return B12X_OK;
}

b12x_status b12x_moe_run_stage(const b12x_moe_binding* binding, int32_t stage, void* stream) {
  BindingImpl b;
  b12x_status st = get_binding(binding, &b);
  if (st) return st;
  if (b.T == 0) return B12X_OK;
  return run_stage(b, stage, (hipStream_t)stream);
}

// A live binding: each path the plan has, launched for the token counts it
// serves, as a copy of the binding whose T is the largest such count; the
// kernels of every path but the one that serves the live count return at once.
static b12x_status run_path(const BindingImpl& b, hipStream_t s);
static b12x_status run_live(const BindingImpl& b, hipStream_t s) {
  const int64_t cap = b.T, k = b.k;
  const int32_t sk = b.splitk_max, dm = b.decode_max;
  struct Leg {
    int path;
    int32_t lo, hi;
  };
  const Leg legs[3] = {{3, 0, sk}, {2, sk, dm}, {1, std::max(sk, dm), INT32_MAX}};
  for (const Leg& l : legs) {
    if (l.hi <= l.lo) continue;
    const int64_t tcap = l.path == 1 ? cap : std::min<int64_t>(cap, l.hi / k);
    if (tcap < 1 || tcap * k <= l.lo) continue;  // no token count reaches this path
    BindingImpl r = b;
    r.path = l.path;
    r.T = tcap;
    r.rlo = l.lo;
    r.rhi = l.hi;
    r.a_f16 = l.path == 1 && b.wfmt == B12X_WEIGHT_NVFP4;
    const b12x_status st = run_path(r, s);
    if (st) return st;
  }
  return B12X_OK;
}

b12x_status b12x_moe_run(const b12x_moe_binding* binding, void* stream) {
  BindingImpl b;
  b12x_status st = get_binding(binding, &b);
  if (st) return st;
  if (b.T == 0) return B12X_OK;
  hipStream_t s = (hipStream_t)stream;
  if (b.path == 4) return run_live(b, s);
  return run_path(b, s);
}

static const char* stage_name(int stage) {
  switch (stage) {
    case B12X_STAGE_ROUTE: return "route";
    case B12X_STAGE_QUANT_X: return "quant_x";
    case B12X_STAGE_GEMM1: return "gemm1";
    case B12X_STAGE_GEMM2: return "gemm2";
    case B12X_STAGE_COMBINE: return "combine";
    case B12X_STAGE_DECODE1: return "decode1";
    case B12X_STAGE_DECODE2: return "decode2";
  }
  return "?";
}

static b12x_status run_path(const BindingImpl& b, hipStream_t s) {
  b12x_status st = B12X_OK;
  static const int grouped[5] = {B12X_STAGE_ROUTE, B12X_STAGE_QUANT_X, B12X_STAGE_GEMM1, B12X_STAGE_GEMM2,
                                 B12X_STAGE_COMBINE};
  static const int decode[4] = {B12X_STAGE_QUANT_X, B12X_STAGE_DECODE1, B12X_STAGE_DECODE2, B12X_STAGE_COMBINE};
  const int* stages = b.path == 1 ? grouped : decode;
  const int n = b.path == 1 ? 5 : 4;
  // debug aid (B12X_TIMING=1 at bind): an event before and after every stage, then one line per stage on
  // stderr; the call waits for its kernels.  Skipped while the stream is being captured.
  const bool timed = b.timing && !stream_capturing(s);
  void* marks[6] = {};
  int ran[5] = {};
  int m = 0;
  if (timed) marks[m] = timing_mark(s);
  for (int i = 0; i < n; ++i) {
    if (!stage_in_path(b, stages[i])) continue;
    st = run_stage(b, stages[i], s);
    if (st) break;
    if (timed) {
      ran[m] = stages[i];
      marks[++m] = timing_mark(s);
    }
  }
  if (timed) {
    for (int i = 0; i < m && !st; ++i)
      fprintf(stderr, "b12x_moe_run: path %d T %lld %-8s %9.2f us\n", b.path, (long long)b.T, stage_name(ran[i]),
              1e3 * timing_ms(marks[i], marks[i + 1]));
    for (int i = 0; i <= m; ++i) timing_free(marks[i]);
  }
  return st;
}

b12x_status b12x_moe_run_noalloc(b12x_moe_plan_t p, const b12x_moe_experts* ex, const void* a, int64_t T,
                                 int64_t a_stride, const int32_t* ids, const float* tw, void* out, int64_t out_stride,
                                 void* stream) {
  BindingImpl b;
  b12x_status st = make_binding(p, nullptr, 0, true, ex, a, T, a_stride, ids, tw, out, out_stride, b);
  if (st) return st;
  if (T == 0) return B12X_OK;
  if (b.path != 3)
    return fail(B12X_ERR_UNSUPPORTED,
                "b12x_moe_run_noalloc runs the split-K decode path only: T * top_k = %lld is above the plan's "
                "split-K limit (%d pairs) or H = %d above %d",
                (long long)(T * p->k), p->splitk_max_pairs, p->H, kSplitKMaxH);
  const uint64_t need = sk_partial_bytes(b);
  if (need > (uint64_t)B12X_NOALLOC_SCRATCH_BYTES)
    return fail(B12X_ERR_CAPACITY, "the partial rows need %llu bytes, more than the static scratch (%llu bytes)",
                (unsigned long long)need, (unsigned long long)B12X_NOALLOC_SCRATCH_BYTES);
  void* ptr = nullptr;
  const int err = sk_static_scratch(&ptr);
  if (err) return hip_fail(err, "hipGetSymbolAddress of the static scratch");
  b.y = (float*)ptr;
  b.y16 = (uint16_t*)ptr;
  hipStream_t s = (hipStream_t)stream;
  st = run_stage(b, B12X_STAGE_DECODE1, s);
  if (st) return st;
  return run_stage(b, B12X_STAGE_COMBINE, s);
}

b12x_status b12x_moe_binding_query(const b12x_moe_binding* binding, int32_t what, int64_t* value) {
  BindingImpl b;
  b12x_status st = get_binding(binding, &b);
  if (st) return st;
  if (!value) return fail(B12X_ERR_INVALID_ARGUMENT, "value is NULL");
  switch (what) {
    case B12X_QUERY_PATH: *value = b.path; break;
    case B12X_QUERY_TILE_ROWS: *value = kTileRows; break;
    case B12X_QUERY_ROW_PAD: *value = kRowPad; break;
    case B12X_QUERY_T: *value = b.T; break;
    case B12X_QUERY_NUM_STAGES:
      *value = b.path == 4 ? 0  // a live binding has no stages of its own
               : b.path == 3 ? 2
                             : (b.path == 2 ? (decode_fused(b) ? 2 : 3) : 4) + (stage_in_path(b, B12X_STAGE_QUANT_X) ? 1 : 0);
      break;
    default: return fail(B12X_ERR_INVALID_ARGUMENT, "unknown query %d", what);
  }
  return B12X_OK;
}

b12x_status b12x_mxfp8_quantize_rows(const void* x, int64_t rows, int64_t cols, int64_t stride, uint8_t* codes,
                                     uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0) return fail(B12X_ERR_INVALID_ARGUMENT, "negative size");
  if (cols % 32) return fail(B12X_ERR_UNSUPPORTED, "cols (%lld) must be a multiple of 32", (long long)cols);
  if (rows == 0 || cols == 0) return B12X_OK;
  if (!x || !codes || !scales) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (stride < cols) return fail(B12X_ERR_INVALID_ARGUMENT, "stride smaller than cols");
  if (stride % 8 || !aligned(x, 16) || !aligned(codes, 16))
    return fail(B12X_ERR_MISALIGNED, "x, codes and the row stride must be 16-byte aligned");
  int err = launch_quant_rows((const uint16_t*)x, LiveT{nullptr, rows, 1, 0, 0}, cols, stride, codes, cols, scales, cols / 32,
                              (hipStream_t)stream);
  if (err) return hip_fail(err, "quantize rows");
  return B12X_OK;
}

static b12x_status dense_layout(int32_t n, int32_t k, int32_t weight_format, MatrixLayout* l) {
  if (weight_format != B12X_WEIGHT_MXFP4 && weight_format != B12X_WEIGHT_NVFP4)
    return fail(B12X_ERR_INVALID_ARGUMENT, "unknown weight format %d", weight_format);
  if (n < 16 || k < 32) return fail(B12X_ERR_INVALID_ARGUMENT, "n must be >= 16 and k >= 32");
  if (n % 16 || k % 32) return fail(B12X_ERR_UNSUPPORTED, "n (%d) must be a multiple of 16 and k (%d) of 32", n, k);
  *l = make_matrix_layout(n, k, weight_format);
  if (l->codes_per_expert >= (uint64_t)kMaxBufferBytes || l->scales_per_expert >= (uint64_t)kMaxBufferBytes)
    return fail(B12X_ERR_UNSUPPORTED, "packed weight reaches 1 GiB");
  return B12X_OK;
}

b12x_status b12x_gemm_packed_bytes(int32_t n, int32_t k, int32_t weight_format, uint64_t* bytes) {
  if (!bytes) return fail(B12X_ERR_INVALID_ARGUMENT, "bytes is NULL");
  MatrixLayout l;
  b12x_status st = dense_layout(n, k, weight_format, &l);
  if (st) return st;
  *bytes = dense_scales_offset(l) + l.scales_per_expert;
  return B12X_OK;
}

b12x_status b12x_gemm_pack_weight(int32_t n, int32_t k, int32_t weight_format, const void* codes, const void* scales,
                                  void* dst, uint64_t dst_bytes, void* stream) {
  MatrixLayout l;
  b12x_status st = dense_layout(n, k, weight_format, &l);
  if (st) return st;
  if (!codes || !scales || !dst) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL device pointer");
  const uint64_t need = dense_scales_offset(l) + l.scales_per_expert;
  if (dst_bytes < need)
    return fail(B12X_ERR_SCRATCH_TOO_SMALL, "packed weight buffer %llu < %llu bytes", (unsigned long long)dst_bytes,
                (unsigned long long)need);
  if (!aligned(codes, 16) || !aligned(dst, 256))
    return fail(B12X_ERR_MISALIGNED, "codes must be 16-byte aligned and dst 256-byte aligned");
  PackArgs a;
  a.src_codes = (const uint8_t*)codes;
  a.src_scales = (const uint8_t*)scales;
  a.dst_codes = (uint8_t*)dst;
  a.dst_scales = (uint8_t*)dst + dense_scales_offset(l);
  a.E = 1;
  a.l = l;
  a.wfmt = weight_format;
  a.gated_interleave = 0;
  const int err = launch_pack(a, (hipStream_t)stream);
  if (err) return hip_fail(err, "pack weight");
  return B12X_OK;
}

b12x_status b12x_gemm_mm(const void* x, int64_t m, int64_t x_stride, const void* w_packed, int32_t n, int32_t k,
                         int32_t weight_format, const float* global_scale, void* out, int64_t out_stride,
                         void* stream) {
  MatrixLayout l;
  b12x_status st = dense_layout(n, k, weight_format, &l);
  if (st) return st;
  if (m < 0) return fail(B12X_ERR_INVALID_ARGUMENT, "m must be >= 0");
  if (m == 0) return B12X_OK;
  if (!x || !w_packed || !out) return fail(B12X_ERR_INVALID_ARGUMENT, "NULL device pointer");
  if (weight_format == B12X_WEIGHT_NVFP4 && !global_scale)
    return fail(B12X_ERR_INVALID_ARGUMENT, "NVFP4 weights need their fp32 tensor scale");
  if (x_stride < k || out_stride < n) return fail(B12X_ERR_INVALID_ARGUMENT, "row strides smaller than k or n");
  if (!aligned(x, 16) || x_stride % 8 || !aligned(w_packed, 256) || !aligned(out, 2))
    return fail(B12X_ERR_MISALIGNED, "x and its row stride must be 16-byte aligned, the packed weight 256-byte");
  if (m >= INT32_MAX / 2 || (uint64_t)m * (uint64_t)x_stride * 2 >= (uint64_t)kMaxBufferBytes)
    return fail(B12X_ERR_UNSUPPORTED, "the rows of x span 1 GiB or more");
  const int err = launch_dense_mm((const uint16_t*)x, m, x_stride, (const uint8_t*)w_packed, l, weight_format,
                                  weight_format == B12X_WEIGHT_NVFP4 ? global_scale : nullptr, (uint16_t*)out,
                                  out_stride, (hipStream_t)stream);
  if (err) return hip_fail(err, "dense mm");
  return B12X_OK;
}

}  // extern "C"
