// Internal structures shared by the host runtime (api.cpp) and the kernels.
// Not part of the C ABI.
#pragma once

#include <atomic>
#include <stddef.h>
#include <stdint.h>

#include "../../include/b12x_moe.h"

typedef struct ihipStream_t* hipStream_t;

namespace b12x {

// ---- prepared weight layout -------------------------------------------------
// A matrix with N output rows and K contraction elements is stored as
// fragments of 16 rows x 128 K.  Fragment (f, kf) is 1024 bytes: lane l
// (0..63) owns 16 bytes = the 32 FP4 codes of row (f*16 + l%16) at
// K = 128*kf + 32*(l/16) + [0, 32), low nibble first.  That is exactly the
// fp4 operand of one 16x16x128 scaled MFMA, and, read as four dwords, four
// bf16 MFMA (16x16x32) operands once the K order inside a fragment is taken
// as (lane group, dword) on both operands.  K beyond the matrix is zero.
// Scales: one dword per lane and fragment group; MXFP4 packs the E8M0 codes
// of 4 consecutive fragments (byte j = fragment 4q+j), NVFP4 the two E4M3
// codes (the lane's two 16-element halves) of 2 consecutive fragments
// (bytes 2j, 2j+1 = fragment 2q+j).  Gated w13 interleaves 16-row blocks:
// fragment 2j = gate rows [16j, 16j+16), fragment 2j+1 = up rows of the same
// h columns, so a gate/up pair always sits in one lane.
constexpr int kFragK = 128;
constexpr int kFragN = 16;
constexpr int kFragBytes = 1024;
constexpr int kScaleGroupBytes = 256;
constexpr uint32_t kLayoutId = 0x4d4f4501u;  // "MOE", version 1

// ---- grouped path ------------------------------------------------------------
constexpr int kTileRows = 128;   // most rows per GEMM tile (multiple of kRowPad)
constexpr int kRowPad = 16;      // per-expert row padding = MFMA row block
constexpr int kRouteChunk = 1024;  // routing pairs per workgroup
constexpr int kMaxExperts = 1024;
// ---- decode path -------------------------------------------------------------
constexpr int kDecodePairs = 256;     // T*k at or below which the decode path runs
constexpr int kSplitKPairs = 32;      // T*k at or below which the split-K decode kernel runs (default)
constexpr int kSplitKMaxPairs = 64;   // its routing holds one pair per lane of a wave
constexpr int kSplitKRowPad = 64;     // floats between its partial rows beyond H
constexpr int kSplitKMaxH = 4096;     // its W2 slice (H / 16 fragments x 320 bytes) is staged in LDS
// MXFP8 activations: with MXFP4 weights the scaled fp8 x fp4 MFMA multiplies
// the codes (native); with NVFP4 weights (whose E4M3 block scales per 16 have
// no place in that MFMA) x and h are round-tripped through MXFP8 and the
// exact bf16 values multiply the NVFP4 weights on the bf16 MFMA.
inline bool a8_native(int wfmt, int afmt) { return afmt == B12X_ACT_MXFP8 && wfmt == B12X_WEIGHT_MXFP4; }
inline bool a8_bf16(int wfmt, int afmt) { return afmt == B12X_ACT_MXFP8 && wfmt == B12X_WEIGHT_NVFP4; }
// NVFP4 activations (NVFP4 weights only): operands are the exact NVFP4 round trips
inline bool a4_nv(int afmt) { return afmt == B12X_ACT_NVFP4; }
// decode synchronization region: a uint64 launch counter, then (from byte 64)
// one uint64 completion flag per (touched expert slot, gate/up group of 2
// fragments).  b12x_moe_prime zeroes it once per scratch.
constexpr int kDecodeCounterOffset = 0;  // uint64: kLaunchStep per completed fused launch
constexpr int kDecodeFlagsOffset = 64;   // uint64 per (expert slot, gate/up group): the tag once its h is stored
// Every fused launch adds exactly kLaunchStep to the counter, split over its
// workgroups (each adds its share when done), so between launches the
// counter is n * kLaunchStep after n launches and every workgroup of launch
// n reads a value in [n, n + 1) * kLaunchStep whenever it starts: launch n's
// tag is decode_tag(n).  A grid holds at most kLaunchStep workgroups.
constexpr int kLaunchShift = 16;
constexpr uint64_t kLaunchStep = 1ull << kLaunchShift;
// Tag of fused launch number e: never 0 (so zeroed memory never matches) and
// different for every launch.
constexpr uint32_t kDecodeTagMagic = 0xB12DF1A9u;
__host__ __device__ inline uint64_t decode_tag(uint32_t e) { return ((uint64_t)e << 32) | kDecodeTagMagic; }
// Kernels address each activation buffer and each expert's weights with
// 32-bit buffer offsets; buffers are limited to 1 GiB (so that the sum of
// two out-of-range markers is still out of range).
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 30;
constexpr int kDecodeMaxKPerWave = 8; // K fragments per wave: K <= 4 * 8 * 128

struct MatrixLayout {
  int64_t n = 0, k = 0;     // logical rows / contraction length
  int64_t nf = 0, kf = 0;   // n/16, ceil(k/128)
  int64_t kfs = 0;          // scale dword groups per fragment row
  uint64_t codes_per_expert = 0, scales_per_expert = 0;  // bytes
};

inline MatrixLayout make_matrix_layout(int64_t n, int64_t k, int wfmt) {
  MatrixLayout m;
  m.n = n;
  m.k = k;
  m.nf = n / kFragN;
  m.kf = (k + kFragK - 1) / kFragK;
  m.kfs = wfmt == B12X_WEIGHT_MXFP4 ? (m.kf + 3) / 4 : (m.kf + 1) / 2;
  m.codes_per_expert = (uint64_t)(m.nf * m.kf) * kFragBytes;
  m.scales_per_expert = (uint64_t)(m.nf * m.kfs) * kScaleGroupBytes;
  return m;
}

struct PlanImpl {
  b12x_moe_caps caps;
  int E = 0, H = 0, I = 0, k = 0;
  int gated = 0, wfmt = 0, afmt = 0, act = 0;
  int64_t max_tokens = 0;
  MatrixLayout l13, l2;
  int64_t Hp = 0, Ip = 0;  // H, I rounded up to 128
  int64_t max_pairs = 0, max_rows = 0, max_tiles = 0, max_chunks = 0;
  int decode_max_pairs = 0;  // largest T*k that takes the decode path (0: never)
  int splitk_max_pairs = 0;  // largest T*k that takes the split-K decode kernel (0: never)
  uint64_t off[16] = {0};   // scratch region offsets, indexed by Region
  uint64_t len[16] = {0};   // scratch region sizes
  uint64_t scratch_bytes = 0;
  // kernel resolution (b12x_moe_freeze): bit `path` set once a binding of
  // that path (1 grouped, 2 decode, 3 split-K decode, 4 live token count) was
  // made; once frozen, a binding of a path not set is refused
  std::atomic<uint32_t> resolved{0};
  std::atomic<int> frozen{0};
};

enum Region {
  R_COUNTS = 1, R_OFFSETS = 2, R_POFF = 3, R_SORTED = 4, R_POS = 5, R_TILES = 6, R_NTILES = 7,
  R_CHUNK = 8, R_XQ = 9, R_XS = 10, R_H = 11, R_HS = 12, R_Y = 13, R_DSYNC = 14, R_COUNT_ = 15
};

// Token count of a launch.  An ordinary binding passes t = nullptr and its
// own T as cap.  A binding bound at capacity for a live token count
// (b12x_moe_bind_live) passes the device int32 t, read by the kernel at run
// time, the largest T this launch's path can serve as cap (its grids and
// buffers are sized for it), and the pair counts the path serves: the kernel
// works only while t is in [0, cap] and lo < t * k <= hi (each path of such a
// binding is launched, and all but the one serving t return at once).
struct LiveT {
  const int32_t* t;
  int64_t cap;
  int32_t k, lo, hi;
  __host__ __device__ int64_t tokens() const {
    if (!t) return cap;
    const int64_t v = *t;
    return v < 0 ? 0 : (v > cap ? cap : v);
  }
  __host__ __device__ bool on() const {
    if (!t) return true;
    const int64_t v = *t;
    return v >= 0 && v <= cap && v * k > lo && v * k <= hi;
  }
};

// Everything a run needs, resolved at bind time (trivially copyable).
struct BindingImpl {
  uint32_t magic;
  int32_t path;  // 1 grouped, 2 decode (two-phase), 3 decode (split-K), 4 live token count (all three)
  int32_t E, H, I, k, gated, wfmt, afmt, act;
  int32_t oai;  // gated with SwiGLU-OAI instead of SiLU
  int32_t a_f16;  // grouped path, NVFP4 weights: GEMM1 reads a scaled f16 copy of a (xq; of its MXFP8 round trips
                  // with MXFP8 activations) and row exponents (xs)
  int32_t force_giveup;  // test hook (fused decode kernel): its waits expect a tag no one writes and run out
  int32_t timing;        // B12X_TIMING=1 at bind: run() times each stage and prints the times
  int64_t T, a_stride, out_stride;
  int64_t Hp, Ip, max_rows, max_tiles;
  int64_t nf13, kf13, kfs13, nf2, kf2, kfs2;
  const uint16_t* a;
  const int32_t* ids;
  const float* tw;
  uint16_t* out;
  const uint8_t* w13_codes;
  const uint8_t* w13_scales;
  const float* w13_global;
  const uint8_t* w2_codes;
  const uint8_t* w2_scales;
  const float* w2_global;
  const float* a13_global;  // NVFP4 activations: scale of x [1] and of each expert's h [E]
  const float* a2_global;
  int32_t* counts;
  int32_t* offsets;
  int32_t* poff;
  int32_t* sorted;
  int32_t* pos;
  int32_t* tiles;
  int32_t* ntiles;
  int32_t* chunk;
  uint8_t* xq;
  uint8_t* xs;
  void* h;
  uint8_t* hs;
  float* y;        // decode path: fp32 rows, one per pair id
  uint16_t* y16;   // grouped path: bf16 rows in routing order (same memory as y)
  uint8_t* dsync;  // decode path: launch counter, status and the fused kernel's completion flags
  // live token count (b12x_moe_bind_live; null otherwise).  Such a binding
  // holds its capacity in T; run() launches each path with a copy whose T is
  // the largest that path serves and (rlo, rhi] its pair counts.
  const int32_t* t_live;
  int32_t rlo, rhi;
  int32_t splitk_max, decode_max;  // the plan's path limits (pairs)
  LiveT live() const { return LiveT{t_live, T, k, rlo, rhi}; }
};
constexpr uint32_t kBindingMagic = 0xb12b1d01u;
static_assert(sizeof(BindingImpl) <= sizeof(b12x_moe_binding), "binding does not fit the ABI struct");

// ---- kernel launchers (kernels/*.hip); return hipError_t as int ----------------
struct PackArgs {
  const uint8_t* src_codes;
  const uint8_t* src_scales;
  uint8_t* dst_codes;
  uint8_t* dst_scales;
  int E;
  MatrixLayout l;
  int wfmt;
  int gated_interleave;  // 1: rows are [gate; up] halves to interleave per 16
};
int launch_pack(const PackArgs& a, hipStream_t s);
int launch_copy_f32(const float* src, float* dst, int n, hipStream_t s);
int launch_route(const BindingImpl& b, hipStream_t s);
int launch_quant_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint8_t* codes,
                      int64_t code_stride, uint8_t* scales, int64_t scale_stride, hipStream_t s);
int launch_mx_roundtrip_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint16_t* out,
                             int64_t out_stride, hipStream_t s);
int launch_nv_roundtrip_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, const float* g,
                             uint16_t* out, int64_t out_stride, int32_t* exps, bool f16, hipStream_t s);
int launch_f16_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint16_t* out,
                    int64_t out_stride, int32_t* exps, bool rt, hipStream_t s);
int launch_gemm1(const BindingImpl& b, hipStream_t s);
int launch_gemm2(const BindingImpl& b, hipStream_t s);
int launch_combine(const BindingImpl& b, hipStream_t s);
// dense block-scaled GEMM: packed weight = codes, then scales at this offset
inline uint64_t dense_scales_offset(const MatrixLayout& l) { return (l.codes_per_expert + 255) / 256 * 256; }
int launch_dense_mm(const uint16_t* x, int64_t m, int64_t x_stride, const uint8_t* w, const MatrixLayout& l,
                    int wfmt, const float* global_scale, uint16_t* out, int64_t out_stride, hipStream_t s);
// compute units of the current device (cached per device)
int device_cu_count();
int launch_decode1(const BindingImpl& b, hipStream_t s);
int launch_decode2(const BindingImpl& b, hipStream_t s);
int launch_decode_combine(const BindingImpl& b, hipStream_t s);
// split-K decode (path 3): one kernel for gate/up + activation + partial down
// projections per 32-column slice of h, then the combine of the partials
int launch_decode_prime(uint8_t* dsync, uint64_t bytes, hipStream_t s);  // zero the decode synchronization region
// debug aids (debug.hip)
int launch_fill_words(void* p, uint64_t bytes, uint64_t value, hipStream_t s);
bool stream_capturing(hipStream_t s);
void* timing_mark(hipStream_t s);     // a new event recorded on s, or null
double timing_ms(void* a, void* b);   // waits for b; milliseconds from a to b (< 0 on failure)
void timing_free(void* e);
int launch_decode_sk(const BindingImpl& b, hipStream_t s);
int launch_decode_sk_combine(const BindingImpl& b, hipStream_t s);
// Bytes of the split-K partial rows of a binding (its whole use of scratch).
uint64_t sk_partial_bytes(const BindingImpl& b);
// Device address of the static scratch array of the allocation-free call on the
// current device (looked up once per device); 0 or the HIP error code.
int sk_static_scratch(void** ptr);
// the decode path runs gate/up and down as one launch (DECODE1) for this binding
bool decode_fused(const BindingImpl& b);
const char* hip_error_name(int err);

}  // namespace b12x

// The opaque plan handle of the C ABI.
struct b12x_moe_plan_impl : b12x::PlanImpl {};
