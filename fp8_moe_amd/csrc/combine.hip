// Deterministic top-k-weighted combine (both paths) (b12x README "What's in here": the
// fused routed-expert FFN; the combine weights are the caller's
// topk_weights).  out[t] = sum over slots j = 0..k-1 in ascending order of
// w[t, j] * y[pos[t*k + j]], accumulated in fp32 and rounded once to bf16
// (nearest even).  The grouped path stages y as bf16 rows, the decode path as
// fp32 rows.  A gather, not a scatter: no atomics, so the result does
// not depend on scheduling.  A dropped pair (pos = -1) contributes nothing.
#include "device_common.h"

namespace b12x {

// One thread per 8 output columns of one token.  The slots are taken 8 at a
// time: their rows and weights, then all their y loads (a dropped pair loads
// row 0 and is masked), then the sums in slot order, so the loads of a chunk
// are in flight together.
// Eight consecutive y values of one row, widened to fp32.
__device__ __forceinline__ void load_y8(const float* y, float4& a, float4& b) {
  a = ((const float4*)y)[0];
  b = ((const float4*)y)[1];
}
__device__ __forceinline__ void load_y8(const uint16_t* y, float4& a, float4& b) {
  const uint4 v = *(const uint4*)y;
  a = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u), __uint_as_float(v.y << 16),
                  __uint_as_float(v.y & 0xFFFF0000u));
  b = make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u), __uint_as_float(v.w << 16),
                  __uint_as_float(v.w & 0xFFFF0000u));
}

template <typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT* __restrict__ y, int64_t y_stride,
                                                       const int32_t* __restrict__ pos,
                                                       const int32_t* __restrict__ ids, int E,
                                                       const float* __restrict__ tw, LiveT lv, int k, int H,
                                                       int64_t max_rows, uint16_t* __restrict__ out,
                                                       int64_t out_stride, const uint64_t* counter) {
  constexpr int kChunk = 8;
  const int64_t groups = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t T = lv.tokens();
  if (!lv.on() || idx >= T * groups) return;
  // After a fused decode launch the launch counter is a multiple of kLaunchStep.
  // The output is NaN, not stale, if it is not: a scratch never primed, whose
  // launches' workgroups may not share one tag.
  bool failed = false;
  if (counter) {
    const uint64_t c = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    failed = (c & (kLaunchStep - 1)) != 0;
  }
  const int64_t t = idx / groups, c = (idx % groups) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // grouped path: pos gives the y row; decode path: the row is the pair id
  // itself, so its y loads do not wait for the ids (which only mask them)
  const int32_t* key = pos ? pos : ids;
  for (int j0 = 0; j0 < k; j0 += kChunk) {
    int raw[kChunk], row[kChunk];
    float w[kChunk];
    float4 a[kChunk], b[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {  // clamped slot: every load is in bounds and unconditional
      const int j = min(j0 + u, k - 1);
      raw[u] = key[t * k + j];
      w[u] = tw[t * k + j];
      if (!pos) load_y8(y + (t * k + j) * y_stride + c, a[u], b[u]);  // row t*k + j < T*k <= max_rows
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int j = j0 + u;
      int r;
      if (pos) r = raw[u];
      else r = (raw[u] >= 0 && raw[u] < E) ? (int)(t * k + j) : -1;  // a dropped pair has no row
      row[u] = (j < k && r >= 0 && r < max_rows) ? r : -1;
    }
    if (pos) {
#pragma unroll
      for (int u = 0; u < kChunk; ++u) load_y8(y + (int64_t)(row[u] < 0 ? 0 : row[u]) * y_stride + c, a[u], b[u]);
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (row[u] < 0) continue;
      acc[0] = fmaf(w[u], a[u].x, acc[0]); acc[1] = fmaf(w[u], a[u].y, acc[1]);
      acc[2] = fmaf(w[u], a[u].z, acc[2]); acc[3] = fmaf(w[u], a[u].w, acc[3]);
      acc[4] = fmaf(w[u], b[u].x, acc[4]); acc[5] = fmaf(w[u], b[u].y, acc[5]);
      acc[6] = fmaf(w[u], b[u].z, acc[6]); acc[7] = fmaf(w[u], b[u].w, acc[7]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = failed ? 0x7FC07FC0u : bf16_rne(acc[2 * i]) | (bf16_rne(acc[2 * i + 1]) << 16);
  *(uint4*)(out + t * out_stride + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

template <typename YT>
static int launch_combine_rows(const BindingImpl& b, const YT* y, const int32_t* pos, const uint64_t* counter,
                               hipStream_t s) {
  const int64_t total = b.T * (b.H / 8);
  if (total == 0) return 0;
  hipLaunchKernelGGL(combine_kernel<YT>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, y, (int64_t)b.H,
                     pos, b.ids, b.E, b.tw, b.live(), b.k, b.H, b.max_rows, b.out, b.out_stride, counter);
  return (int)hipGetLastError();
}

// grouped path: bf16 y rows in routing order, located through pos
int launch_combine(const BindingImpl& b, hipStream_t s) {
  return launch_combine_rows(b, (const uint16_t*)b.y16, b.pos, nullptr, s);
}

// decode path: fp32 y rows indexed by pair id
int launch_decode_combine(const BindingImpl& b, hipStream_t s) {
  if (!decode_fused(b)) return launch_combine_rows(b, (const float*)b.y, nullptr, nullptr, s);
  return launch_combine_rows(b, (const float*)b.y, nullptr, (const uint64_t*)(b.dsync + kDecodeCounterOffset), s);
}

}  // namespace b12x
