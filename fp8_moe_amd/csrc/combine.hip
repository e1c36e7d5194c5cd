// Deterministic top-k-weighted combine (both paths) (b12x README "What's in here": the
// fused routed-expert FFN; the combine weights are the caller's
// topk_weights).  out[t] = sum over slots j = 0..k-1 in ascending order of
// w[t, j] * y[pos[t*k + j]], accumulated in fp32 and rounded once to bf16
// (nearest even).  A gather, not a scatter: no atomics, so the result does
// not depend on scheduling.  A dropped pair (pos = -1) contributes nothing.
#include "device_common.h"

namespace b12x {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y, int64_t y_stride,
                                                       const int32_t* __restrict__ pos,
                                                       const int32_t* __restrict__ ids, int E,
                                                       const float* __restrict__ tw, int64_t T, int k, int H,
                                                       int64_t max_rows, uint16_t* __restrict__ out,
                                                       int64_t out_stride) {
  const int64_t groups = H / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * groups) return;
  const int64_t t = idx / groups, c = (idx % groups) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    int row;
    if (pos) {
      row = pos[t * k + j];
    } else {  // rows indexed by pair id; a dropped pair has no row
      const int e = ids[t * k + j];
      row = (e >= 0 && e < E) ? (int)(t * k + j) : -1;
    }
    if (row < 0 || row >= max_rows) continue;
    const float w = tw[t * k + j];
    const float4* src = (const float4*)(y + (int64_t)row * y_stride + c);
    const float4 a = src[0], b = src[1];
    acc[0] = fmaf(w, a.x, acc[0]); acc[1] = fmaf(w, a.y, acc[1]);
    acc[2] = fmaf(w, a.z, acc[2]); acc[3] = fmaf(w, a.w, acc[3]);
    acc[4] = fmaf(w, b.x, acc[4]); acc[5] = fmaf(w, b.y, acc[5]);
    acc[6] = fmaf(w, b.z, acc[6]); acc[7] = fmaf(w, b.w, acc[7]);
  }
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = bf16_rne(acc[2 * i]) | (bf16_rne(acc[2 * i + 1]) << 16);
  *(uint4*)(out + t * out_stride + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

static int launch_combine_rows(const BindingImpl& b, const int32_t* pos, hipStream_t s) {
  const int64_t total = b.T * (b.H / 8);
  if (total == 0) return 0;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, b.y, (int64_t)b.H, pos,
                     b.ids, b.E, b.tw, b.T, b.k, b.H, b.max_rows, b.out, b.out_stride);
  return (int)hipGetLastError();
}

// grouped path: y rows in routing order, located through pos
int launch_combine(const BindingImpl& b, hipStream_t s) { return launch_combine_rows(b, b.pos, s); }

// decode path: y rows indexed by pair id
int launch_decode_combine(const BindingImpl& b, hipStream_t s) { return launch_combine_rows(b, nullptr, s); }

}  // namespace b12x
