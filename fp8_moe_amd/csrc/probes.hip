// Achievable-ceiling probes, reported beside the datasheet peaks: a plain
// streaming read of device memory (what HBM delivers to a kernel that only
// reads) and an MFMA register loop (what the matrix cores sustain with no
// memory traffic, at whatever clock the part holds under that load).
#include <type_traits>

#include "b12x_probes.h"
#include "device_common.h"

namespace b12x {

// Workgroup b reads its contiguous share of `words` 16-byte words, four loads
// in flight per lane, and writes one XOR per thread (so no load is dead).
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ src, uint64_t words,
                                                          uint32_t* __restrict__ sink) {
  const uint64_t per = words / gridDim.x;
  const uint64_t base = per * blockIdx.x;
  uint32_t acc = 0;
  for (uint64_t i = threadIdx.x; i + 3 * 256 < per; i += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = src[base + i + d * 256];
#pragma unroll
    for (int d = 0; d < 4; ++d) acc ^= v[d].x ^ v[d].y ^ v[d].z ^ v[d].w;
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// Every wave issues `iters` rounds of 16 independent 16x16x32 MFMAs (bf16 or
// f16) on register operands.
template <bool F16>
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ sink, int iters, float seed) {
  using OpT = std::conditional_t<F16, f16x8, bf16x8>;
  using ElT = std::conditional_t<F16, _Float16, __bf16>;
  const float v = seed + (float)(threadIdx.x & 7);
  OpT a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (ElT)(v * 0.25f);
    b[i] = (ElT)(v * 0.5f);
  }
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (F16) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
      else acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace b12x

extern "C" {

int32_t b12x_probe_stream_read(const void* src, uint64_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink || workgroups < 1) return 1;
  if (bytes % 16 || (uintptr_t)src % 16) return 5;
  hipLaunchKernelGGL(b12x::probe_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

int32_t b12x_probe_mfma(float* sink, int32_t workgroups, int32_t iterations, int32_t f16, void* stream) {
  if (!sink || workgroups < 1 || iterations < 1) return 1;
  const hipStream_t s = (hipStream_t)stream;
  if (f16)
    hipLaunchKernelGGL(b12x::probe_mfma_kernel<true>, dim3((unsigned)workgroups), dim3(256), 0, s, sink, iterations,
                       1.0f);
  else
    hipLaunchKernelGGL(b12x::probe_mfma_kernel<false>, dim3((unsigned)workgroups), dim3(256), 0, s, sink, iterations,
                       1.0f);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

}  // extern "C"
