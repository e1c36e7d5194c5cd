// Debug aids of the host runtime: the scratch fill of b12x_moe_prime
// (B12X_DEBUG_SCRATCH_FILL=1) and the per-stage timing of b12x_moe_run
// (B12X_TIMING=1).  Neither is on the path of an ordinary call.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace b12x {

// Every 8-byte word of [p, p + 8 n) set to value (a kernel, not a memset, so
// that a captured graph may hold it).
__global__ __launch_bounds__(256) void fill_words_kernel(uint64_t* __restrict__ w, int64_t n, uint64_t value) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = value;
}

int launch_fill_words(void* p, uint64_t bytes, uint64_t value, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 8);
  if (!p || n == 0) return 0;
  hipLaunchKernelGGL(fill_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint64_t*)p, n, value);
  return (int)hipGetLastError();
}

bool stream_capturing(hipStream_t s) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) != hipSuccess || st != hipStreamCaptureStatusNone;
}

void* timing_mark(hipStream_t s) {
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  if (hipEventRecord(e, s) != hipSuccess) {
    (void)hipEventDestroy(e);
    return nullptr;
  }
  return (void*)e;
}

double timing_ms(void* a, void* b) {
  float ms = -1.0f;
  if (!a || !b || hipEventSynchronize((hipEvent_t)b) != hipSuccess) return -1.0;
  if (hipEventElapsedTime(&ms, (hipEvent_t)a, (hipEvent_t)b) != hipSuccess) return -1.0;
  return ms;
}

void timing_free(void* e) {
  if (e) (void)hipEventDestroy((hipEvent_t)e);
}

}  // namespace b12x
