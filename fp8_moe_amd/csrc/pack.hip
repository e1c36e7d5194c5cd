// Weight packer: source FP4 codes and block scales -> the fragment layout the
// grouped GEMMs stream (b12x README "Using it": prepare_weights; vLLM b12x
// page "ModelOpt block codecs": packing rearranges encoded blocks and never
// expands to BF16).  Byte moves only.
#include "device_common.h"

namespace b12x {

// Source row of packed fragment f, row r (0..15).
__device__ __forceinline__ int64_t src_row(int64_t f, int r, int gated_interleave, int64_t half_rows) {
  if (!gated_interleave) return f * kFragN + r;
  return (f & 1 ? half_rows : 0) + (f >> 1) * kFragN + r;
}

// One thread per (expert, fragment, K fragment, lane): 16 bytes of codes.
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int64_t total, int64_t N, int64_t K, int64_t NF,
                                                          int64_t KF, int gated_interleave) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t t = idx >> 6;
  const int64_t kf = t % KF;
  t /= KF;
  const int64_t f = t % NF;
  const int64_t e = t / NF;
  const int64_t n = src_row(f, lane & 15, gated_interleave, N / 2);
  const int64_t k0 = kf * kFragK + 32 * (lane >> 4);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (k0 < K) v = *(const uint4*)(src + (e * N + n) * (K / 2) + k0 / 2);
  *(uint4*)(dst + idx * 16) = v;
}

// One thread per (expert, fragment, scale group, lane): one dword of scales.
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                           int64_t total, int64_t N, int64_t K, int64_t NF,
                                                           int64_t KF, int64_t KFS, int gated_interleave, int nv) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t t = idx >> 6;
  const int64_t q = t % KFS;
  t /= KFS;
  const int64_t f = t % NF;
  const int64_t e = t / NF;
  const int64_t n = src_row(f, lane & 15, gated_interleave, N / 2);
  const int g = lane >> 4;
  uint32_t word = 0;
  if (!nv) {  // E8M0 per 32: byte j = fragment 4q+j, block (128 kf + 32 g) / 32
    const int64_t row_blocks = K / 32;
    for (int j = 0; j < 4; ++j) {
      const int64_t kf = 4 * q + j;
      const int64_t blk = 4 * kf + g;
      const uint32_t b = (kf < KF && blk < row_blocks) ? src[(e * N + n) * row_blocks + blk] : 127u;
      word |= b << (8 * j);
    }
  } else {  // E4M3 per 16: bytes 2j, 2j+1 = fragment 2q+j, halves of the lane's 32 elements
    const int64_t row_blocks = K / 16;
    for (int j = 0; j < 2; ++j) {
      const int64_t kf = 2 * q + j;
      for (int hh = 0; hh < 2; ++hh) {
        const int64_t blk = 8 * kf + 2 * g + hh;
        const uint32_t b = (kf < KF && blk < row_blocks) ? src[(e * N + n) * row_blocks + blk] : 0x38u;
        word |= b << (8 * (2 * j + hh));
      }
    }
  }
  *(uint32_t*)(dst + idx * 4) = word;
}

__global__ void copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

int launch_pack(const PackArgs& a, hipStream_t s) {
  const MatrixLayout& l = a.l;
  const int64_t total_codes = (int64_t)a.E * l.nf * l.kf * 64;
  const int64_t total_scales = (int64_t)a.E * l.nf * l.kfs * 64;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((total_codes + 255) / 256)), dim3(256), 0, s, a.src_codes,
                     a.dst_codes, total_codes, l.n, l.k, l.nf, l.kf, a.gated_interleave);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((total_scales + 255) / 256)), dim3(256), 0, s,
                     a.src_scales, a.dst_scales, total_scales, l.n, l.k, l.nf, l.kf, l.kfs, a.gated_interleave,
                     a.wfmt == B12X_WEIGHT_NVFP4 ? 1 : 0);
  return (int)hipGetLastError();
}

int launch_copy_f32(const float* src, float* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL(copy_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return (int)hipGetLastError();
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace b12x
