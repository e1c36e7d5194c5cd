// MXFP8 row quantizer (b12x README "What's in here": quantization.mxfp8 row
// quantizer, the dynamic activation quantization of the W4A8 MoE modes;
// "PCIe DMA wire modes": one E8M0 scale per 32 values): amax, shared
// exponent and E4M3 codes per 32-element block, integer only.
#include "device_common.h"

namespace b12x {

// Eight lanes per 32-element block, four values each (an aligned group of 8
// lanes of a wave, so a group is wholly in or out of range): the block's
// largest magnitude by lane exchange, then each lane encodes its four values.
// The row count is lv's (a binding's T, or the live token count).
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, LiveT lv,
                                                          int64_t blocks_per_row, int64_t stride,
                                                          uint8_t* __restrict__ codes, int64_t code_stride,
                                                          uint8_t* __restrict__ scales, int64_t scale_stride) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk_all = idx >> 3;
  const int64_t rows = lv.tokens();
  if (!lv.on() || blk_all >= rows * blocks_per_row) return;
  const int part = (int)(idx & 7);  // elements [4 part, 4 part + 4) of the block
  const int64_t r = blk_all / blocks_per_row, blk = blk_all % blocks_per_row;
  const uint2 v = *(const uint2*)(x + r * stride + blk * 32 + 4 * part);
  // bf16 magnitude bits compare like the values
  uint32_t amax = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4));
  const int s = mx_scale_exp(amax << 16);
  const uint32_t word = e4m3_encode_scaled(v.x << 16, s) | (e4m3_encode_scaled(v.x & 0xFFFF0000u, s) << 8) |
                        (e4m3_encode_scaled(v.y << 16, s) << 16) | (e4m3_encode_scaled(v.y & 0xFFFF0000u, s) << 24);
  *(uint32_t*)(codes + r * code_stride + blk * 32 + 4 * part) = word;
  if (part == 0) scales[r * scale_stride + blk] = (uint8_t)(s + 127);
}

// The same blocks, writing bf16 of each value's MXFP8 round trip instead of
// codes and scales (NVFP4 weights x MXFP8 activations).
__global__ __launch_bounds__(256) void mx_roundtrip_rows_kernel(const uint16_t* __restrict__ x, LiveT lv,
                                                                 int64_t blocks_per_row, int64_t stride,
                                                                 uint16_t* __restrict__ out, int64_t out_stride) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk_all = idx >> 3;
  const int64_t rows = lv.tokens();
  if (!lv.on() || blk_all >= rows * blocks_per_row) return;
  const int part = (int)(idx & 7);
  const int64_t r = blk_all / blocks_per_row, blk = blk_all % blocks_per_row;
  const uint2 v = *(const uint2*)(x + r * stride + blk * 32 + 4 * part);
  uint32_t amax = max(max(v.x & 0x7FFFu, (v.x >> 16) & 0x7FFFu), max(v.y & 0x7FFFu, (v.y >> 16) & 0x7FFFu));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 4));
  const int s = mx_scale_exp(amax << 16);
  const uint32_t lo = mx_roundtrip_bf16(bits_f32(v.x << 16), s) | (mx_roundtrip_bf16(bits_f32(v.x & 0xFFFF0000u), s) << 16);
  const uint32_t hi = mx_roundtrip_bf16(bits_f32(v.y << 16), s) | (mx_roundtrip_bf16(bits_f32(v.y & 0xFFFF0000u), s) << 16);
  *(uint2*)(out + r * out_stride + blk * 32 + 4 * part) = make_uint2(lo, hi);
}

int launch_mx_roundtrip_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint16_t* out,
                             int64_t out_stride, hipStream_t s) {
  const int64_t bpr = cols / 32;
  const int64_t total = lv.cap * bpr;
  if (total == 0) return 0;
  hipLaunchKernelGGL(mx_roundtrip_rows_kernel, dim3((unsigned)((8 * total + 255) / 256)), dim3(256), 0, s, x, lv,
                     bpr, stride, out, out_stride);
  return (int)hipGetLastError();
}

// NVFP4 round trips of bf16 rows against the per-tensor activation scale
// g[0] (NVFP4 activations with NVFP4 weights): per block of 16, the E4M3
// scale s nearest to amax / (6 g) and each value's E2M1 code nearest to
// v / (s g), both decided exactly (nv_block_scale, nv_roundtrip); out holds
// E2M1 * s (exact), the scale g is left to the GEMM.
// Two threads per block of 16 (8 values each).  F16: f16 values plus a row
// exponent of 0 for the f16 operand path of the grouped GEMM; else bf16.
template <bool F16>
__global__ __launch_bounds__(256) void nv_roundtrip_rows_kernel(const uint16_t* __restrict__ x, LiveT lv,
                                                                int64_t blocks_per_row, int64_t stride,
                                                                const float* __restrict__ g,
                                                                uint16_t* __restrict__ out, int64_t out_stride,
                                                                int32_t* __restrict__ exps) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk_all = idx >> 1;
  const int64_t rows = lv.tokens();
  if (!lv.on() || blk_all >= rows * blocks_per_row) return;
  const int part = (int)(idx & 1);
  const int64_t r = blk_all / blocks_per_row, blk = blk_all % blocks_per_row;
  const uint4 v = *(const uint4*)(x + r * stride + blk * 16 + 8 * part);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t amax = 0;  // bf16 magnitude bits compare like the values
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  const float gs = g[0];
  const float sc = nv_block_scale(bits_f32(amax << 16), gs);
  const float rc = nv_recip(sc, gs);
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = nv_roundtrip(bf16_to_f32(w[i] & 0xFFFFu), sc, gs, rc);
    const float hi = nv_roundtrip(bf16_to_f32(w[i] >> 16), sc, gs, rc);
    if constexpr (F16)
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    else
      o[i] = bf16_rne(lo) | (bf16_rne(hi) << 16);
  }
  *(uint4*)(out + r * out_stride + blk * 16 + 8 * part) = make_uint4(o[0], o[1], o[2], o[3]);
  if (F16 && blk == 0 && part == 0) exps[r] = 0;
}

int launch_nv_roundtrip_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, const float* g,
                             uint16_t* out, int64_t out_stride, int32_t* exps, bool f16, hipStream_t s) {
  const int64_t bpr = cols / 16;
  const int64_t total = lv.cap * bpr;
  if (total == 0) return 0;
  const dim3 grid((unsigned)((2 * total + 255) / 256));
  if (f16)
    hipLaunchKernelGGL(nv_roundtrip_rows_kernel<true>, grid, dim3(256), 0, s, x, lv, bpr, stride, g, out,
                       out_stride, exps);
  else
    hipLaunchKernelGGL(nv_roundtrip_rows_kernel<false>, grid, dim3(256), 0, s, x, lv, bpr, stride, g, out,
                       out_stride, exps);
  return (int)hipGetLastError();
}

int launch_quant_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint8_t* codes,
                      int64_t code_stride, uint8_t* scales, int64_t scale_stride, hipStream_t s) {
  const int64_t bpr = cols / 32;
  const int64_t total = lv.cap * bpr;
  if (total == 0) return 0;
  hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((8 * total + 255) / 256)), dim3(256), 0, s, x, lv, bpr,
                     stride, codes, code_stride, scales, scale_stride);
  return (int)hipGetLastError();
}

// Scaled f16 copy of bf16 rows for the NVFP4 weight GEMMs, which dequantize
// the weights to f16 (half the conversion work of bf16 on gfx950, see the
// grouped GEMM).  Row r is multiplied by 2^-e[r] with e[r] = floor(log2
// max|x_r|) - 14 (at least -126, so that 2^-e and 2^e are normal fp32
// values; 0 for an all-zero row; bf16 maxima give at most 113), which puts
// the row maximum in [2^14, 2^15): every bf16 value above 2^-31 of the row
// maximum is then exact in f16, and the GEMM multiplies its fp32 results by
// 2^e[r].  One workgroup per row.
// RT: the values copied are the MXFP8 round trips of the row (blocks of 32 =
// 4 consecutive threads, 8 values each); their magnitudes stay within
// 1 + 2^-4 of the bf16 row maximum the exponent is taken from (a saturated
// block maximum rounds down), so the f16 copy stays below 2^16.
template <bool RT>
__global__ __launch_bounds__(256) void f16_rows_kernel(const uint16_t* __restrict__ x, int64_t cols, int64_t stride,
                                                        uint16_t* __restrict__ out, int64_t out_stride,
                                                        int32_t* __restrict__ exps, LiveT lv) {
  __shared__ uint32_t s_max[4];
  const int64_t r = blockIdx.x;
  const int64_t rows = lv.tokens();
  if (!lv.on() || r >= rows) return;
  const uint16_t* src = x + r * stride;
  uint32_t m = 0;  // bf16 magnitude bits compare like the values
  for (int64_t c = threadIdx.x * 8; c < cols; c += 256 * 8) {
    const uint4 v = *(const uint4*)(src + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  m = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  int e = m ? ilog2_mag(m << 16) - 14 : 0;
  e = e < -126 ? -126 : e;
  const float mul = bits_f32((uint32_t)(127 - e) << 23);  // 2^-e, exact
  // cols is a multiple of 32: a whole 32-block is 4 threads of one pass, all active or all idle
  for (int64_t c0 = 0; c0 < cols; c0 += 256 * 8) {
    const int64_t c = c0 + threadIdx.x * 8;
    const bool act = c < cols;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (act) v = *(const uint4*)(src + c);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if constexpr (RT) {
      uint32_t bm = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) bm = max(bm, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
      bm = max(bm, (uint32_t)__shfl_xor((int)bm, 1));
      bm = max(bm, (uint32_t)__shfl_xor((int)bm, 2));
      const int sb = mx_scale_exp(bm << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = mx_roundtrip_bf16(bf16_to_f32(w[i] & 0xFFFFu), sb) | (mx_roundtrip_bf16(bf16_to_f32(w[i] >> 16), sb) << 16);
    }
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 lo = (_Float16)(bf16_to_f32(w[i] & 0xFFFFu) * mul);
      const _Float16 hi = (_Float16)(bf16_to_f32(w[i] >> 16) * mul);
      o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    if (act) *(uint4*)(out + r * out_stride + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (threadIdx.x == 0) exps[r] = e;
}

int launch_f16_rows(const uint16_t* x, LiveT lv, int64_t cols, int64_t stride, uint16_t* out,
                    int64_t out_stride, int32_t* exps, bool rt, hipStream_t s) {
  if (lv.cap == 0) return 0;
  if (rt)
    hipLaunchKernelGGL(f16_rows_kernel<true>, dim3((unsigned)lv.cap), dim3(256), 0, s, x, cols, stride, out,
                       out_stride, exps, lv);
  else
    hipLaunchKernelGGL(f16_rows_kernel<false>, dim3((unsigned)lv.cap), dim3(256), 0, s, x, cols, stride, out,
                       out_stride, exps, lv);
  return (int)hipGetLastError();
}

}  // namespace b12x
