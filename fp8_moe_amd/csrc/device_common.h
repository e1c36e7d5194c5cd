// Device helpers shared by the gfx950 kernels: vector types, bf16 and
// E4M3 / E8M0 encoders written with integer operations (so that results do
// not depend on denormal modes), and the MXFP8 block-scale rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace b12x {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Activation format of the grouped GEMMs beyond the public ones: a scaled f16
// copy of bf16 activations (one power-of-two exponent per row), used with
// NVFP4 weights.
constexpr int kActF16 = 3;
// bf16 activations that are MXFP8 round trips (NVFP4 weights x MXFP8
// activations): the operand path is bf16, and the gate/up epilogue stores h
// as the bf16 value of its own MXFP8 round trip.
constexpr int kActRt = 4;
// The same round trips as a scaled f16 copy (NVFP4 weights x MXFP8
// activations on the grouped path): the f16 operand path of kActF16 with the
// round-trip epilogue of kActRt.
constexpr int kActF16Rt = 5;
// NVFP4 activations with NVFP4 weights (W4A4): the operands are the exact
// values E2M1 * E4M3 of the NVFP4 round trips (at most 6 significant bits, so
// exact in bf16 and in f16), the per-tensor activation scale is applied to
// the fp32 accumulator with the weights' one, and the gate/up epilogue stores
// h as its own NVFP4 round trip (against the expert's activation scale).
// kActNvRt: bf16 operand path; kActF16NvRt: f16 operand path (grouped GEMM).
constexpr int kActNvRt = 6;
constexpr int kActF16NvRt = 7;

// Raw buffer loads (CDNA buffer resource, stride 0).  A byte offset at or
// past the record count returns zeros without a memory access, so a guarded
// load needs no branch and every load of a loop is issued unconditionally;
// the compiler then counts outstanding loads exactly and waits only for the
// ones a step consumes.  Records are limited to kMaxBufferBytes (1 GiB,
// checked on the host); kBufOOB = 1.5 GiB is out of range, and so are
// kBufOOB + any in-range offset and 2 * kBufOOB (no 32-bit wrap).
constexpr uint32_t kBufOOB = 0x60000000u;
static_assert(kMaxBufferBytes <= (int64_t)kBufOOB && 2ull * kBufOOB < (1ull << 32) &&
                  (uint64_t)kBufOOB + kMaxBufferBytes < (1ull << 32), "out-of-range marker");
typedef __amdgpu_buffer_rsrc_t BufRsrc;

__device__ __forceinline__ BufRsrc make_rsrc(const void* base, int64_t bytes) {
  const int n = (int)(bytes < kMaxBufferBytes ? bytes : kMaxBufferBytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(BufRsrc r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// The same with a scalar (wave-uniform) part of the offset in soff.  Callers
// keep voff + soff inside the resource for every in-range voff, so the result
// does not depend on whether the hardware range-checks soff.
__device__ __forceinline__ uint4 buf_load16s(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4s(BufRsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ int buf_load1(BufRsrc r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// Device-coherent accesses: cache policy SC1 (device scope), the accesses the
// compiler emits for relaxed device-scope atomic loads and stores.  The L2
// caches of the XCDs are not coherent with each other for ordinary accesses;
// an SC1 store writes through to the device's coherence point and counts as
// complete (vmcnt) once it is visible there, and an SC1 load reads from that
// point.  Data handed between workgroups of one kernel this way needs no
// cache writeback or invalidation: the writer waits for its stores
// (vmcnt(0)) before it raises a flag with a device-scope store, and the
// reader loads with SC1 after it has seen the flag.
constexpr int kCpolDevice = 16;  // SC1
__device__ __forceinline__ uint4 buf_load16_dev(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ uint64_t buf_load8_dev(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCpolDevice));
}
__device__ __forceinline__ void buf_store2_dev(BufRsrc r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, kCpolDevice);
}
// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt at their maxima; gfx9 encoding)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return bits_f32(h << 16); }

// floor(log2 m) for a non-zero fp32 magnitude given by its bits.
__device__ __forceinline__ int ilog2_mag(uint32_t mag) {
  const uint32_t e = mag >> 23;
  if (e) return (int)e - 127;
  return (31 - __builtin_clz(mag)) - 149;  // subnormal: m * 2^-149
}

// MXFP8 shared exponent of a 32-block from its largest magnitude (fp32 bits):
// clamp(floor(log2 amax) - 8, -127, 127), or -127 for an all-zero block.
__device__ __forceinline__ int mx_scale_exp(uint32_t amax_mag) {
  if (amax_mag == 0) return -127;
  int s = ilog2_mag(amax_mag) - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// Round sig / 2^sh to the nearest integer, ties to even (sig < 2^24, sh >= 1).
__device__ __forceinline__ uint32_t rne_shift(uint32_t sig, int sh) {
  if (sh >= 25) return 0;  // sig < 2^24 <= half: below one half
  const uint32_t r = sig >> sh, rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
  return r + ((rem > half || (rem == half && (r & 1u))) ? 1u : 0u);
}

// E4M3 (FN) code of v * 2^-s (v given as fp32 bits, s the block exponent):
// round half to even onto the E4M3 grid, subnormals kept, saturating at
// +-448, sign of zero kept.
__device__ __forceinline__ uint32_t e4m3_encode_scaled(uint32_t vbits, int s) {
  const uint32_t sign = (vbits >> 24) & 0x80u;
  const uint32_t mag = vbits & 0x7FFFFFFFu;
  if (mag == 0) return sign;
  uint32_t sig;
  int ev;
  if (mag >> 23) {
    sig = (mag & 0x7FFFFFu) | 0x800000u;
    ev = (int)(mag >> 23) - 127;
  } else {
    const int lz = __builtin_clz(mag) - 8;
    sig = mag << lz;
    ev = -126 - lz;
  }
  const int eq = ev - s;  // value = sig * 2^(eq - 23)
  int code;
  if (eq >= -6) {
    code = ((eq + 7) << 3) + (int)rne_shift(sig, 20) - 8;  // a carry into 16 bumps the exponent
    if (code > 0x7E) code = 0x7E;
  } else {
    code = (int)rne_shift(sig, 14 - eq);  // units of 2^-9; 8 is the smallest normal
  }
  return sign | (uint32_t)code;
}

// Value of an E4M3 (FN) code as fp32 (finite codes).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? bits_f32(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Operands of the scaled E4M3 conversions for a block with exponent s
// (-127 .. 127): the scale 2^s (the conversions read only its exponent
// field, so s = -127 gives 2^-127) and the saturation limit 448 * 2^s.
struct MxScale {
  float scale, lim;
};
__device__ __forceinline__ MxScale mx_scale(int s) { return {bits_f32((uint32_t)(s + 127) << 23), ldexpf(448.0f, s)}; }

// E4M3 codes of a / 2^s and b / 2^s (finite a, b) into byte pair HI of o:
// the hardware conversion rounds to nearest even but does not saturate, so
// both are clamped to 448 * 2^s first.  Equal to e4m3_encode_scaled up to the
// sign of a zero (mx_roundtrip_bf16, built on it, is compared element by
// element with the integer encoder's round trip over every finite bf16 value
// and every block exponent).
template <bool HI>
__device__ __forceinline__ s16x2 e4m3_pk_scaled(s16x2 o, float a, float b, MxScale m) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, __builtin_amdgcn_fmed3f(a, -m.lim, m.lim),
                                                  __builtin_amdgcn_fmed3f(b, -m.lim, m.lim), m.scale, HI);
}

// E4M3 codes of the 4 bf16 values in w0, w1 (low half first) of a block: one dword.
__device__ __forceinline__ uint32_t e4m3_codes4_bf16(uint32_t w0, uint32_t w1, MxScale m) {
  s16x2 o = {0, 0};
  o = e4m3_pk_scaled<false>(o, bits_f32(w0 << 16), bits_f32(w0 & 0xFFFF0000u), m);
  o = e4m3_pk_scaled<true>(o, bits_f32(w1 << 16), bits_f32(w1 & 0xFFFF0000u), m);
  return __builtin_bit_cast(uint32_t, o);
}

// bf16 bits of the MXFP8 round trip of v (fp32, finite) in a block with
// exponent s (-127 .. 127): E4M3 code of v / 2^s, decoded and multiplied by
// 2^s (exact in fp32; exact in bf16 above its subnormal range, 2^-133), by
// the scaled hardware conversions both ways.
__device__ __forceinline__ uint32_t mx_roundtrip_bf16(float v, int s) {
  const MxScale m = mx_scale(s);
  const s16x2 o = e4m3_pk_scaled<false>(s16x2{0, 0}, v, v, m);
  return bf16_rne(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)(uint16_t)o.x, m.scale, false)[0]);
}

// SwiGLU-OAI (b12x README "What's in here" names it; the definition is the one
// published with the gpt-oss models): the gate clamped from above at 7, up to
// [-7, 7], h = gate * sigmoid(1.702 gate) * (up + 1).  A gate far below zero
// makes the exponential infinite and h a signed zero.
constexpr float kOaiAlpha = 1.702f, kOaiLimit = 7.0f;
__device__ __forceinline__ float swiglu_oai(float gt, float up) {
  gt = fminf(gt, kOaiLimit);
  up = fminf(fmaxf(up, -kOaiLimit), kOaiLimit);
  return gt * __builtin_amdgcn_rcpf(1.0f + __expf(-kOaiAlpha * gt)) * (up + 1.0f);
}

// Largest value over the 16 lanes of this lane's DPP row (lanes 16r .. 16r+15),
// in every lane of the row: max with the lane ^ 1 and ^ 2 (quad permutes),
// then with the mirrored lane in the half row and in the row.  VALU only.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, bits_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f32_bits(v), 0x140, 0xF, 0xF, false)));
  return v;
}

// NVFP4 activation quantization, exact rule: per block of 16 the E4M3 value s
// nearest to amax / (6 g) (ties to the even code, saturating at 448), per
// element the E2M1 value nearest to v / (s g) (ties to the even code,
// saturating at 6); a block with s = 0 quantizes to zeros.  A candidate comes
// from the binary32 quotient and the hardware conversions (round to nearest
// even); it is at most one code from the exact answer (the quotient is within
// 2^-22 relative of the exact one, and neighbouring codes are at least a
// sixteenth apart).  It is then corrected by the exact comparisons of the
// magnitude with the two midpoints next to it: a midpoint times the unit
// (6 g or s g) is mid6 * g or (mid * s) * g, whose first factor is exact in
// binary32 (at most 7 significant bits), and fma(first, g, -|v|) has the sign
// of the exact difference.  Domain: g in [2^-64, 2^64] (every product and
// nonzero difference then stays a normal binary32), finite v.
typedef short nv_s16x2 __attribute__((ext_vector_type(2)));

// Magnitude of the E4M3 code c in [0, 0x7E] and its distance to code c + 1.
__device__ __forceinline__ float e4m3_mag(uint32_t c) { return e4m3_value(c & 0x7Fu); }
__device__ __forceinline__ float e4m3_step(uint32_t c) {  // 2^(max(e, 1) - 10)
  const uint32_t e = c >> 3;
  return bits_f32((uint32_t)((e ? e : 1u) + 117u) << 23);
}

__device__ __forceinline__ float nv_block_scale(float amax, float g) {
  const float t = fminf(__fdiv_rn(amax, 6.0f * g), 448.0f);
  nv_s16x2 o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, t, t, 1.0f, false);
  uint32_t c = (uint32_t)(uint16_t)o.x & 0x7Fu;
  const float v = e4m3_mag(c);
  if (c < 0x7Eu) {  // midpoint with the next code
    const float d = fmaf((v + 0.5f * e4m3_step(c)) * 6.0f, g, -amax);
    if (d < 0.0f || (d == 0.0f && (c & 1u))) return e4m3_mag(c + 1u);
  }
  if (c > 0u) {  // midpoint with the previous code
    const float d = fmaf((v - 0.5f * e4m3_step(c - 1u)) * 6.0f, g, -amax);
    if (d > 0.0f || (d == 0.0f && (c & 1u))) return e4m3_mag(c - 1u);
  }
  return v;
}

// Reciprocal of s g for the candidate element quotients of a block with
// scale s: 1 / (s g) rounded, at most the largest finite fp32, and 0 for a
// block whose scale is 0.
__device__ __forceinline__ float nv_recip(float s, float g) {
  const float u = s * g;
  return u > 0.0f ? fminf(__fdiv_rn(1.0f, u), 3.40282347e38f) : 0.0f;
}

// E2M1 magnitude of the 3-bit code c (the hardware decode).
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c & 7u, 1.0f, 0)[0];
}

// E2M1 * s of the NVFP4 round trip of v in a block with scale s (g, the
// per-tensor scale, is left to the GEMM; r = nv_recip(s, g)); sign of v kept.
// Exact in fp32, bf16 and f16.
__device__ __forceinline__ float nv_roundtrip(float v, float s, float g, float r) {
  if (s == 0.0f) return v * 0.0f;
  const float a = fabsf(v);
  const float q = fminf(a * r, 8.0f);
  uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q, q, 1.0f, 0) & 7u;
  const float m = e2m1_mag(c);
  float mag = m;
  if (c < 7u) {
    const float d = fmaf((0.5f * (m + e2m1_mag(c + 1u))) * s, g, -a);
    if (d < 0.0f || (d == 0.0f && (c & 1u))) mag = e2m1_mag(c + 1u);
  }
  if (c > 0u) {
    const float d = fmaf((0.5f * (m + e2m1_mag(c - 1u))) * s, g, -a);
    if (d > 0.0f || (d == 0.0f && (c & 1u))) mag = e2m1_mag(c - 1u);
  }
  return copysignf(mag * s, v);
}

// E8M0 scale code as the fp32 whose exponent field is the code; the gfx950
// scaled FP4 conversions read exactly that field.
__device__ __forceinline__ float e8m0_as_scale(uint32_t c) { return bits_f32(c << 23); }

__device__ __forceinline__ bf16x8 u32x4_as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  i32x4 v = {(int)a, (int)b, (int)c, (int)d};
  return __builtin_bit_cast(bf16x8, v);
}

// Eight FP4 codes (one dword, low nibble first) -> eight bf16 (as 4 dwords).
template <int WF>
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t codes, float scale) {
  if constexpr (WF == B12X_WEIGHT_MXFP4) {
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return u32x4_as_bf16x8(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                           __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
  } else {
    uint32_t out[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x2 v;
      if (b == 0) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
      if (b == 1) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
      if (b == 2) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
      if (b == 3) v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
      const uint32_t lo = f32_bits(v.x * scale), hi = f32_bits(v.y * scale);
      out[b] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // exact: <= 6 significant bits
    }
    return u32x4_as_bf16x8(out[0], out[1], out[2], out[3]);
  }
}

// NVFP4 weights for the f16 MFMA: one E4M3 block scale s = 2^E * F (F in
// [1, 2) with at most 4 significant bits; sign kept in F).  The scaled FP4
// conversion applies 2^E (it reads only the exponent field of its scale) and
// one packed f16 multiply applies F to two values: 8 instructions for 8
// weights.  Every product has at most 6 significant bits and lies in
// [2^-10, 2688] (or is zero), so it is exact in f16.
struct NvScaleF16 {
  float e;   // 2^E as the scaled conversion's scale operand
  f16x2 f;   // F, F
};
__device__ __forceinline__ NvScaleF16 nv_scale_f16(float s) {
  const uint32_t b = f32_bits(s);
  NvScaleF16 r;
  r.e = bits_f32(b & 0x7F800000u);  // s = 0: exponent field 0, the products are 0
  const float fm = bits_f32((b & 0x807FFFFFu) | 0x3F800000u);
  r.f = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(fm, fm));  // exact: <= 4 significant bits
  return r;
}
__device__ __forceinline__ f16x8 dequant8_f16_nv(uint32_t codes, const NvScaleF16& sc) {
  const f16x2 p0 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc.e, 0)) * sc.f;
  const f16x2 p1 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc.e, 1)) * sc.f;
  const f16x2 p2 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc.e, 2)) * sc.f;
  const f16x2 p3 = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, sc.e, 3)) * sc.f;
  return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

}  // namespace b12x
