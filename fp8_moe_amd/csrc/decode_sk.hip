// Split-K decode kernel of the fused MoE for the smallest batches (b12x
// README "What's in here": the micro-kernel decode path of fused_moe).
//
// With a handful of routing pairs the cost of a call is latency, not
// bandwidth: the down projection of the plain two-phase order cannot start
// before the whole h of its expert exists.  Here the intermediate dimension
// is cut into slices of 32 columns and one workgroup owns one (touched expert,
// slice) item from start to end:
//   1. it issues the DMA of the slice's W2 columns (one 32-wide lane group of
//      every W2 fragment, codes and scales) into LDS, which runs while
//   2. its 4 waves split K of the slice's gate/up (or w1) rows: weights,
//      scales and activation rows go straight to registers, all of a wave's
//      K fragments in flight at once; the activations are quantized in
//      registers when the format asks for it (MXFP8 codes for the scaled
//      fp8 x fp4 MFMA, or the exact MXFP8 / NVFP4 round trips as bf16);
//   3. the split-K partial sums meet in LDS in a fixed wave order, wave 0
//      applies the activation and the requantization of h (bf16, MXFP8 codes,
//      or the MXFP8 / NVFP4 round trip) and leaves the h tile in LDS;
//   4. the 4 waves multiply the h tile by the W2 slice from LDS (each wave a
//      quarter of the output rows) and write fp32 partial rows
//      part[pair][slice][H].
// No workgroup waits for another, so the result does not depend on which
// workgroups are resident.  The combine (decode_sk_combine_kernel) sums the
// slices of each pair in ascending slice order and the pairs of each token
// in ascending slot order, in fp32, and rounds once to bf16.
#include "decode_common.h"

namespace b12x {

constexpr int kSkSlice = 32;  // h columns per item: one E8M0 block, one W2 lane group
// Partial rows are H + 64 floats apart: rows H floats apart (a power of two here)
// put the same columns of every slice in the same memory channel, and the
// combine's loads, which read one column range of many rows at once, then
// queue on a few channels.
constexpr int kSkRowPad = kSplitKRowPad;
__host__ __device__ inline int sk_row_stride(int H) { return (H / 16 + 3) / 4 * 64 + kSkRowPad; }

struct SkParams {
  const int32_t* ids;
  const float* tw;
  int T, k, E, P;
  const uint16_t* x;  // bf16 activations [T, H]
  int64_t x_stride;   // elements
  int64_t x_bytes;
  int H, I;
  int KF1, KFS1;      // W13 / W1: K fragments over H and scale groups per fragment row
  int KF2, KFS2, NF2; // W2: K fragments over I, scale groups, fragments (H / 16)
  int n_slices;       // I / 32
  const uint8_t* w13c;
  const uint8_t* w13s;
  const float* g13;   // NVFP4: per-expert scale of W13
  int64_t w13c_e, w13s_e;
  const uint8_t* w2c;
  const uint8_t* w2s;
  const float* g2;
  int64_t w2c_e, w2s_e;
  const float* ax;    // NVFP4 activations: scale of x [1]
  const float* ah;    // and of each expert's h [E]
  float* part;        // [P][n_slices][row_stride]: per fragment group G (4 fragments), column n,
                      // fragment q: position 64 G + 4 n + q
  int64_t part_bytes;
  int row_stride;     // 64 per fragment group + 64: consecutive rows start on different memory channels
};

// LDS of one workgroup: routing, the split-K exchange, the h tile, and the
// W2 slice (dynamic part after the static one).
struct SkLds {
  uint32_t bits[4][32];         // each wave's copy of the touched-expert bitmap
  f32x4 red[3][4][64];          // partial sums of waves 1..3, up to 4 fragments
  uint16_t h16[16][kSkSlice];   // h tile, bf16 (16 rows x 32 columns)
  uint8_t h8[16][kSkSlice];     // or MXFP8 codes
  uint32_t hs[16];              // and their E8M0 scale codes
  uint4 zero;                   // zeros for the lanes outside the slice
  uint32_t neutral;             // a scale of 1 for those lanes
};

template <int WF>
__device__ __forceinline__ float w_scale(uint32_t word, int kf, int s) {
  if constexpr (WF == B12X_WEIGHT_MXFP4) return e8m0_as_scale((word >> (8 * (kf & 3))) & 0xFFu);
  else return e4m3_value((word >> (8 * (2 * (kf & 1) + (s >> 1)))) & 0xFFu);
}

// The bf16 operand of 8 activations from 4 dwords of bf16 values.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// MXFP8 round trip of the lane's 32 consecutive bf16 values (one E8M0 block):
// bf16 values of E4M3(v / 2^s) * 2^s.
__device__ __forceinline__ void mx_roundtrip32(uint4 (&v)[4]) {
  uint32_t amax = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t w[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  }
  const int sx = mx_scale_exp(amax << 16);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t* w = (uint32_t*)&v[s];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = mx_roundtrip_bf16(bf16_to_f32(w[i] & 0xFFFFu), sx) | (mx_roundtrip_bf16(bf16_to_f32(w[i] >> 16), sx) << 16);
  }
}

// NVFP4 round trip (E2M1 * E4M3, exact in bf16) of the lane's 32 bf16 values
// = two blocks of 16, against the per-tensor scale g.
__device__ __forceinline__ void nv_roundtrip32(uint4 (&v)[4], float g) {
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    uint32_t amax = 0;
#pragma unroll
    for (int s = 2 * b; s < 2 * b + 2; ++s) {
      const uint32_t w[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = max(amax, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
    const float sc = nv_block_scale(bits_f32(amax << 16), g), rc = nv_recip(sc, g);
#pragma unroll
    for (int s = 2 * b; s < 2 * b + 2; ++s) {
      uint32_t* w = (uint32_t*)&v[s];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = bf16_rne(nv_roundtrip(bf16_to_f32(w[i] & 0xFFFFu), sc, g, rc)) |
               (bf16_rne(nv_roundtrip(bf16_to_f32(w[i] >> 16), sc, g, rc)) << 16);
    }
  }
}

// E4M3 codes of 8 bf16 values (one uint4) in a block with exponent s, as 2 dwords.
__device__ __forceinline__ uint2 e4m3_codes8(const uint4& v, int s) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    o[h] = e4m3_encode_scaled(w[2 * h] << 16, s) | (e4m3_encode_scaled(w[2 * h] & 0xFFFF0000u, s) << 8) |
           (e4m3_encode_scaled(w[2 * h + 1] << 16, s) << 16) | (e4m3_encode_scaled(w[2 * h + 1] & 0xFFFF0000u, s) << 24);
  return make_uint2(o[0], o[1]);
}

__device__ __forceinline__ uint32_t max_mag16(const uint4& a, const uint4& b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}

// Routing of the split-K kernel, one wave at a time in registers (P <= 64: pair q
// in lane q).  Every wave builds its own bitmap of the touched experts in its own
// LDS words (a wave's LDS operations complete in order, so no barrier is needed),
// then finds the expert of a slot from per-word popcounts and the pairs of an
// expert from a ballot.

// Position of the n-th (0-based) set bit of a 64-bit mask (n < popcount(mask)).
__device__ __forceinline__ int nth_set_bit(uint64_t mask, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const uint64_t low = mask & ((1ull << w) - 1ull);
    const int c = __builtin_popcountll(low);
    if (n >= c) {
      n -= c;
      mask >>= w;
      pos += w;
    }
  }
  return pos;
}

struct SkRoute {
  int id;         // lane q: expert of pair q, -1 for no pair or a dropped one
  uint32_t word;  // lane w < 32: bitmap word w of the touched experts
  int below;      // lane w: touched experts in words 0 .. w-1
  int n_touched;
};

__device__ __forceinline__ SkRoute sk_route(const SkParams& p, uint32_t* wbits) {
  const int lane = threadIdx.x & 63;
  SkRoute r;
  int id = -1;
  if (lane < p.P) {
    const int e = p.ids[lane];
    id = (e >= 0 && e < p.E) ? e : -1;
  }
  r.id = id;
  if (lane < 32) wbits[lane] = 0u;
  if (id >= 0) atomicOr(&wbits[id >> 5], 1u << (id & 31));
  r.word = lane < 32 ? wbits[lane] : 0u;
  const int c = __builtin_popcount(r.word);
  int incl = c;
#pragma unroll
  for (int off = 1; off < 32; off <<= 1) {
    const int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  r.below = incl - c;
  r.n_touched = __builtin_amdgcn_readlane(incl, 31);
  return r;
}

// Expert of touched slot `slot` (the slot-th smallest distinct valid id).
__device__ __forceinline__ int sk_expert(const SkRoute& r, int slot) {
  const int lane = threadIdx.x & 63;
  const bool here = lane < 32 && slot >= r.below && slot < r.below + (int)__builtin_popcount(r.word);
  const uint64_t b = __ballot(here);
  const int w = __builtin_ctzll(b);
  const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)r.word, w);
  const int below = __builtin_amdgcn_readlane(r.below, w);
  return 32 * w + nth_set_bit(word, slot - below);
}

// Split-K decode kernel.  AF: B12X_ACT_BF16, B12X_ACT_MXFP8 (MXFP4 weights,
// scaled fp8 x fp4 MFMA), kActRt (NVFP4 weights, MXFP8 round trips as bf16)
// or kActNvRt (NVFP4 weights and activations).  KW: K fragments of W13 per
// wave held in registers at once (the wave's K range is taken KW at a time).
template <int WF, int AF, int MODE, int KW>
__global__ __launch_bounds__(kDecThreads) void decode_sk_kernel(const SkParams p) {
  constexpr bool A8 = AF == B12X_ACT_MXFP8;
  constexpr bool RT = AF == kActRt;
  constexpr bool NVRT = AF == kActNvRt;
  constexpr bool GATED = MODE == 1;
  constexpr int NF1 = GATED ? 4 : 2;  // W13 fragments of one slice (gate/up interleaved, or w1)
  __shared__ SkLds L;
  extern __shared__ __attribute__((aligned(1024))) uint8_t dyn[];  // W2 slice: codes [NF2][256], scales [NF2][16]
  uint8_t* const w2_lds = dyn;
  uint32_t* const w2s_lds = (uint32_t*)(dyn + (size_t)((p.NF2 + 3) / 4 * 4) * 256);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  if (tid == 0) {
    L.zero = make_uint4(0, 0, 0, 0);
    L.neutral = WF == B12X_WEIGHT_MXFP4 ? 0x7F7F7F7Fu : 0x38383838u;
  }
  const SkRoute route = sk_route(p, L.bits[wave]);
  const int64_t items = (int64_t)route.n_touched * p.n_slices;
  const int kper = (p.KF1 + 3) / 4;
  const int kb = wave * kper, ke = min(p.KF1, kb + kper);
  const BufRsrc x_rsrc = make_rsrc(p.x, p.x_bytes);
  const BufRsrc part_rsrc = make_rsrc(p.part, p.part_bytes);

  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int slot = (int)(item / p.n_slices), j = (int)(item % p.n_slices);
    const int e = sk_expert(route, slot);
    const uint64_t pairs = __ballot(route.id == e);  // the expert's pairs, ascending
    const int m = __builtin_popcountll(pairs);
    const int kf2 = j >> 2, gb = j & 3;
    if (item != blockIdx.x) __syncthreads();  // the previous item is done with the LDS

    // W2 slice -> LDS by DMA: lane group gb of K fragment kf2 of every W2 fragment row.
    // Issued once per item, after the first gate/up loads (vector memory operations
    // complete in order, so those loads do not wait for it); it lands while the
    // gate/up part runs.
    const BufRsrc w2c_rsrc = make_rsrc(p.w2c + (int64_t)e * p.w2c_e, p.w2c_e);
    const BufRsrc w2s_rsrc = make_rsrc(p.w2s + (int64_t)e * p.w2s_e, p.w2s_e);
    auto issue_w2_dma = [&]() {
      const int sgrp = WF == B12X_WEIGHT_MXFP4 ? kf2 >> 2 : kf2 >> 1;
      const int n_dma = (p.NF2 + 3) / 4;  // each DMA instruction: 4 fragments x 16 lanes
      for (int i = wave; i < n_dma; i += 4) {
        const int f2 = 4 * i + (lane >> 4);
        const bool v = f2 < p.NF2;
        const uint32_t co = v ? (uint32_t)((f2 * p.KF2 + kf2) * kFragBytes + (gb * 16 + r16) * 16) : kBufOOB;
        const uint32_t so = v ? (uint32_t)((f2 * p.KFS2 + sgrp) * kScaleGroupBytes + (gb * 16 + r16) * 4) : kBufOOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w2c_rsrc, (__attribute__((address_space(3))) void*)(w2_lds + i * 1024),
                                                 16, co, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(w2s_rsrc, (__attribute__((address_space(3))) void*)(w2s_lds + i * 64),
                                                 4, so, 0, 0, 0);
      }
    };
    bool dma_issued = false;

    float g1 = p.g13 ? p.g13[e] : 1.0f;
    if (NVRT) g1 *= p.ax[0];
    float g2 = p.g2 ? p.g2[e] : 1.0f;
    if (NVRT) g2 *= p.ah[e];
    const BufRsrc b_rsrc = make_rsrc(p.w13c + (int64_t)e * p.w13c_e, p.w13c_e);
    const BufRsrc bs_rsrc = make_rsrc(p.w13s + (int64_t)e * p.w13s_e, p.w13s_e);
    const int f1 = NF1 * j;  // first W13 fragment of the slice

    for (int r0 = 0; r0 < m; r0 += 16) {
      // ---- 2. gate/up (or w1) over this wave's K range, KW fragments at a time
      const int rr = r0 + r16;
      const int tok = rr < m ? nth_set_bit(pairs, rr) / p.k : -1;
      f32x4 acc[NF1];
#pragma unroll
      for (int f = 0; f < NF1; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = kb; c0 < ke; c0 += KW) {
        uint4 q[KW][NF1];
        uint32_t bs[KW][NF1];
        uint4 xa[KW][4];
        // scale words: one per fragment and scale group (4 K fragments for MXFP4, 2 for
        // NVFP4); the chunk spans at most NG groups
        constexpr int GK = WF == B12X_WEIGHT_MXFP4 ? 4 : 2;
        constexpr int NG = (KW + GK - 1) / GK + 1;
        const int sg0 = c0 / GK;
        uint32_t sw[NG][NF1];
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          const bool v = (sg0 + u) * GK < ke;
#pragma unroll
          for (int f = 0; f < NF1; ++f)
            sw[u][f] = buf_load4(bs_rsrc, v ? (uint32_t)(((f1 + f) * p.KFS1 + sg0 + u) * kScaleGroupBytes + lane * 4)
                                            : kBufOOB);
        }
#pragma unroll
        for (int i = 0; i < KW; ++i) {
          const int kf = c0 + i;
          const bool v = kf < ke;
          const int su = kf / GK - sg0;  // 0 .. NG-1
#pragma unroll
          for (int f = 0; f < NF1; ++f) {
            q[i][f] = buf_load16(b_rsrc, v ? (uint32_t)(((f1 + f) * p.KF1 + kf) * kFragBytes + lane * 16) : kBufOOB);
            uint32_t word = sw[0][f];
#pragma unroll
            for (int u = 1; u < NG; ++u) word = su == u ? sw[u][f] : word;
            bs[i][f] = word;
          }
          // activations of row r16: bf16 operands hold K 32 g + [0, 32) of the fragment;
          // the fp8 operand holds K 16 g + [0, 16) and 64 + 16 g + [0, 16)
          const int64_t k0 = (int64_t)kf * kFragK;
          const bool rv = v && tok >= 0;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            int64_t kk;
            if constexpr (A8) kk = k0 + (s < 2 ? 16 * g + 8 * s : 64 + 16 * g + 8 * (s - 2));
            else kk = k0 + 32 * g + 8 * s;
            xa[i][s] = buf_load16(x_rsrc, rv && kk < p.H ? (uint32_t)((tok * p.x_stride + kk) * 2) : kBufOOB);
          }
        }
        if (!dma_issued) {
          issue_w2_dma();
          dma_issued = true;
        }
        // every load of the chunk is in flight before the first MFMA waits
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < KW; ++i) {
          const int kf = c0 + i;
          if constexpr (!A8) {
            if constexpr (RT) mx_roundtrip32(xa[i]);
            if constexpr (NVRT) nv_roundtrip32(xa[i], p.ax[0]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
              for (int f = 0; f < NF1; ++f) {
                const uint32_t dw = s == 0 ? q[i][f].x : s == 1 ? q[i][f].y : s == 2 ? q[i][f].z : q[i][f].w;
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[i][s]),
                                                                 dequant8_bf16<WF>(dw, w_scale<WF>(bs[i][f], kf, s)),
                                                                 acc[f], 0, 0, 0);
              }
            }
          } else {
            // MXFP8 quantization of the activations: the first half (K 16 g ..) lies in
            // block g / 2 and the second (K 64 + 16 g ..) in block 2 + g / 2; each block's
            // other half sits in lane ^ 16
            uint32_t m1 = max_mag16(xa[i][0], xa[i][1]), m2 = max_mag16(xa[i][2], xa[i][3]);
            m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16));
            m2 = max(m2, (uint32_t)__shfl_xor((int)m2, 16));
            const int s1 = mx_scale_exp(m1 << 16), s2 = mx_scale_exp(m2 << 16);
            const uint2 c0w = e4m3_codes8(xa[i][0], s1), c1w = e4m3_codes8(xa[i][1], s1);
            const uint2 c2w = e4m3_codes8(xa[i][2], s2), c3w = e4m3_codes8(xa[i][3], s2);
            const i32x8 afr = {(int)c0w.x, (int)c0w.y, (int)c1w.x, (int)c1w.y,
                               (int)c2w.x, (int)c2w.y, (int)c3w.x, (int)c3w.y};
            // the scale operand of lane group g is block g's: 0 <- own first half,
            // 1 <- first half of lane group 2, 2 <- second half of lane group 1, 3 <- own second half
            const int t1 = __shfl_xor(s1, 48), t2 = __shfl_xor(s2, 48);
            const int sa = (g == 0 ? s1 : g == 1 ? t1 : g == 2 ? t2 : s2) + 127;
#pragma unroll
            for (int f = 0; f < NF1; ++f) {
              const i32x8 bfr = {(int)q[i][f].x, (int)q[i][f].y, (int)q[i][f].z, (int)q[i][f].w, 0, 0, 0, 0};
              const int sb = (int)((bs[i][f] >> (8 * (kf & 3))) & 0xFFu);
              acc[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr, acc[f], 0, 4, 0, sa, 0, sb);
            }
          }
        }
      }

      if (!dma_issued) {
        issue_w2_dma();
        dma_issued = true;
      }
      // ---- 3. split-K sums in wave order, activation and requantization of h by wave 0
      if (wave != 0) {
#pragma unroll
        for (int f = 0; f < NF1; ++f) L.red[wave - 1][f][lane] = acc[f];
      }
      __syncthreads();
      if (wave == 0) {
        f32x4 v[NF1];
#pragma unroll
        for (int f = 0; f < NF1; ++f) v[f] = acc[f] + L.red[0][f][lane] + L.red[1][f][lane] + L.red[2][f][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * g + i;
          float hv[2];  // columns r16 and 16 + r16 of the slice
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            if constexpr (GATED) {
              const float gt = v[2 * qq][i] * g1, up = v[2 * qq + 1][i] * g1;
              hv[qq] = gt / (1.0f + __expf(-gt)) * up;
            } else {
              const float z = v[qq][i] * g1;
              hv[qq] = z > 0.f ? z * z : 0.f;
            }
          }
          if constexpr (A8) {
            const float mx = row16_max(fmaxf(fabsf(hv[0]), fabsf(hv[1])));
            const int sx = mx_scale_exp(f32_bits(mx));
            L.h8[row][r16] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[0]), sx);
            L.h8[row][16 + r16] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[1]), sx);
            if (r16 == 0) L.hs[row] = (uint32_t)(sx + 127);
          } else if constexpr (RT) {
            const float mx = row16_max(fmaxf(fabsf(hv[0]), fabsf(hv[1])));
            const int sx = mx_scale_exp(f32_bits(mx));
            L.h16[row][r16] = (uint16_t)mx_roundtrip_bf16(hv[0], sx);
            L.h16[row][16 + r16] = (uint16_t)mx_roundtrip_bf16(hv[1], sx);
          } else if constexpr (NVRT) {
            const float gh = p.ah[e];
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const float mx = row16_max(fabsf(hv[qq]));
              const float sc = nv_block_scale(mx, gh), rc = nv_recip(sc, gh);
              L.h16[row][16 * qq + r16] = (uint16_t)bf16_rne(nv_roundtrip(hv[qq], sc, gh, rc));
            }
          } else {
            L.h16[row][r16] = (uint16_t)bf16_rne(hv[0]);
            L.h16[row][16 + r16] = (uint16_t)bf16_rne(hv[1]);
          }
        }
      }
      // every wave's W2 DMA has landed and the h tile is written
      wait_vmem();
      __syncthreads();

      // ---- 4. partial down projection of the slice, a quarter of the W2 fragments per wave.
      // One LDS read gives 4 fragments: lane group q holds the slice's K (32 values) of
      // fragment f + q.  The MFMA with the h tile placed in lane group q only (zeros in
      // the other lane groups) then yields fragment f + q's output rows.
      uint4 hq[4];  // the h tile row r16: bf16 [8 s, 8 s + 8) for s = 0..3, or the codes
      int hsc = 127;
      if constexpr (!A8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) hq[q] = *(const uint4*)&L.h16[r16][8 * q];
      } else {
        hq[0] = *(const uint4*)&L.h8[r16][0];
        hq[1] = *(const uint4*)&L.h8[r16][16];
        hsc = (int)L.hs[r16];
      }
      // output offsets of the lane's rows 4 g + i (column r16 of fragment 0), or out of range
      uint32_t row_off[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = r0 + 4 * g + i;
        row_off[i] = row < m ? (uint32_t)((((int64_t)nth_set_bit(pairs, row) * p.n_slices + j) * p.row_stride + 4 * r16) * 4)
                             : kBufOOB;
      }
      // the 16 operands: h in lane group q, zeros in the others (bf16 path)
      [[maybe_unused]] bf16x8 hvar[4][4];
      if constexpr (!A8) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) hvar[q][s2] = as_bf16x8(g == q ? hq[s2] : L.zero);
      }
      const int per = (p.NF2 + 15) / 16 * 4;  // fragments per wave, a multiple of 4
      const int fb = wave * per, fe = min(p.NF2, fb + per);
      for (int f0 = fb; f0 < fe; f0 += 4) {
        // lane (r16, g) reads fragment f0 + g (fragments past the end repeat the last one)
        const int fq = min(f0 + g, p.NF2 - 1);
        const uint4 bq = *(const uint4*)(w2_lds + fq * 256 + r16 * 16);
        const uint32_t bsw = w2s_lds[fq * 16 + r16];
        f32x4 y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) y[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (!A8) {
          bf16x8 wb[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t dw = s == 0 ? bq.x : s == 1 ? bq.y : s == 2 ? bq.z : bq.w;
            wb[s] = dequant8_bf16<WF>(dw, w_scale<WF>(bsw, kf2, s));
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int q = 0; q < 4; ++q) y[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hvar[q][s], wb[s], y[q], 0, 0, 0);
          }
        } else {
          // fp8 operand: K [32 q, 32 q + 32) sits in lane groups 2 (q & 1) and 2 (q & 1) + 1,
          // first half for q < 2, second half otherwise
          const i32x8 bfr = {(int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w, 0, 0, 0, 0};
          const int sb = (int)((bsw >> (8 * (kf2 & 3))) & 0xFFu);
          const uint4 hv = hq[g & 1];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const bool act = (g >> 1) == (q & 1);
            const uint4 lo = act && (q >> 1) == 0 ? hv : L.zero;
            const uint4 hi = act && (q >> 1) == 1 ? hv : L.zero;
            const i32x8 afr = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            y[q] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr, y[q], 0, 4, 0, g == q ? hsc : 127, 0,
                                                                    sb);
          }
        }
        // lane (r16, g) holds rows 4 g + i of output columns 16 (f0 + q) + r16, q = 0..3:
        // one 16-byte store per row (the partial rows keep the 4 fragments of a group
        // side by side for each column; the combine reads them in that order)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (r0 + i >= m) continue;  // no lane holds a live row i (rows 4 g + i >= i)
          const uint32_t off = row_off[i] != kBufOOB ? row_off[i] + (uint32_t)(64 * f0) : kBufOOB;
          const float4 v = make_float4(y[0][i] * g2, y[1][i] * g2, y[2][i] * g2, y[3][i] * g2);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), part_rsrc, off, 0, 0);
        }
      }
    }
  }
  // no DMA into LDS may still be in flight when the workgroup's LDS is released
  wait_vmem();
}

// out[t] = sum_j w[t, j] * (sum_s part[t k + j][s]) over the valid pairs:
// slices in ascending order, then slots in ascending order, fp32, one bf16
// rounding.  One wave per workgroup; lane (g, j) covers 4 positions of the
// partial rows (columns n of the 4 fragments of a group) for slot j: it loads
// all of the slot's slices, 16 at a time in flight, and sums them.  The lanes
// of the k slots of one position group then meet through lane exchanges, added
// in slot order.  A call with a few tokens thus spreads its partial rows over
// many compute units, with no LDS and no barrier.
constexpr int kSkCombineLoads = 16;
__global__ __launch_bounds__(64) void decode_sk_combine_kernel(const float* __restrict__ part, int64_t part_bytes,
                                                                const int32_t* __restrict__ ids, int E,
                                                                const float* __restrict__ tw, int64_t T, int k,
                                                                int H, int n_slices, int row_stride, int n_groups,
                                                                uint16_t* __restrict__ out, int64_t out_stride) {
  const int lane = threadIdx.x;
  const int PG = 64 / k;                     // position groups per wave (k <= 64)
  const int pg = lane / k, j = lane % k;
  const int64_t t = blockIdx.y;
  const int grp = blockIdx.x * PG + pg;      // 4 positions: fragments 4 G .. 4 G + 3, column n
  const bool in = pg < PG && grp < n_groups;
  const int pos = 4 * grp;
  const int fg = pos >> 6, n = (pos >> 2) & 15;
  const int col = 64 * fg + n;               // output column of fragment 4 G (the first of the 4)
  const BufRsrc rsrc = make_rsrc(part, part_bytes);
  // the slot's id and weight load together with its partial rows; the rows of a
  // dropped pair are read but never added
  const int e = ids[t * k + j];
  const float w = tw[t * k + j];
  const uint32_t base = in ? (uint32_t)((((t * k + j) * n_slices) * (int64_t)row_stride + pos) * 4) : kBufOOB;
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_slices; s0 += kSkCombineLoads) {
    float4 v[kSkCombineLoads];
#pragma unroll
    for (int u = 0; u < kSkCombineLoads; ++u) {
      const uint32_t off = s0 + u < n_slices ? base + (uint32_t)((s0 + u) * row_stride * 4) : kBufOOB;
      v[u] = __builtin_bit_cast(float4, buf_load16(rsrc, off));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kSkCombineLoads; ++u) {
      y.x += v[u].x; y.y += v[u].y; y.z += v[u].z; y.w += v[u].w;
    }
  }
  const bool live = e >= 0 && e < E;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int src0 = pg * k;
  for (int u = 0; u < k; ++u) {  // slot u of this position group, in slot order
    const float yx = __shfl(y.x, src0 + u), yy = __shfl(y.y, src0 + u);
    const float yz = __shfl(y.z, src0 + u), yw = __shfl(y.w, src0 + u);
    const float wu = __shfl(w, src0 + u);
    const int lu = __shfl((int)live, src0 + u);
    if (lu) {
      acc.x = fmaf(wu, yx, acc.x); acc.y = fmaf(wu, yy, acc.y);
      acc.z = fmaf(wu, yz, acc.z); acc.w = fmaf(wu, yw, acc.w);
    }
  }
  if (in && j == 0) {  // columns 64 G + 16 q + n
    const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (col + 16 * q < H) out[t * out_stride + col + 16 * q] = (uint16_t)bf16_rne(a4[q]);
  }
}

// ---------------------------------------------------------------- launch

static SkParams sk_params(const BindingImpl& b) {
  SkParams p = {};
  p.ids = b.ids;
  p.tw = b.tw;
  p.T = (int)b.T;
  p.k = b.k;
  p.E = b.E;
  p.P = (int)(b.T * b.k);
  p.x = b.a;
  p.x_stride = b.a_stride;
  p.x_bytes = ((b.T - 1) * b.a_stride + b.H) * 2;
  p.H = b.H;
  p.I = b.I;
  p.KF1 = (int)b.kf13;
  p.KFS1 = (int)b.kfs13;
  p.KF2 = (int)b.kf2;
  p.KFS2 = (int)b.kfs2;
  p.NF2 = (int)b.nf2;
  p.n_slices = b.I / kSkSlice;
  p.w13c = b.w13_codes;
  p.w13s = b.w13_scales;
  p.g13 = b.w13_global;
  p.w13c_e = b.nf13 * b.kf13 * kFragBytes;
  p.w13s_e = b.nf13 * b.kfs13 * kScaleGroupBytes;
  p.w2c = b.w2_codes;
  p.w2s = b.w2_scales;
  p.g2 = b.w2_global;
  p.w2c_e = b.nf2 * b.kf2 * kFragBytes;
  p.w2s_e = b.nf2 * b.kfs2 * kScaleGroupBytes;
  p.ax = b.a13_global;
  p.ah = b.a2_global;
  p.part = b.y;
  p.row_stride = sk_row_stride(b.H);
  p.part_bytes = b.T * b.k * (int64_t)p.n_slices * p.row_stride * 4;
  return p;
}

size_t sk_dyn_lds(int nf2) { return (size_t)((nf2 + 3) / 4 * 4) * (256 + 64); }

template <int WF, int AF, int MODE, int KW>
static int launch_sk_t(const BindingImpl& b, const SkParams& p, hipStream_t s) {
  static int cache[64];
  auto kernel = decode_sk_kernel<WF, AF, MODE, KW>;
  const size_t lds = sk_dyn_lds(p.NF2);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cache[dev]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecThreads, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cache[dev] = per_cu * device_cu_count();
  }
  const int64_t max_slots = b.T * b.k < b.E ? b.T * b.k : b.E;
  int64_t grid = cache[dev];
  if (grid > max_slots * p.n_slices) grid = max_slots * p.n_slices;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecThreads), lds, s, p);
  return (int)hipGetLastError();
}

template <int WF, int AF, int MODE>
static int launch_sk_kw(const BindingImpl& b, const SkParams& p, hipStream_t s) {
  const int kper = (p.KF1 + 3) / 4;
  if (kper <= 2) return launch_sk_t<WF, AF, MODE, 2>(b, p, s);
  return launch_sk_t<WF, AF, MODE, 4>(b, p, s);
}

template <int MODE>
static int launch_sk_fmt(const BindingImpl& b, const SkParams& p, hipStream_t s) {
  if (a8_native(b.wfmt, b.afmt)) return launch_sk_kw<B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE>(b, p, s);
  if (a8_bf16(b.wfmt, b.afmt)) return launch_sk_kw<B12X_WEIGHT_NVFP4, kActRt, MODE>(b, p, s);
  if (a4_nv(b.afmt)) return launch_sk_kw<B12X_WEIGHT_NVFP4, kActNvRt, MODE>(b, p, s);
  if (b.wfmt == B12X_WEIGHT_NVFP4) return launch_sk_kw<B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE>(b, p, s);
  return launch_sk_kw<B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE>(b, p, s);
}

int launch_decode_sk(const BindingImpl& b, hipStream_t s) {
  const SkParams p = sk_params(b);
  return b.gated ? launch_sk_fmt<1>(b, p, s) : launch_sk_fmt<2>(b, p, s);
}

int launch_decode_sk_combine(const BindingImpl& b, hipStream_t s) {
  if (b.T == 0) return 0;
  const int row_stride = sk_row_stride(b.H);
  const int n_groups = (row_stride - kSkRowPad) / 4;
  const int per_wave = 64 / b.k;
  const dim3 grid((unsigned)((n_groups + per_wave - 1) / per_wave), (unsigned)b.T);
  const int64_t part_bytes = b.T * b.k * (int64_t)(b.I / kSkSlice) * row_stride * 4;
  hipLaunchKernelGGL(decode_sk_combine_kernel, grid, dim3(64), 0, s, (const float*)b.y, part_bytes, b.ids, b.E, b.tw,
                     b.T, b.k, b.H, b.I / kSkSlice, row_stride, n_groups, b.out, b.out_stride);
  return (int)hipGetLastError();
}

}  // namespace b12x
