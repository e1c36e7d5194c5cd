// Split-K decode kernel of the fused MoE for the smallest batches (b12x
// README "What's in here": the micro-kernel decode path of fused_moe).
//
// With a handful of routing pairs the cost of a call is latency, not
// bandwidth: the down projection of the plain two-phase order cannot start
// before the whole h of its expert exists.  Here the intermediate dimension
// is cut into slices of 32 columns and one workgroup owns one (touched expert,
// slice) item from start to end:
//   1. its 4 waves split K of the slice's gate/up (or w1) rows; each wave
//      issues all of its weight loads at once, then the DMA of the slice's W2
//      columns (one 32-wide lane group of every W2 fragment, codes and
//      scales) into LDS, which lands while the rest runs;
//   2. each wave stages the activation rows of the item's pairs over its own
//      K range in its own LDS region, converted once per value: bf16, the
//      exact MXFP8 / NVFP4 round trips as bf16, or MXFP8 codes and scales for
//      the scaled fp8 x fp4 MFMA; the MFMAs read their activation operand
//      from there;
//   3. the split-K partial sums meet in LDS in a fixed wave order, wave 0
//      applies the activation and the requantization of h (bf16, or the
//      bf16 value of its MXFP8 / NVFP4 round trip) and leaves the h tile in
//      LDS;
//   4. the 4 waves multiply the h tile by the W2 slice from LDS, one bf16
//      MFMA per W2 fragment (each wave a quarter of the output rows), and
//      write fp32 partial rows part[pair][slice][H].
// No workgroup waits for another, so the result does not depend on which
// workgroups are resident.  The combine (decode_sk_combine_kernel) sums the
// slices of each pair and the pairs of each token in a fixed order, in fp32,
// and rounds once to bf16.
#include <mutex>

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
  int oai;            // gated: SwiGLU-OAI instead of SiLU
  float* part;        // [P][n_slices][row_stride]: per fragment group G (4 fragments), column n,
                      // fragment q: position 64 G + 4 n + q
  int64_t part_bytes;
  int row_stride;     // 64 per fragment group + 64: consecutive rows start on different memory channels
  int R;              // activation rows per tile (pairs of one expert processed together), <= kSkRows
  int kper;           // W13 K fragments per wave
  int xs;             // bytes per staged activation row
  int xsc;            // offset of the staged E8M0 scales in a wave's region (MXFP8 codes)
  int xwb;            // bytes of one wave's LDS region
  int x_off;          // offset of the wave regions in the dynamic LDS
  LiveT lv;           // token count (T; or the live one)
};

// Static LDS of one workgroup: routing and the h tile.  The dynamic part holds
// the W2 slice (codes [NF2][256], scales [NF2][16] dwords, NF2 rounded up to
// a multiple of 4) and one region per wave: that wave's staged activation
// rows (row 0 all zeros for the rows outside the tile, rows 1..R the tile's
// rows), which after its gate/up MFMAs holds its split-K partial sums.
struct SkLds {
  uint32_t bits[4][32];         // each wave's copy of the touched-expert bitmap
  alignas(16) uint16_t h16[16][kSkSlice];  // h tile, bf16 (16 rows x 32 columns)
};
constexpr int kSkRows = 4;       // largest tile (rows staged per wave region)

template <int WF>
__device__ __forceinline__ float w_scale(uint32_t word, int kf, int s) {
  if constexpr (WF == B12X_WEIGHT_MXFP4) return e8m0_as_scale((word >> (8 * (kf & 3))) & 0xFFu);
  else return e4m3_value((word >> (8 * (2 * (kf & 1) + (s >> 1)))) & 0xFFu);
}

// The bf16 operand of 8 activations from 4 dwords of bf16 values.
__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Largest bf16 magnitude (bits) of the 8 values of a unit.
__device__ __forceinline__ uint32_t unit_amax(const uint4& v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
  return m;
}
// max with lane ^ 1 (DPP quad permute [1, 0, 3, 2]) and with lane ^ 2 ([2, 3, 0, 1])
__device__ __forceinline__ uint32_t max_lane_xor1(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t max_lane_xor2(uint32_t v) {
  return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
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

__device__ __forceinline__ SkRoute sk_route(const SkParams& p, int P, uint32_t* wbits) {
  const int lane = threadIdx.x & 63;
  SkRoute r;
  int id = -1;
  if (lane < P) {
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
  constexpr int GK = WF == B12X_WEIGHT_MXFP4 ? 4 : 2;  // K fragments per scale group
  __shared__ SkLds L;
  extern __shared__ __attribute__((aligned(1024))) uint8_t dyn[];
  const int nf2r = (p.NF2 + 3) / 4 * 4;
  uint8_t* const w2_lds = dyn;
  uint32_t* const w2s_lds = (uint32_t*)(dyn + (size_t)nf2r * 256);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  uint8_t* const xw = dyn + p.x_off + wave * p.xwb;  // this wave's region
  if (!p.lv.on()) return;
  const SkRoute route = sk_route(p, (int)(p.lv.tokens() * p.k), L.bits[wave]);
  const int items = route.n_touched * p.n_slices;
  const int kb = wave * p.kper, ke = min(p.KF1, kb + p.kper);
  const int nu = p.kper * 16;         // activation units per staged row
  const BufRsrc x_rsrc = make_rsrc(p.x, p.x_bytes);
  const BufRsrc part_rsrc = make_rsrc(p.part, p.part_bytes);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int slot = item / p.n_slices, j = item - slot * p.n_slices;
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
      const int n_dma = nf2r / 4;  // each DMA instruction: 4 fragments x 16 lanes
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

    for (int r0 = 0; r0 < m; r0 += p.R) {
      const int live = min(p.R, m - r0);  // rows of this tile
      // tokens of the tile's rows (wave-uniform)
      int pr[kSkRows], tok[kSkRows];
#pragma unroll
      for (int r = 0; r < kSkRows; ++r) {
        pr[r] = r < live ? nth_set_bit(pairs, r0 + r) : 0;
        tok[r] = pr[r] / p.k;
      }
      // this lane's staged row in the MFMA operand: r16 + 1, or the zero row 0
      const int xrow = r16 < live ? r16 + 1 : 0;

      // ---- 1./2. gate/up (or w1) over this wave's K range, KW fragments at a time
      f32x4 acc[NF1];
#pragma unroll
      for (int f = 0; f < NF1; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int c0 = kb; c0 < ke; c0 += KW) {
        uint4 q[KW][NF1];
        // scale words: one per fragment and scale group; the chunk spans at most NG groups
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
#pragma unroll
          for (int f = 0; f < NF1; ++f)
            q[i][f] = buf_load16(b_rsrc, v ? (uint32_t)(((f1 + f) * p.KF1 + kf) * kFragBytes + lane * 16) : kBufOOB);
        }
        __builtin_amdgcn_sched_barrier(0);  // the chunk's loads are all in flight before any MFMA waits
        if (c0 == kb) {
          // activation units of the tile over the wave's K range: lane unit (r, i) = row r,
          // values 8 c .. 8 c + 7 of the wave's K range, c = lane + 64 i (nu <= 128);
          // loaded after the weights, so the conversion below waits for everything
          // issued so far
          uint4 xv[kSkRows][2];
#pragma unroll
          for (int r = 0; r < kSkRows; ++r)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              const int c = lane + 64 * i;
              const int kk = kb * kFragK + 8 * c;
              const bool v = r < live && c < nu && kk < p.H;
              xv[r][i] = buf_load16(x_rsrc, v ? (uint32_t)(((int64_t)tok[r] * p.x_stride + kk) * 2) : kBufOOB);
            }
          if (!dma_issued) {
            issue_w2_dma();
            dma_issued = true;
          }
          __builtin_amdgcn_sched_barrier(0);
          // zero row, then the tile's rows, converted once per value
          if constexpr (!A8) {
            for (int c = lane; c < nu; c += 64) *(uint4*)(xw + 16 * c) = make_uint4(0, 0, 0, 0);
          } else {
            for (int c = lane; c < nu / 2; c += 64) *(uint4*)(xw + 16 * c) = make_uint4(0, 0, 0, 0);
            if (lane < p.kper) *(uint32_t*)(xw + p.xsc + 4 * lane) = 0u;
          }
#pragma unroll
          for (int r = 0; r < kSkRows; ++r) {
            if (r >= p.R) break;  // wave-uniform
#pragma unroll
            for (int i = 0; i < 2; ++i) {
              if (64 * i >= nu) break;  // wave-uniform
              const int c = lane + 64 * i;
              const bool in = c < nu;
              uint4 v = xv[r][i];
              if constexpr (A8) {
                // one E8M0 block = 4 units = 4 neighbouring lanes
                const uint32_t amax = max_lane_xor2(max_lane_xor1(unit_amax(v)));
                const int sx = mx_scale_exp(amax << 16);
                const MxScale ms = mx_scale(sx);
                const uint2 cw = make_uint2(e4m3_codes4_bf16(v.x, v.y, ms), e4m3_codes4_bf16(v.z, v.w, ms));
                if (in) {
                  *(uint2*)(xw + (r + 1) * p.xs + 8 * c) = cw;
                  if ((c & 3) == 0) xw[p.xsc + (r + 1) * p.kper * 4 + (c >> 2)] = (uint8_t)(sx + 127);
                }
              } else {
                if constexpr (RT) {
                  const uint32_t amax = max_lane_xor2(max_lane_xor1(unit_amax(v)));
                  const int sx = mx_scale_exp(amax << 16);
                  uint32_t* w = (uint32_t*)&v;
#pragma unroll
                  for (int h = 0; h < 4; ++h)
                    w[h] = mx_roundtrip_bf16(bf16_to_f32(w[h] & 0xFFFFu), sx) |
                           (mx_roundtrip_bf16(bf16_to_f32(w[h] >> 16), sx) << 16);
                }
                if constexpr (NVRT) {  // one NVFP4 block = 2 units
                  const float ga = p.ax[0];
                  const uint32_t amax = max_lane_xor1(unit_amax(v));
                  const float sc = nv_block_scale(bits_f32(amax << 16), ga), rc = nv_recip(sc, ga);
                  uint32_t* w = (uint32_t*)&v;
#pragma unroll
                  for (int h = 0; h < 4; ++h)
                    w[h] = bf16_rne(nv_roundtrip(bf16_to_f32(w[h] & 0xFFFFu), sc, ga, rc)) |
                           (bf16_rne(nv_roundtrip(bf16_to_f32(w[h] >> 16), sc, ga, rc)) << 16);
                }
                if (in) *(uint4*)(xw + (r + 1) * p.xs + 16 * c) = v;
              }
            }
          }
        }
        // the chunk's MFMAs; a wave's LDS operations complete in order, so its staged
        // rows are visible to its own reads
#pragma unroll
        for (int i = 0; i < KW; ++i) {
          const int kf = c0 + i;
          if (kf >= ke) break;  // wave-uniform
          const int kl = kf - kb;
          // scale words of this K fragment (selected here, where the loads are waited
          // for anyway, not at issue time)
          const int su = kf / GK - sg0;  // 0 .. NG-1, wave-uniform
          uint32_t bs[NF1];
#pragma unroll
          for (int f = 0; f < NF1; ++f) {
            bs[f] = sw[0][f];
#pragma unroll
            for (int u = 1; u < NG; ++u) bs[f] = su == u ? sw[u][f] : bs[f];
          }
          if constexpr (!A8) {
            const uint8_t* xa = xw + xrow * p.xs + kl * 256 + g * 64;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x8 a = as_bf16x8(*(const uint4*)(xa + 16 * s));
#pragma unroll
              for (int f = 0; f < NF1; ++f) {
                const uint32_t dw = s == 0 ? q[i][f].x : s == 1 ? q[i][f].y : s == 2 ? q[i][f].z : q[i][f].w;
                acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dequant8_bf16<WF>(dw, w_scale<WF>(bs[f], kf, s)),
                                                                 acc[f], 0, 0, 0);
              }
            }
          } else {
            // fp8 operand of lane (r16, g): K 16 g + [0, 16) and 64 + 16 g + [0, 16) of the
            // fragment; its scale operand is the E8M0 scale of K block g
            const uint8_t* xa = xw + xrow * p.xs + kl * kFragK + 16 * g;
            const uint4 lo = *(const uint4*)xa, hi = *(const uint4*)(xa + 64);
            const int sa = xw[p.xsc + xrow * p.kper * 4 + kl * 4 + g];
            const i32x8 afr = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
            for (int f = 0; f < NF1; ++f) {
              const i32x8 bfr = {(int)q[i][f].x, (int)q[i][f].y, (int)q[i][f].z, (int)q[i][f].w, 0, 0, 0, 0};
              const int sb = (int)((bs[f] >> (8 * (kf & 3))) & 0xFFu);
              acc[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr, acc[f], 0, 4, 0, sa, 0, sb);
            }
          }
        }
      }

      if (!dma_issued) {
        issue_w2_dma();
        dma_issued = true;
      }
      // ---- 3. split-K sums in wave order (waves 1..3 leave theirs in their own regions),
      // activation and requantization of h by wave 0
      if (wave != 0) {
#pragma unroll
        for (int f = 0; f < NF1; ++f) *(f32x4*)(xw + f * 1024 + lane * 16) = acc[f];
      }
      __syncthreads();
      if (wave == 0) {
        f32x4 v[NF1];
#pragma unroll
        for (int f = 0; f < NF1; ++f) {
          v[f] = acc[f];
#pragma unroll
          for (int w = 1; w < 4; ++w) v[f] += *(const f32x4*)(dyn + p.x_off + w * p.xwb + f * 1024 + lane * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * g + i;
          float hv[2];  // columns r16 and 16 + r16 of the slice
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            if constexpr (GATED) {
              const float gt = v[2 * qq][i] * g1, up = v[2 * qq + 1][i] * g1;
              hv[qq] = p.oai ? swiglu_oai(gt, up) : gt / (1.0f + __expf(-gt)) * up;
            } else {
              const float z = v[qq][i] * g1;
              hv[qq] = z > 0.f ? z * z : 0.f;
            }
          }
          if constexpr (A8 || RT) {  // bf16 value of the MXFP8 round trip (exact)
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

      // ---- 4. partial down projection of the slice, a quarter of the W2 fragments per
      // wave: A = the h tile (lane (r16, g): row r16, K 8 g ..), B = fragment f's slice
      // (lane (n, g): dword g of row n, K 8 g ..), one MFMA per fragment
      const bf16x8 hA = as_bf16x8(*(const uint4*)&L.h16[r16][8 * g]);
      // output offsets of the lane's rows 4 g + i (column r16 of fragment 0), or out of
      // range: the tile's live rows (at most kSkRows = 4) are rows 0..3, in lane group 0
      static_assert(kSkRows <= 4, "the live rows of a tile sit in lane group 0");
      uint32_t row_off[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        row_off[i] = g == 0 && i < live ? (uint32_t)((((int64_t)pr[i] * p.n_slices + j) * p.row_stride + 4 * r16) * 4)
                                        : kBufOOB;
      const int per = (p.NF2 + 15) / 16 * 4;  // fragments per wave, a multiple of 4
      const int fb = wave * per, fe = min(p.NF2, fb + per);
      const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
      constexpr int FB = 16;  // fragments per batch: their LDS reads are all issued first
      for (int f00 = fb; f00 < fe; f00 += FB) {
        uint32_t dw[FB], bsw[FB];
#pragma unroll
        for (int qf = 0; qf < FB; ++qf) {
          const int f = min(f00 + qf, p.NF2 - 1);  // fragments past the end repeat the last one
          dw[qf] = *(const uint32_t*)(w2_lds + f * 256 + r16 * 16 + g * 4);
          bsw[qf] = w2s_lds[f * 16 + r16];
        }
#pragma unroll
        for (int b4 = 0; b4 < FB / 4; ++b4) {
          const int f0 = f00 + 4 * b4;
          if (f0 >= fe) break;  // wave-uniform
          f32x4 y[4];
#pragma unroll
          for (int qf = 0; qf < 4; ++qf)
            y[qf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                hA, dequant8_bf16<WF>(dw[4 * b4 + qf], w_scale<WF>(bsw[4 * b4 + qf], kf2, g)), zero4, 0, 0, 0);
          // lane (r16, g) holds rows 4 g + i of output columns 16 (f0 + q) + r16, q = 0..3:
          // one 16-byte store per row (the partial rows keep the 4 fragments of a group
          // side by side for each column; the combine reads them in that order)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (i >= live) continue;  // no lane holds a live row i (rows 4 g + i >= i)
            const uint32_t off = row_off[i] != kBufOOB ? row_off[i] + (uint32_t)(64 * f0) : kBufOOB;
            const float4 v = make_float4(y[0][i] * g2, y[1][i] * g2, y[2][i] * g2, y[3][i] * g2);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), part_rsrc, off, 0, 0);
          }
        }
      }
    }
  }
  // no DMA into LDS may still be in flight when the workgroup's LDS is released
  wait_vmem();
}

// out[t] = sum_j w[t, j] * (sum_s part[t k + j][s]) over the valid pairs, in
// fp32 with one bf16 rounding.  One wave per workgroup; lane (g, j, u) covers
// 4 positions of the partial rows (column n of the 4 fragments of a group G)
// for slot j and part u of the slices: it loads the slices
// [u c, u c + c) of its pair (c = ceil(slices / S)), 16 at a time in flight,
// and sums them in ascending order.  The S parts of a slot are then added in
// part order and the slots in slot order through lane exchanges, so the sum
// order is fixed by (k, S, number of slices) alone.  A call with a few tokens
// thus spreads its partial rows over many compute units, each lane with few
// loads, and with no LDS and no barrier.
constexpr int kSkCombineLoads = 16;
__global__ __launch_bounds__(64) void decode_sk_combine_kernel(const float* __restrict__ part, int64_t part_bytes,
                                                                const int32_t* __restrict__ ids, int E,
                                                                const float* __restrict__ tw, LiveT lv, int k,
                                                                int S, int H, int n_slices, int row_stride,
                                                                int n_groups, uint16_t* __restrict__ out,
                                                                int64_t out_stride) {
  if (!lv.on() || (int64_t)blockIdx.y >= lv.tokens()) return;
  const int lane = threadIdx.x;
  const int KS = k * S;                      // lanes per position group (<= 64)
  const int PG = 64 / KS;                    // position groups per wave
  const int pg = lane / KS, j = (lane % KS) / S, u = lane % S;
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
  const int c = (n_slices + S - 1) / S;
  const int s_beg = u * c, s_end = min(n_slices, s_beg + c);
  const uint32_t base = in ? (uint32_t)((((t * k + j) * n_slices) * (int64_t)row_stride + pos) * 4) : kBufOOB;
  float4 y = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = s_beg; s0 < s_end; s0 += kSkCombineLoads) {
    float4 v[kSkCombineLoads];
#pragma unroll
    for (int q = 0; q < kSkCombineLoads; ++q) {
      const uint32_t off = s0 + q < s_end ? base + (uint32_t)((s0 + q) * row_stride * 4) : kBufOOB;
      v[q] = __builtin_bit_cast(float4, buf_load16(rsrc, off));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kSkCombineLoads; ++q) {
      y.x += v[q].x; y.y += v[q].y; y.z += v[q].z; y.w += v[q].w;
    }
  }
  // parts of this lane's slot, in part order (every lane of the slot gets the sum)
  const int src_j = pg * KS + j * S;
  float4 ys = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int q = 0; q < S; ++q) {
    ys.x += __shfl(y.x, src_j + q); ys.y += __shfl(y.y, src_j + q);
    ys.z += __shfl(y.z, src_j + q); ys.w += __shfl(y.w, src_j + q);
  }
  const bool live = e >= 0 && e < E;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int src0 = pg * KS;
  for (int q = 0; q < k; ++q) {  // slot q of this position group, in slot order
    const int src = src0 + q * S;
    const float yx = __shfl(ys.x, src), yy = __shfl(ys.y, src);
    const float yz = __shfl(ys.z, src), yw = __shfl(ys.w, src);
    const float wq = __shfl(w, src);
    const int lq = __shfl((int)live, src);
    if (lq) {
      acc.x = fmaf(wq, yx, acc.x); acc.y = fmaf(wq, yy, acc.y);
      acc.z = fmaf(wq, yz, acc.z); acc.w = fmaf(wq, yw, acc.w);
    }
  }
  if (in && j == 0 && u == 0) {  // columns 64 G + 16 q + n
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
  p.lv = b.live();
  p.oai = b.oai;
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
  // LDS: the W2 slice, then one region per wave (staged activation rows: a zero row
  // and R rows over the wave's K range, bf16 or MXFP8 codes plus their scales; at
  // least the wave's split-K partial sums)
  const bool codes = a8_native(b.wfmt, b.afmt);
  p.R = (int)(b.T < kSkRows ? (b.T > 0 ? b.T : 1) : kSkRows);
  p.kper = (p.KF1 + 3) / 4;
  const int kw = p.kper * kFragK;
  p.xs = codes ? kw + 32 : 2 * kw + 32;
  p.xsc = (p.R + 1) * p.xs;
  int bytes = p.xsc + (codes ? (p.R + 1) * p.kper * 4 : 0);
  if (bytes < (b.gated ? 4 : 2) * 1024) bytes = (b.gated ? 4 : 2) * 1024;
  p.xwb = (bytes + 15) / 16 * 16;
  p.x_off = (p.NF2 + 3) / 4 * 4 * (256 + 64);
  return p;
}

static size_t sk_dyn_lds(const SkParams& p) { return (size_t)p.x_off + 4 * (size_t)p.xwb; }

template <int WF, int AF, int MODE, int KW>
static int launch_sk_t(const BindingImpl& b, const SkParams& p, hipStream_t s) {
  // resident workgroups per device, for the LDS size they were computed with
  static int cache[64];
  static size_t cache_lds[64];
  auto kernel = decode_sk_kernel<WF, AF, MODE, KW>;
  const size_t lds = sk_dyn_lds(p);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cache[dev] || cache_lds[dev] != lds) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecThreads, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cache_lds[dev] = lds;
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
  // a wave holds up to 4 K fragments of the 4 gate/up fragment rows, or 8 of the 2 w1 rows
  if constexpr (MODE == 1) {
    return launch_sk_t<WF, AF, MODE, 4>(b, p, s);
  } else {
    if (p.kper <= 4) return launch_sk_t<WF, AF, MODE, 4>(b, p, s);
    return launch_sk_t<WF, AF, MODE, 8>(b, p, s);
  }
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
  // the staging holds up to kSkRows rows of at most 128 units (8 K fragments) per wave
  if (p.R > kSkRows || p.kper > 8) return (int)hipErrorInvalidValue;
  return b.gated ? launch_sk_fmt<1>(b, p, s) : launch_sk_fmt<2>(b, p, s);
}

uint64_t sk_partial_bytes(const BindingImpl& b) {
  return (uint64_t)(b.T * b.k) * (uint64_t)(b.I / kSkSlice) * (uint64_t)sk_row_stride(b.H) * 4u;
}

// Scratch of the allocation-free call (b12x_moe_run_noalloc): the split-K partial
// rows, in a static array that every device the library runs on holds until the
// process ends.  In host code `scratch` only names the symbol: its device address
// is looked up with hipGetSymbolAddress, once per device with that device current,
// and that address (never the array's name) is what the kernels receive.
static __device__ __align__(256) uint8_t scratch[B12X_NOALLOC_SCRATCH_BYTES];
static void* g_scratch_ptr[64];
static std::mutex g_scratch_mu;

int sk_static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= 64) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

int launch_decode_sk_combine(const BindingImpl& b, hipStream_t s) {
  if (b.T == 0) return 0;
  const int row_stride = sk_row_stride(b.H);
  const int n_groups = (row_stride - kSkRowPad) / 4;
  const int n_slices = b.I / kSkSlice;
  // split the slices of a slot over S lanes: k * S = 16 lanes per position group where
  // the slices allow (4 position groups, 64 contiguous bytes of each row per wave, the
  // fastest measured at top-4 and top-8), more while a lane would wait for more than
  // two rounds of loads
  int S = 1;
  while (b.k * S < 16 && S < n_slices) S *= 2;
  while (b.k * S * 2 <= 64 && (n_slices + S - 1) / S > 2 * kSkCombineLoads) S *= 2;
  const int per_wave = 64 / (b.k * S);
  const dim3 grid((unsigned)((n_groups + per_wave - 1) / per_wave), (unsigned)b.T);
  const int64_t part_bytes = b.T * b.k * (int64_t)n_slices * row_stride * 4;
  hipLaunchKernelGGL(decode_sk_combine_kernel, grid, dim3(64), 0, s, (const float*)b.y, part_bytes, b.ids, b.E, b.tw,
                     b.live(), b.k, S, b.H, n_slices, row_stride, n_groups, b.out, b.out_stride);
  return (int)hipGetLastError();
}

}  // namespace b12x
