// Small-batch decode path of the fused MoE (b12x README "What's in here": the
// micro-kernel decode path of fused_moe).  For T*k <= kDecodePairs these
// kernels replace the routing buffers and the grouped GEMMs; every touched
// expert's weights are read exactly once:
//   D1 (gate/up) and D2 (down): a grid of at most as many workgroups as the
//      chip holds at once.  Every workgroup reads topk_ids into LDS, finds the
//      touched experts (a bitmap and its prefix popcounts) and takes its share
//      of the items (touched expert in ascending id, group of FR weight
//      fragments): one contiguous share, or chunks of items dealt round-robin
//      when there are at least two per workgroup; for each expert of its share
//      it builds that expert's pair list (stable by pair id).  Its 4 waves
//      split K, keep their share of the activation rows in registers and take
//      the groups one at a time (the other resident waves cover the load
//      latency); wave 0 adds the other waves' partial sums from LDS to its own
//      in a fixed wave order.  D1 applies SiLU-gated or ReLU^2 and writes h by
//      pair id (bf16, MXFP8 codes and scales for W4A8, or the bf16 value of an
//      MXFP8 / NVFP4 round trip with NVFP4 weights); D2 writes y by pair id in
//      fp32.
//   With 16-bit activations D1 and D2 run as one kernel: each workgroup does
//      its gate/up share, publishes each finished group with a completion
//      flag, then does its down share, waiting (bounded) for the flags of the
//      gate/up groups of each expert it reaches.  Other formats launch D1 and
//      D2 separately.
//   D3 (combine): out[t] = sum_j w[t,j] * y[t*k+j] in ascending slot order,
//      fp32, one bf16 rounding (the grouped path's combine kernel, reading y
//      by pair id).
// No atomics on data: every value is computed by one workgroup in a fixed
// order, so the result does not depend on scheduling or on the grid size.
#include "decode_common.h"

namespace b12x {

struct DecodeParams {
  const int32_t* ids;
  const float* tw;
  int T, k, E, P;
  // A operand: bf16 rows or MXFP8 codes + scales, indexed by token (D1) or pair (D2)
  const uint16_t* a16;
  const uint8_t* a8;
  const uint8_t* as;
  int64_t a_stride;   // elements (bf16) or bytes (codes)
  int64_t as_stride;  // bytes
  int64_t a_bytes, as_bytes;  // extents of a16 / a8 and as (at most 1 GiB)
  int a_by_token;
  int64_t K;
  int KF;
  // B operand (prepared weights)
  const uint8_t* bcodes;
  const uint8_t* bscales;
  const float* bglobal;
  // NVFP4 activations: activation scale applied with bglobal (x: one value;
  // h: one per expert, aglobal_per_expert = 1) and the scale of each expert's
  // h for the gate/up epilogue's requantization
  const float* aglobal;
  int aglobal_per_expert;
  const float* hglobal;
  int oai;  // gated: SwiGLU-OAI instead of SiLU
  int64_t b_codes_expert, b_scales_expert;
  int NF, KFS;
  int n_groups;  // fragment groups per expert
  // D1 outputs
  uint16_t* h16;
  uint8_t* h8;
  uint8_t* hs;
  int64_t h_stride, hs_stride;
  // D2 output
  float* y;
  int64_t y_stride;
  // fused gate/up + down (one launch): completion flag of every (touched
  // expert slot, gate/up group), flags_per_slot of them per slot; a flag
  // holds the launch's tag once that group's h rows are stored.  Every
  // workgroup reads the launch counter when it starts and adds its share of
  // kLaunchStep when it is done, so each launch has a tag of its own.  A
  // wait that has polled max_polls times computes the groups still missing
  // itself.
  uint64_t* flags;
  int flags_per_slot;
  uint64_t* counter;
  uint64_t expect_xor;  // 0; the test hook's waits expect tag ^ expect_xor, which no flag holds
  int max_polls;
  int64_t h_bytes;  // extent of h16 (device-coherent stores and loads)
  int deal;         // 0: one contiguous share per workgroup; else chunks of this many items dealt round-robin
  int prev_groups;  // down phase of the fused kernel: the gate/up phase's groups per expert (same deal)
  LiveT lv;         // token count (T; or the live one)
};

enum { DMODE_SILU = 1, DMODE_RELU2 = 2, DMODE_DOWN = 3 };

// Tag of this launch's completion flags: decode_tag of the launch number,
// the counter's value in units of kLaunchStep.
__device__ __forceinline__ uint64_t flag_tag(const uint64_t* counter) {
  return decode_tag((uint32_t)(__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >> kLaunchShift));
}

// Polls of one wait before the waiting workgroup computes the missing groups
// itself (each poll is a round trip to memory plus a sleep, about a
// microsecond: some hundred times the longest wait measured with the whole
// grid resident).
constexpr int kWaitPolls = 1 << 11;

// No fallback: the plain decode kernels and the fused kernel's own gate/up phase.
struct NoFallback {
  __device__ void operator()(int, uint64_t) const {}
};

// This workgroup's share of the (touched expert slot, group of FR weight
// fragments) items of one GEMV.  FUSE = 0: a launch of its own.  FUSE = 1:
// the gate/up phase of the fused kernel: h is stored device-coherent and
// each finished group raises its flag.  FUSE = 2: the down phase: before an
// expert's part, wave 0 waits until every gate/up group of that expert has
// raised its flag, and h is loaded device-coherent; a wait that runs out of
// polls hands the groups still missing to fallback(slot, mask), which
// computes them in this workgroup.  FUSE = 3: that fallback, gate/up items
// [lo_in, hi_in) of one slot computed as in FUSE = 1.  A group computed
// twice (by its owner and by a waiter that gave up on it) is stored twice
// with the same bytes: the computation does not depend on who runs it.
template <int WF, int AF, int MODE, int FR, int KW, int FUSE, typename Fallback>
__device__ __forceinline__ void decode_items(const DecodeParams& p, DecodeLds& L, f32x4* red, int n_touched,
                                             uint64_t tag, int P, int lo_in, int hi_in, const Fallback& fallback) {
  constexpr bool GU = FUSE == 1 || FUSE == 3;  // a gate/up phase of the fused kernel
  constexpr bool A8 = AF == B12X_ACT_MXFP8;
  constexpr bool RT = AF == kActRt;  // bf16 MXFP8 round trips: h stored as its own round trip
  constexpr bool NVRT = AF == kActNvRt;  // bf16 NVFP4 round trips: h stored as its own NVFP4 round trip
  static_assert(FUSE == 0 || !A8, "the fused kernel runs 16-bit activations");
  static_assert(FUSE == 0 || (!RT && !NVRT), "the fused kernel stores plain bf16 h");
  static_assert(!GU || MODE != DMODE_DOWN, "phase 1 is gate/up");
  static_assert(FUSE != 2 || MODE == DMODE_DOWN, "phase 2 is down");
  int* const s_ids = L.ids;
  int* const s_rows = L.rows;
  uint32_t* const s_bits = L.bits;
  int* const s_wpre = L.wpre;
  int* const s_info = L.info;
  // split-K partials of waves 1..3 (wave 0 keeps its own in registers and sums)
  auto s_red = [&](int par, int w, int j) -> f32x4& {
    return red[((par * 3 + (w - 1)) * FR + j) * 64 + (threadIdx.x & 63)];
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;

  // this workgroup's share of the (touched expert, fragment group) items
  const int64_t items = (int64_t)n_touched * p.n_groups;
  int lo, hi;
  // With at least p.deal items per workgroup: chunks of p.deal consecutive
  // items dealt round-robin (chunk c to workgroup c % grid).  Otherwise (and
  // with p.deal = 0) one contiguous share per workgroup.
  const int deal = FUSE != 3 && p.deal && items >= (int64_t)p.deal * gridDim.x ? p.deal : 0;
  // When the gate/up phase dealt between one and two rounds of chunks, its
  // first C1 % grid workgroups took two chunks and the others one.  The down
  // phase then continues that deal (its chunk c goes to workgroup
  // (C1 + c) % grid), so the workgroups with one gate/up chunk take the first
  // down chunks instead of leaving a few workgroups with two of each at the
  // end.  With more gate/up rounds the imbalance is a small share and the
  // down phase deals from workgroup 0.
  int chunk_id = (int)blockIdx.x;
  if (FUSE == 2 && deal) {
    const int64_t prev = (int64_t)n_touched * p.prev_groups;
    const int64_t c1 = (prev + deal - 1) / deal;
    if (c1 >= (int64_t)gridDim.x && c1 < 2 * (int64_t)gridDim.x) {
      const int start = (int)(c1 - gridDim.x);
      chunk_id = ((int)blockIdx.x - start + (int)gridDim.x) % (int)gridDim.x;
    }
  }
  if (FUSE == 3) {
    lo = lo_in;
    hi = hi_in;
  } else if (deal) {
    lo = chunk_id * deal;
    hi = (int)min(items, (int64_t)lo + deal);
  } else {  // one contiguous share
    lo = (int)(items * blockIdx.x / gridDim.x);
    hi = (int)(items * (blockIdx.x + 1) / gridDim.x);
  }

  // ---- this wave's K fragments
  const int kper = (p.KF + 3) / 4;
  const int kb = wave * kper, ke = min(p.KF, kb + kper);

  int par = 0;  // s_red buffer of the current group
  for (;;) {
  for (int item = lo; item < hi;) {
  // ---- one expert's part of the share: groups [g_begin, g_end) of `slot`
  const int slot = item / p.n_groups;
  const int g_begin = item - slot * p.n_groups;
  const int g_end = min(p.n_groups, g_begin + (hi - item));
  item += g_end - g_begin;
  if constexpr (FUSE == 2) {
    // wave 0 waits until every gate/up group of this expert has raised its
    // flag; should its polls run out (a producer not resident, the device
    // shared with other work), the groups still missing are computed here
    if (wave == 0) {
      const uint64_t* f = p.flags + (int64_t)slot * p.flags_per_slot;
      const uint64_t expect = tag ^ p.expect_xor;
      uint64_t miss = 0;
      for (int poll = 0;; ++poll) {
        const bool ok = lane >= p.flags_per_slot ||
                        __hip_atomic_load(f + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == expect;
        miss = __ballot(!ok);
        if (miss == 0 || poll >= p.max_polls) break;
        __builtin_amdgcn_s_sleep(8);
      }
      if (lane == 0) {  // published by the barrier that opens decode_expert
        s_info[2] = (int)(uint32_t)miss;
        s_info[3] = (int)(uint32_t)(miss >> 32);
      }
    }
  }
  int e;
  const int m = decode_expert(P, p.E, slot, s_ids, s_bits, s_wpre, s_rows, s_info, e);
  if constexpr (FUSE == 2) {
    const uint64_t miss = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(s_info[2]) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane(s_info[3]) << 32);
    if (miss) {
      // (it rebuilds this slot's pair list in LDS, the same one, and ends with wave 0
      // waiting for its h stores, which the barrier then orders before this part's h loads)
      fallback(slot, miss);
      __syncthreads();
    }
  }
  const uint8_t* bcodes = p.bcodes + (int64_t)e * p.b_codes_expert;
  const uint8_t* bscales = p.bscales + (int64_t)e * p.b_scales_expert;
  float gsc = p.bglobal ? p.bglobal[e] : 1.0f;
  if (p.aglobal) gsc *= p.aglobal[p.aglobal_per_expert ? e : 0];

  // raw buffer loads: a fragment outside the wave's K range or the expert's
  // matrix (the resources end with the expert) reads zeros, so no load is
  // behind a branch
  const BufRsrc b_rsrc = make_rsrc(bcodes, p.b_codes_expert);
  const BufRsrc bs_rsrc = make_rsrc(bscales, p.b_scales_expert);
  auto load_b = [&](uint4 (&bq)[FR][KW], uint32_t (&bs)[FR][KW], int grp) {
    const uint32_t cb = (uint32_t)(grp * FR * p.KF * kFragBytes);
    const uint32_t sb = (uint32_t)(grp * FR * p.KFS * kScaleGroupBytes);
#pragma unroll
    for (int j = 0; j < FR; ++j) {
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        const int kf = kb + i;
        const int sg = WF == B12X_WEIGHT_MXFP4 ? kf >> 2 : kf >> 1;
        const bool v = kf < ke;
        bq[j][i] = buf_load16(b_rsrc, v ? cb + (uint32_t)((j * p.KF + kf) * kFragBytes + lane * 16) : kBufOOB);
        bs[j][i] = buf_load4(bs_rsrc, v ? sb + (uint32_t)((j * p.KFS + sg) * kScaleGroupBytes + lane * 4) : kBufOOB);
      }
    }
  };
  const BufRsrc a_rsrc = make_rsrc(A8 ? (const void*)p.a8 : (const void*)p.a16, p.a_bytes);
  [[maybe_unused]] const BufRsrc h_rsrc = make_rsrc(p.h16, GU ? p.h_bytes : 0);
  const BufRsrc as_rsrc = make_rsrc(p.as, p.as_bytes);

  for (int r0 = 0; r0 < m; r0 += 16) {
    // ---- activation rows: lane (r16, g) owns row r0 + r16, this wave's K range
    const int rr = r0 + r16;
    int64_t src = -1;
    if (rr < m) src = p.a_by_token ? s_rows[rr] / p.k : s_rows[rr];
    uint4 av[KW][A8 ? 2 : 4];
    int sa[KW];
    const int kblocks = (int)(p.K / 32);
#pragma unroll
    for (int i = 0; i < KW; ++i) {
      const int kf = kb + i;
      const int64_t k0 = (int64_t)kf * kFragK;
      const bool rv = kf < ke && src >= 0;
      if constexpr (!A8) {
        const uint32_t o = rv && k0 + 32 * g < p.K ? (uint32_t)((src * p.a_stride + k0 + 32 * g) * 2) : kBufOOB;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if constexpr (FUSE == 2) av[i][s] = buf_load16_dev(a_rsrc, o == kBufOOB ? kBufOOB : o + 16 * s);
          else av[i][s] = buf_load16(a_rsrc, o == kBufOOB ? kBufOOB : o + 16 * s);
        }
        sa[i] = 0;
      } else {
        const uint32_t o = rv ? (uint32_t)(src * p.a_stride + k0) : kBufOOB;
        av[i][0] = buf_load16(a_rsrc, o != kBufOOB && k0 + 16 * g < p.K ? o + 16 * g : kBufOOB);
        av[i][1] = buf_load16(a_rsrc, o != kBufOOB && k0 + 64 + 16 * g < p.K ? o + 64 + 16 * g : kBufOOB);
        // one E8M0 byte per lane; a block past K reads code 0 (2^-127), which
        // multiplies zero codes on both sides
        const bool sv = rv && 4 * kf + g < kblocks;
        sa[i] = buf_load1(as_rsrc, sv ? (uint32_t)(src * p.as_stride + 4 * kf + g) : kBufOOB);
      }
    }

    // one fragment group: MFMAs over this wave's K range, split-K sum, epilogue
    auto group = [&](uint4 (&bq)[FR][KW], uint32_t (&bs)[FR][KW], int grp) {
      f32x4 acc[FR];
#pragma unroll
      for (int j = 0; j < FR; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < KW; ++i) {
        const int kf = kb + i;  // past the wave's K range A and B are zero
        {
          if constexpr (!A8) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const bf16x8 afr = __builtin_bit_cast(bf16x8, av[i][s]);
#pragma unroll
              for (int j = 0; j < FR; ++j) {
                const uint4 q = bq[j][i];
                const uint32_t dw = s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
                float sc;
                if constexpr (WF == B12X_WEIGHT_MXFP4) sc = e8m0_as_scale((bs[j][i] >> (8 * (kf & 3))) & 0xFFu);
                else sc = e4m3_value((bs[j][i] >> (8 * (2 * (kf & 1) + (s >> 1)))) & 0xFFu);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, dequant8_bf16<WF>(dw, sc), acc[j], 0, 0, 0);
              }
            }
          } else {
            const i32x8 afr = {(int)av[i][0].x, (int)av[i][0].y, (int)av[i][0].z, (int)av[i][0].w,
                               (int)av[i][1].x, (int)av[i][1].y, (int)av[i][1].z, (int)av[i][1].w};
#pragma unroll
            for (int j = 0; j < FR; ++j) {
              const uint4 q = bq[j][i];
              const i32x8 bfr = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
              const int sb = (int)((bs[j][i] >> (8 * (kf & 3))) & 0xFFu);
              acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr, acc[j], 0, 4, 0, sa[i], 0, sb);
            }
          }
        }
      }
      if (wave != 0) {
#pragma unroll
        for (int j = 0; j < FR; ++j) s_red(par, wave, j) = acc[j];
      }
      __syncthreads();
      if (wave == 0) {
        f32x4 v[FR];
#pragma unroll
        for (int j = 0; j < FR; ++j) {
          v[j] = acc[j];
#pragma unroll
          for (int w = 1; w < 4; ++w) v[j] += s_red(par, w, j);
        }
        const int f0 = grp * FR;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = r0 + 4 * g + i;
          const bool live = row < m;
          const int64_t pr = live ? s_rows[row] : 0;
          if constexpr (MODE == DMODE_DOWN) {
#pragma unroll
            for (int j = 0; j < FR; ++j)
              if (live && f0 + j < p.NF) p.y[pr * p.y_stride + 16 * (f0 + j) + r16] = v[j][i] * gsc;
          } else {
            constexpr int NH = MODE == DMODE_SILU ? FR / 2 : FR;  // h column blocks of 16
            float hv[NH];
#pragma unroll
            for (int q = 0; q < NH; ++q) {
              if constexpr (MODE == DMODE_SILU) {
                const float gt = v[2 * q][i] * gsc, up = v[2 * q + 1][i] * gsc;
                hv[q] = p.oai ? swiglu_oai(gt, up) : gt / (1.0f + __expf(-gt)) * up;
              } else {
                const float z = v[q][i] * gsc;
                hv[q] = z > 0.f ? z * z : 0.f;
              }
            }
            const int hcol0 = MODE == DMODE_SILU ? 16 * (f0 / 2) : 16 * f0;
            const int nh = MODE == DMODE_SILU ? max(0, min(NH, (p.NF - f0) / 2)) : max(0, min(NH, p.NF - f0));
            if constexpr (NVRT) {
              // h as the bf16 value E2M1 * E4M3 of its NVFP4 round trip
              // (blocks of 16 columns = one column block, the 16 lanes of a
              // row); the down kernel applies the expert's activation scale
              const float gh = p.hglobal[e];
#pragma unroll
              for (int q = 0; q < NH; ++q) {
                if (q < nh) {
                  float mx = fabsf(hv[q]);
                  mx = row16_max(mx);
                  const float sc = nv_block_scale(mx, gh), rc = nv_recip(sc, gh);
                  if (live) p.h16[pr * p.h_stride + hcol0 + 16 * q + r16] = (uint16_t)bf16_rne(nv_roundtrip(hv[q], sc, gh, rc));
                }
              }
            } else if constexpr (RT) {
              // h as the bf16 value of its MXFP8 round trip (blocks of 32
              // columns = column blocks (2b, 2b+1))
              static_assert(NH % 2 == 0, "whole MXFP8 blocks per group");
#pragma unroll
              for (int blk = 0; blk < NH / 2; ++blk) {
                if (2 * blk < nh) {
                  float mx = fmaxf(fabsf(hv[2 * blk]), fabsf(hv[2 * blk + 1]));
                  mx = row16_max(mx);
                  const int sx = mx_scale_exp(f32_bits(mx));
                  const int64_t col = hcol0 + 32 * blk + r16;
                  if (live) {
                    p.h16[pr * p.h_stride + col] = (uint16_t)mx_roundtrip_bf16(hv[2 * blk], sx);
                    p.h16[pr * p.h_stride + col + 16] = (uint16_t)mx_roundtrip_bf16(hv[2 * blk + 1], sx);
                  }
                }
              }
            } else if constexpr (!A8) {
#pragma unroll
              for (int q = 0; q < NH; ++q) {
                if (live && q < nh) {
                  if constexpr (GU)
                    buf_store2_dev(h_rsrc, (uint32_t)((pr * p.h_stride + hcol0 + 16 * q + r16) * 2),
                                   (uint16_t)bf16_rne(hv[q]));
                  else
                    p.h16[pr * p.h_stride + hcol0 + 16 * q + r16] = (uint16_t)bf16_rne(hv[q]);
                }
              }
            } else {
#pragma unroll
              for (int blk = 0; blk < NH / 2; ++blk) {
                if (2 * blk < nh) {
                  float mx = fmaxf(fabsf(hv[2 * blk]), fabsf(hv[2 * blk + 1]));
                  mx = row16_max(mx);
                  const int sx = mx_scale_exp(f32_bits(mx));
                  const int64_t col = hcol0 + 32 * blk + r16;
                  if (live) {
                    p.h8[pr * p.h_stride + col] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[2 * blk]), sx);
                    p.h8[pr * p.h_stride + col + 16] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[2 * blk + 1]), sx);
                    if (r16 == 0) p.hs[pr * p.hs_stride + (hcol0 + 32 * blk) / 32] = (uint8_t)(sx + 127);
                  }
                }
              }
            }
          }
        }
      }
      par ^= 1;  // the next group writes the other buffer; one barrier per group suffices
    };

    // ---- the groups of this part, one at a time: the other waves and
    // workgroups on the compute unit keep the memory system busy meanwhile
    uint4 bq[FR][KW];
    uint32_t bs[FR][KW];
    for (int gi = g_begin; gi < g_end; ++gi) {
      load_b(bq, bs, gi);
      group(bq, bs, gi);
    }
  }
  if constexpr (GU) {
    // wave 0 stored this part's h rows; once they are visible device-wide,
    // raise the groups' flags
    if (wave == 0) {
      wait_vmem();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      uint64_t* f = p.flags + (int64_t)slot * p.flags_per_slot;
      for (int gi = g_begin + lane; gi < g_end; gi += 64)
        __hip_atomic_store(f + gi, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  }
  if (!deal) break;
  chunk_id += (int)gridDim.x;
  lo = chunk_id * deal;
  if (lo >= items) break;
  hi = (int)min(items, (int64_t)lo + deal);
  }
}

template <int WF, int AF, int MODE, int FR, int KW>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecodeParams p) {
  __shared__ DecodeLds L;
  __shared__ f32x4 s_red[2 * 3 * FR * 64];
  if (!p.lv.on()) return;
  const int P = (int)(p.lv.tokens() * p.k);
  const int n_touched = decode_prep(p.ids, P, p.E, L.ids, L.bits, L.wpre);
  decode_items<WF, AF, MODE, FR, KW, 0>(p, L, s_red, n_touched, 0, P, 0, 0, NoFallback{});
}

// Gate/up and down in one launch (16-bit activations): every workgroup takes
// its share of the gate/up items, then its share of the down items; a down
// part waits only for the gate/up groups of its own expert.  The grid is at
// most the resident capacity, and no workgroup waits before its gate/up
// share is done, so every awaited group is being computed by a running
// workgroup as long as the whole grid is resident.  Should a workgroup not
// be (the device shared with other work), a wait for its groups runs out
// after kWaitPolls polls and the waiting workgroup computes them itself:
// slower, with the same result.
//
// The launch's tag: every workgroup reads the launch counter first thing and
// adds its share of kLaunchStep (the shares of a grid sum to kLaunchStep, and
// each is at least 1) as its last action.  So whenever a workgroup of launch
// n starts, some of its own launch's shares are still missing (its own among
// them) and none of the next launch's are there: it reads a value in
// [n, n + 1) * kLaunchStep, whatever the order in which workgroups start and
// end.  The counter must start at a multiple of kLaunchStep (b12x_moe_prime
// zeroes it); the combine checks that it still is one.
template <int WF, int MODE1, int FR1, int KW1, int FR2, int KW2>
__global__ __launch_bounds__(kDecThreads) void decode_fused_kernel(const DecodeParams p1, const DecodeParams p2) {
  constexpr int FRM = FR1 > FR2 ? FR1 : FR2;
  __shared__ DecodeLds L;
  __shared__ f32x4 s_red[2 * 3 * FRM * 64];
  const uint64_t tag = flag_tag(p1.counter);
  if (p1.lv.on()) {  // (a live token count that another path serves: nothing but the counter share)
    const int P = (int)(p1.lv.tokens() * p1.k);
    const int n_touched = decode_prep(p1.ids, P, p1.E, L.ids, L.bits, L.wpre);
    decode_items<WF, B12X_ACT_BF16, MODE1, FR1, KW1, 1>(p1, L, s_red, n_touched, tag, P, 0, 0, NoFallback{});
    // a down part whose wait ran out computes the gate/up groups still missing: each
    // run of consecutive missing groups as one part of the gate/up phase
    auto fallback = [&](int slot, uint64_t miss) {
      const int base = slot * p1.n_groups;
      while (miss) {
        const int g0 = __builtin_ctzll(miss);
        const uint64_t above = miss >> g0;
        const int len = ~above ? __builtin_ctzll(~above) : 64 - g0;
        decode_items<WF, B12X_ACT_BF16, MODE1, FR1, KW1, 3>(p1, L, s_red, n_touched, tag, P, base + g0,
                                                            base + g0 + len, NoFallback{});
        miss = g0 + len >= 64 ? 0ull : miss & (~0ull << (g0 + len));
      }
    };
    decode_items<WF, B12X_ACT_BF16, DMODE_DOWN, FR2, KW2, 2>(p2, L, s_red, n_touched, tag, P, 0, 0, fallback);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t share = kLaunchStep / gridDim.x + (blockIdx.x < kLaunchStep % gridDim.x ? 1 : 0);
    __hip_atomic_fetch_add(p1.counter, share, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One workgroup per resident slot, never more than the items of the largest
// possible touched set (min(T*k, E) experts).
template <int WF, int AF, int MODE, int FR, int KW>
static int launch_decode_kw(const BindingImpl& b, const DecodeParams& p, hipStream_t s) {
  static int cache[64];
  auto kernel = decode_kernel<WF, AF, MODE, FR, KW>;
  const int64_t max_slots = b.T * b.k < b.E ? b.T * b.k : b.E;
  int64_t grid = resident_workgroups(kernel, cache);
  if (grid > max_slots * p.n_groups) grid = max_slots * p.n_groups;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecThreads), 0, s, p);
  return (int)hipGetLastError();
}

// K fragments per wave: the smallest of 2, 4, 8 that covers ceil(KF / 4).
template <int WF, int AF, int MODE, int FR>
static int launch_decode_t(const BindingImpl& b, DecodeParams& p, hipStream_t s) {
  p.n_groups = (p.NF + FR - 1) / FR;
  const int kper = (p.KF + 3) / 4;
  if (kper <= 2) return launch_decode_kw<WF, AF, MODE, FR, 2>(b, p, s);
  if (kper <= 4) return launch_decode_kw<WF, AF, MODE, FR, 4>(b, p, s);
  return launch_decode_kw<WF, AF, MODE, FR, 8>(b, p, s);
}

template <int MODE, int FR>
static int launch_decode_fmt(const BindingImpl& b, DecodeParams& p, hipStream_t s) {
  if (a8_native(b.wfmt, b.afmt)) return launch_decode_t<B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, MODE, FR>(b, p, s);
  if (b.wfmt == B12X_WEIGHT_NVFP4) return launch_decode_t<B12X_WEIGHT_NVFP4, B12X_ACT_BF16, MODE, FR>(b, p, s);
  return launch_decode_t<B12X_WEIGHT_MXFP4, B12X_ACT_BF16, MODE, FR>(b, p, s);
}

static DecodeParams common_params(const BindingImpl& b) {
  DecodeParams p = {};
  p.ids = b.ids;
  p.tw = b.tw;
  p.T = (int)b.T;
  p.lv = b.live();
  p.k = b.k;
  p.E = b.E;
  p.P = (int)(b.T * b.k);
  return p;
}

static DecodeParams gate_up_params(const BindingImpl& b) {
  DecodeParams p = common_params(b);
  p.oai = b.oai;
  const bool a8 = a8_native(b.wfmt, b.afmt);
  p.a16 = b.a;
  p.a8 = b.xq;
  p.as = b.xs;
  p.a_stride = a8 ? b.Hp : b.a_stride;
  p.as_stride = b.Hp / 32;
  p.a_bytes = a8 ? b.T * b.Hp : b.T * b.a_stride * 2;
  p.as_bytes = a8 ? b.T * (b.Hp / 32) : 0;
  if (a8_bf16(b.wfmt, b.afmt) || a4_nv(b.afmt)) {  // NVFP4 weights: the bf16 copy of a's MXFP8 / NVFP4 round trips
    p.a16 = (const uint16_t*)b.xq;
    p.a_stride = b.Hp;
    p.a_bytes = b.T * b.Hp * 2;
  }
  if (a4_nv(b.afmt)) {
    p.aglobal = b.a13_global;  // x's activation scale, one value
    p.aglobal_per_expert = 0;
    p.hglobal = b.a2_global;   // h is requantized against its expert's scale
  }
  p.a_by_token = 1;
  p.K = b.H;
  p.KF = (int)b.kf13;
  p.bcodes = b.w13_codes;
  p.bscales = b.w13_scales;
  p.bglobal = b.w13_global;
  p.b_codes_expert = b.nf13 * b.kf13 * kFragBytes;
  p.b_scales_expert = b.nf13 * b.kfs13 * kScaleGroupBytes;
  p.NF = (int)b.nf13;
  p.KFS = (int)b.kfs13;
  p.h16 = (uint16_t*)b.h;
  p.h8 = (uint8_t*)b.h;
  p.hs = b.hs;
  p.h_stride = b.Ip;
  p.hs_stride = b.Ip / 32;
  p.h_bytes = b.T * b.k * b.Ip * 2;
  return p;
}

static DecodeParams down_params(const BindingImpl& b) {
  DecodeParams p = common_params(b);
  p.a16 = (const uint16_t*)b.h;
  p.a8 = (const uint8_t*)b.h;
  p.as = b.hs;
  p.a_stride = b.Ip;
  p.as_stride = b.Ip / 32;
  const bool a8 = a8_native(b.wfmt, b.afmt);  // else h is bf16
  p.a_bytes = b.T * b.k * b.Ip * (a8 ? 1 : 2);
  p.as_bytes = a8 ? b.T * b.k * (b.Ip / 32) : 0;
  p.a_by_token = 0;
  p.K = b.I;
  p.KF = (int)b.kf2;
  p.bcodes = b.w2_codes;
  p.bscales = b.w2_scales;
  p.bglobal = b.w2_global;
  p.b_codes_expert = b.nf2 * b.kf2 * kFragBytes;
  p.b_scales_expert = b.nf2 * b.kfs2 * kScaleGroupBytes;
  p.NF = (int)b.nf2;
  p.KFS = (int)b.kfs2;
  p.y = b.y;
  p.y_stride = b.H;
  if (a4_nv(b.afmt)) {  // h's activation scale, one per expert
    p.aglobal = b.a2_global;
    p.aglobal_per_expert = 1;
  }
  return p;
}

bool decode_fused(const BindingImpl& b) {
  // one wave polls the flags of an expert: at most 64 gate/up groups
  return b.path == 2 && b.afmt == B12X_ACT_BF16 && b.dsync && (b.kf13 + 3) / 4 <= 4 && (b.kf2 + 3) / 4 <= 4 &&
         (b.nf13 + 1) / 2 <= 64;
}

// Gate/up groups of FR1 = 2 fragments, down groups of FR2 = 4 (as the
// separate launches use them at these K), grid as for one launch of the
// larger item count.
template <int WF, int MODE1, int KW1, int KW2>
static int launch_fused_kw(const BindingImpl& b, DecodeParams& p1, DecodeParams& p2, hipStream_t s) {
  static int cache[64];
  auto kernel = decode_fused_kernel<WF, MODE1, 2, KW1, 4, KW2>;
  p1.n_groups = (p1.NF + 1) / 2;
  p2.n_groups = (p2.NF + 3) / 4;
  p2.prev_groups = p1.n_groups;
  const int64_t max_slots = b.T * b.k < b.E ? b.T * b.k : b.E;
  const int64_t items = max_slots * (p1.n_groups > p2.n_groups ? p1.n_groups : p2.n_groups);
  int64_t grid = resident_workgroups(kernel, cache);
  if (grid > items) grid = items;
  if (grid < 1) grid = 1;
  if (grid > (int64_t)kLaunchStep) grid = (int64_t)kLaunchStep;  // every share of the launch counter >= 1
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kDecThreads), 0, s, p1, p2);
  return (int)hipGetLastError();
}

template <int WF, int MODE1>
static int launch_fused_t(const BindingImpl& b, DecodeParams& p1, DecodeParams& p2, hipStream_t s) {
  const bool k1 = (p1.KF + 3) / 4 <= 2, k2 = (p2.KF + 3) / 4 <= 2;
  if (k1 && k2) return launch_fused_kw<WF, MODE1, 2, 2>(b, p1, p2, s);
  if (k1) return launch_fused_kw<WF, MODE1, 2, 4>(b, p1, p2, s);
  if (k2) return launch_fused_kw<WF, MODE1, 4, 2>(b, p1, p2, s);
  return launch_fused_kw<WF, MODE1, 4, 4>(b, p1, p2, s);
}

static int launch_fused(const BindingImpl& b, hipStream_t s) {
  DecodeParams p1 = gate_up_params(b), p2 = down_params(b);
  uint8_t* sync = b.dsync;
  for (DecodeParams* p : {&p1, &p2}) {
    p->counter = (uint64_t*)(sync + kDecodeCounterOffset);
    p->flags = (uint64_t*)(sync + kDecodeFlagsOffset);
    p->flags_per_slot = (int)((b.nf13 + 1) / 2);
    p->deal = 2;
    // test hook: waits that cannot succeed and run out after a few polls, so that every
    // down part computes its expert's gate/up groups itself
    p->expect_xor = b.force_giveup ? 0x80000000ull : 0ull;
    p->max_polls = b.force_giveup ? 4 : kWaitPolls;
  }
  const bool nv = b.wfmt == B12X_WEIGHT_NVFP4;
  if (b.gated)
    return nv ? launch_fused_t<B12X_WEIGHT_NVFP4, DMODE_SILU>(b, p1, p2, s)
              : launch_fused_t<B12X_WEIGHT_MXFP4, DMODE_SILU>(b, p1, p2, s);
  return nv ? launch_fused_t<B12X_WEIGHT_NVFP4, DMODE_RELU2>(b, p1, p2, s)
            : launch_fused_t<B12X_WEIGHT_MXFP4, DMODE_RELU2>(b, p1, p2, s);
}

// The decode synchronization region zeroed by a fill kernel (not a memset
// node, so that a captured graph may hold it): counter 0, flags 0
// (no flag then holds a launch's tag, which is never 0).
__global__ __launch_bounds__(256) void zero_words_kernel(uint64_t* __restrict__ w, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0;
}

int launch_decode_prime(uint8_t* dsync, uint64_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 8);
  if (!dsync || n == 0) return 0;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (uint64_t*)dsync, n);
  return (int)hipGetLastError();
}

int launch_decode1(const BindingImpl& b, hipStream_t s) {
  if (decode_fused(b)) return launch_fused(b, s);
  DecodeParams p = gate_up_params(b);
  if (b.gated && a8_native(b.wfmt, b.afmt))  // an MXFP8 block of h (32 columns) = two gate/up pairs
    return launch_decode_t<B12X_WEIGHT_MXFP4, B12X_ACT_MXFP8, DMODE_SILU, 4>(b, p, s);
  if (a8_bf16(b.wfmt, b.afmt))
    return b.gated ? launch_decode_t<B12X_WEIGHT_NVFP4, kActRt, DMODE_SILU, 4>(b, p, s)
                   : launch_decode_t<B12X_WEIGHT_NVFP4, kActRt, DMODE_RELU2, 2>(b, p, s);
  if (a4_nv(b.afmt))  // an NVFP4 block of h (16 columns) = one gate/up pair
    return b.gated ? launch_decode_t<B12X_WEIGHT_NVFP4, kActNvRt, DMODE_SILU, 2>(b, p, s)
                   : launch_decode_t<B12X_WEIGHT_NVFP4, kActNvRt, DMODE_RELU2, 2>(b, p, s);
  if (b.gated) return launch_decode_fmt<DMODE_SILU, 2>(b, p, s);
  return launch_decode_fmt<DMODE_RELU2, 2>(b, p, s);
}

int launch_decode2(const BindingImpl& b, hipStream_t s) {
  DecodeParams p = down_params(b);
  // 4 fragments (64 output columns) per group unless 8 K fragments per wave need the registers
  if ((p.KF + 3) / 4 > 4) return launch_decode_fmt<DMODE_DOWN, 2>(b, p, s);
  return launch_decode_fmt<DMODE_DOWN, 4>(b, p, s);
}

}  // namespace b12x
