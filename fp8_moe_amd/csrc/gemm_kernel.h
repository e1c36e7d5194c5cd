// Grouped expert GEMMs of the fused MoE on gfx950 MFMA (b12x README "What's in
// here": the unified dynamic path runs routed experts on a persistent grid;
// W4A16 dequantizes the FP4 weights inline with no activation-scale math;
// w4a8_mx multiplies FP4 weights with dynamically quantized MXFP8
// activations).  One kernel template serves
//   GEMM1: h[row] = act(x[token(row)] . W13_e^T)   (SiLU-gated or ReLU^2)
//   GEMM2: y[row] = h[row] . W2_e^T                (stored as bf16)
// over the routing tiles (expert, first row, rows).  A workgroup of 4 waves
// owns one routing tile (up to kTileRows = 128 rows) x 4*NFW weight fragments
// (16 columns each), and two workgroups share a CU: one wave per SIMD cannot
// keep the matrix core busy with 16x16x32 MFMAs (a register-only loop of them
// reaches ~53% of the datasheet rate at one wave per SIMD, ~82% at two), so
// each wave holds at most 256 registers and each workgroup at most half of
// the LDS, and the other workgroup's MFMAs run while one waits at its step
// barrier.  Every wave covers all rows of the tile, so each dequantized
// weight feeds 128 rows of MFMAs.  The packed FP4 fragments stream from
// global memory straight into registers.  The activation rows reach LDS by
// DMA (buffer_load ... lds) for 16-bit activations, in two stages loaded one
// K step ahead, or through registers into two LDS buffers for MXFP8
// activations.  All loads are raw buffer loads whose out-of-range
// offsets read zeros, so none of them sits behind a branch.
//   W4A16: each 1 KB fragment is four 16x16x32 MFMA operands; FP4 is turned
//          into bf16 in registers (v_cvt_scalef32_pk_bf16_fp4 with the E8M0
//          scale, or fp32 conversion times the E4M3 scale for NVFP4; both
//          products are exact in bf16), or into f16 for NVFP4 weights with
//          the scaled f16 copy of the activations (see dequant8_f16_nv).
//   W4A8:  each fragment is one 16x16x128 scaled MFMA operand (fp8 A x fp4 B,
//          one E8M0 scale per lane on each side).
// The NVFP4 per-expert fp32 scale multiplies the fp32 accumulators.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace b12x {

constexpr int kGemmThreads = 256;

struct GemmParams {
  const int32_t* tiles;
  const int32_t* ntiles;
  int n_ntiles;
  int max_tiles;  // bounds that make a stale tile list harmless
  int max_rows;
  int E;
  // A operand: bf16 rows (a16) or MXFP8 codes + scales (a8, as); GEMM1 maps
  // a row to its token through sorted / k_top, GEMM2 reads rows directly.
  const uint16_t* a16;
  const uint8_t* a8;
  const uint8_t* as;
  int64_t a_stride;   // elements (bf16) or bytes (codes)
  int64_t as_stride;  // bytes
  int64_t a_bytes, as_bytes;  // extents of a16 / a8 and as (at most 1 GiB)
  const int32_t* a_exp;       // f16 activations: power-of-two exponent of each token row
  const int32_t* sorted;
  int k_top;
  int64_t n_pairs;
  int64_t K;
  int KF;
  // B operand (prepared weights)
  const uint8_t* bcodes;
  const uint8_t* bscales;
  const float* bglobal;
  // NVFP4 activations: activation scale multiplied into the accumulator with
  // bglobal (x: one value, aglobal_per_expert = 0; h: one per expert), and the
  // scale of each expert's h for the gate/up epilogue's requantization
  const float* aglobal;
  int aglobal_per_expert;
  const float* hglobal;
  int oai;  // gated: SwiGLU-OAI instead of SiLU
  int64_t b_codes_expert;
  int64_t b_scales_expert;
  int NF;
  int KFS;
  // outputs
  uint16_t* h16;
  uint8_t* h8;
  uint8_t* hs;
  int64_t h_stride;
  int64_t hs_stride;
  // bf16 output rows: y (MODE_DOWN, one row per routed row, pads included)
  // or the dense GEMM's out (MODE_DENSE: dense_m rows of a, tiles of
  // kTileRows rows in order, no tile list, one weight matrix)
  uint16_t* out16;
  int64_t out_stride;
  int64_t dense_m;
  LiveT lv;  // live token count: the whole grid returns unless the grouped path serves it
};

enum { MODE_SILU = 1, MODE_RELU2 = 2, MODE_DOWN = 3, MODE_DENSE = 4 };

// Work items are (tile, N tile); the items are split into 8 contiguous ranges,
// one per XCD (workgroup i runs on XCD i % 8), so that the workgroups sharing
// an L2 work on the same row tiles (A reuse) and the same experts (B reuse).
//
// Wave w owns all rows of the tile and weight fragments [NFW w, NFW w +
// NFW): every fragment is dequantized by exactly one wave.  A full tile
// (kTileRows rows) runs a branch-free MFMA loop; a partial tile skips whole
// 16-row blocks.  Missing fragments (a partial N tile) load zeros and are dropped
// in the epilogue.
template <int WF, int AF, int MODE, int NFW>
__global__ __launch_bounds__(kGemmThreads, 2) void moe_gemm_kernel(const GemmParams p) {
  constexpr bool A8 = AF == B12X_ACT_MXFP8;
  // f16 activations x NVFP4 weights dequantized to f16
  constexpr bool F16 = AF == kActF16 || AF == kActF16Rt || AF == kActF16NvRt;
  // MXFP8 round trips as activations (NVFP4 x MXFP8): h stored as its own round trip
  constexpr bool RT = AF == kActRt || AF == kActF16Rt;
  // NVFP4 round trips as activations (W4A4): h stored as its own NVFP4 round trip
  constexpr bool NVRT = AF == kActNvRt || AF == kActF16NvRt;
  static_assert(!F16 || WF == B12X_WEIGHT_NVFP4, "f16 activations run with NVFP4 weights");
  using OpT = std::conditional_t<F16, f16x8, bf16x8>;  // 16-bit MFMA operand type
  constexpr int ROWB = A8 ? 144 : 272;  // LDS bytes per A row: 128 K elements + 16 bytes of skew
  constexpr int NT = 4 * NFW;           // weight fragments per workgroup tile
  constexpr int LOADS = (kTileRows * (A8 ? 8 : 16) + kGemmThreads - 1) / kGemmThreads;  // A row chunks per thread
  constexpr int CHUNKS = A8 ? 8 : 16;   // 16-byte chunks per 128-element row
  constexpr int MF = kTileRows / 16;    // 16-row blocks per tile
  static_assert(kTileRows % 16 == 0 && kTileRows <= kGemmThreads, "tile rows");
  // W4A8: activations through registers into two LDS buffers of ROWB-byte rows
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][A8 ? kTileRows * ROWB : 16];
  __shared__ uint32_t lds_s[2][A8 ? kTileRows : 1];
  // W4A16 (bf16 or f16 activations): kStages LDS stages of 256-byte rows filled by DMA; each
  // stage is its own array so that the compiler tracks the DMA of each stage separately
  constexpr int kStageBytes = A8 ? 16 : kTileRows * 256;
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds_st1[kStageBytes];
  __shared__ float lds_rs[F16 ? kTileRows : 1];  // f16: 2^exponent of each tile row

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int c = tid % CHUNKS;

  if (!p.lv.on()) return;
  const int n_row_tiles =
      MODE == MODE_DENSE ? (int)((p.dense_m + kTileRows - 1) / kTileRows) : min(max(p.ntiles[0], 0), p.max_tiles);
  const int n_items = n_row_tiles * p.n_ntiles;
  const int xcd = blockIdx.x & 7, n_local = gridDim.x >> 3;
  const int lo = (int)((int64_t)n_items * xcd / 8), hi = (int)((int64_t)n_items * (xcd + 1) / 8);

  for (int w = lo + (int)(blockIdx.x >> 3); w < hi; w += n_local) {
    const int tile = w / p.n_ntiles;
    const int nt = w - tile * p.n_ntiles;
    int e, row0, nrows;
    if constexpr (MODE == MODE_DENSE) {
      e = 0;
      row0 = tile * kTileRows;
      nrows = (int)min((int64_t)kTileRows, p.dense_m - row0);
    } else {
      e = p.tiles[4 * tile];
      row0 = p.tiles[4 * tile + 1];
      nrows = p.tiles[4 * tile + 2];
    }
    if (e < 0 || e >= p.E || row0 < 0 || nrows <= 0 || nrows > kTileRows || row0 + nrows > p.max_rows) continue;
    const int nmf = (nrows + 15) / 16;
    const int f0 = nt * NT + wave * NFW;
    const int nnf = max(0, min(NFW, p.NF - f0));
    const uint8_t* bcodes = p.bcodes + (int64_t)e * p.b_codes_expert;
    const uint8_t* bscales = p.bscales + (int64_t)e * p.b_scales_expert;
    float gsc = p.bglobal ? p.bglobal[e] : 1.0f;
    if (p.aglobal) gsc *= p.aglobal[p.aglobal_per_expert ? e : 0];

    // ---- buffer resources: every load below is unconditional; a row, K chunk
    // or fragment outside the problem gets an out-of-range offset (zeros)
    constexpr int ESZ = A8 ? 1 : 2;  // bytes per A element
    const BufRsrc a_rsrc = make_rsrc(A8 ? (const void*)p.a8 : (const void*)p.a16, p.a_bytes);
    const BufRsrc s_rsrc = make_rsrc(p.as, p.as_bytes);
    const BufRsrc b_rsrc = make_rsrc(bcodes, p.b_codes_expert);
    const BufRsrc bs_rsrc = make_rsrc(bscales, p.b_scales_expert);

    // Per-lane offsets are fixed for the work item; the K step adds a scalar
    // offset.  Steps past the last K fragment (the prefetch at the end of the
    // loop) reload the last fragment, whose data is never used, so every
    // address stays inside its row.
    // byte offset of this thread's 16-byte chunk c of each of its A rows
    // (token row for GEMM1, h row for GEMM2); rows outside the tile read zeros
    uint32_t a_voff[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int rr = tid / CHUNKS + (kGemmThreads / CHUNKS) * i;
      int sr = -1;
      if (rr < nrows && rr < kTileRows) {
        if (p.sorted) {
          const int pair = p.sorted[row0 + rr];
          sr = (pair >= 0 && pair < p.n_pairs) ? pair / p.k_top : -1;
        } else {
          sr = row0 + rr;
        }
      }
      a_voff[i] = sr >= 0 ? (uint32_t)(sr * p.a_stride * ESZ + 16 * c) : kBufOOB;
    }
    uint32_t s_voff = kBufOOB;  // A8: scale row of threads 0..kTileRows-1
    if (A8 && tid < kTileRows && tid < nrows) {
      int sr = -1;
      if (p.sorted) {
        const int pair = p.sorted[row0 + tid];
        sr = (pair >= 0 && pair < p.n_pairs) ? pair / p.k_top : -1;
      } else {
        sr = row0 + tid;
      }
      if (sr >= 0) s_voff = (uint32_t)(sr * p.as_stride);
    }
    const int kblocks = (int)(p.K / 32);
    // K not a multiple of 128: in the last fragment a chunk past K reads zeros
    const int k_last = (int)(p.K - (int64_t)(p.KF - 1) * kFragK);  // elements in the last fragment
    const bool ragged = k_last < kFragK;
    const bool chunk_in_last = (A8 ? 16 : 8) * c < k_last;

    // A chunks of K fragment kf; A8: the 4 block scales of the row, with the
    // byte mask of real blocks
    auto load_a = [&](uint4 (&ra)[LOADS], uint32_t& rs, uint32_t& rk, int kf) {
      const int kfc = min(kf, p.KF - 1);
      const uint32_t soff = (uint32_t)(kfc * kFragK * ESZ);
      if (ragged && kfc == p.KF - 1) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) ra[i] = buf_load16s(a_rsrc, chunk_in_last ? a_voff[i] : kBufOOB, soff);
      } else {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) ra[i] = buf_load16s(a_rsrc, a_voff[i], soff);
      }
      if constexpr (A8) {
        const int nb = min(max(kblocks - 4 * kfc, 0), 4);
        rs = buf_load4s(s_rsrc, s_voff, (uint32_t)(4 * kfc));
        rk = nb >= 4 ? 0xFFFFFFFFu : (1u << (8 * nb)) - 1u;
      }
    };
    auto store_a = [&](const uint4 (&ra)[LOADS], uint32_t rs, uint32_t rk, int buf) {
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        const int rr = tid / CHUNKS + (kGemmThreads / CHUNKS) * i;
        if ((kTileRows * CHUNKS) % kGemmThreads == 0 || rr < kTileRows)
          *(uint4*)(&lds_a[buf][rr * ROWB + 16 * c]) = ra[i];
      }
      if constexpr (A8) {
        // blocks past K get the neutral scale 2^0 (their codes are zero)
        if (tid < kTileRows) lds_s[buf][tid] = (rs & rk) | (0x7F7F7F7Fu & ~rk);
      }
    };
    // weight fragments f0 + j: the lane's offset in a fragment, and the fragment and
    // K step as a scalar offset.  Fragments past the matrix (a partial N tile) reload
    // the last one; their results are dropped in the epilogue.
    const uint32_t b_voff = (uint32_t)(lane * 16), bs_voff = (uint32_t)(lane * 4);
    auto load_b = [&](uint4 (&q)[NFW], uint32_t (&sc)[NFW], int kf) {
      const int kfc = min(kf, p.KF - 1);
      const int sgrp = WF == B12X_WEIGHT_MXFP4 ? kfc >> 2 : kfc >> 1;
      // scales first: a step needs them before its codes
#pragma unroll
      for (int j = 0; j < NFW; ++j) {
        const int f = min(f0 + j, p.NF - 1);
        sc[j] = buf_load4s(bs_rsrc, bs_voff, (uint32_t)((f * p.KFS + sgrp) * kScaleGroupBytes));
      }
#pragma unroll
      for (int j = 0; j < NFW; ++j) {
        const int f = min(f0 + j, p.NF - 1);
        q[j] = buf_load16s(b_rsrc, b_voff, (uint32_t)((f * p.KF + kfc) * kFragBytes));
      }
    };

    f32x4 acc[MF][NFW];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NFW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMAs of one K fragment over the first NMF 16-row blocks.  W4A16: per
    // sub-step the weights are dequantized in registers, then every 16-row
    // block's activations are read from LDS; with two waves per SIMD the
    // other wave's MFMAs run under this wave's VALU and LDS work.
    auto compute = [&](auto nmf_tag, auto par_tag, const uint8_t* la, const uint4 (&bq)[NFW],
                       const uint32_t (&bs)[NFW], int kf) {
      constexpr int NMF = decltype(nmf_tag)::value;
      constexpr int par = decltype(par_tag)::value;  // parity of kf (selects the NVFP4 scale word)
      if constexpr (!A8) {
        float scl[NFW][2];       // per fragment: scale of the lane's first / second 16 K (NVFP4), or the E8M0 scale
        NvScaleF16 scf[NFW][2];  // the same split for the f16 dequantization
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          if constexpr (WF == B12X_WEIGHT_MXFP4) {
            scl[j][0] = scl[j][1] = e8m0_as_scale((bs[j] >> (8 * (kf & 3))) & 0xFFu);
          } else {  // the two E4M3 scales of this K fragment, decoded by the hardware (OCP E4M3)
            const f32x2 sv = __builtin_amdgcn_cvt_pk_f32_fp8((int)bs[j], par == 1);
            if constexpr (F16) {
              scf[j][0] = nv_scale_f16(sv.x);
              scf[j][1] = nv_scale_f16(sv.y);
            } else {
              scl[j][0] = sv.x;
              scl[j][1] = sv.y;
            }
          }
        }
        auto dq = [&](OpT (&out)[NFW], int s) {
#pragma unroll
          for (int j = 0; j < NFW; ++j) {
            const uint32_t dw = s == 0 ? bq[j].x : s == 1 ? bq[j].y : s == 2 ? bq[j].z : bq[j].w;
            if constexpr (F16) out[j] = dequant8_f16_nv(dw, scf[j][s >> 1]);
            else out[j] = dequant8_bf16<WF>(dw, scl[j][s >> 1]);
          }
        };
        // sub-step s: the 4 fragments' operands, then each 16-row block's LDS read and
        // its NFW MFMAs
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          OpT b[NFW];
          dq(b, s);
#pragma unroll
          for (int mf = 0; mf < NMF; ++mf) {
            const OpT afr = __builtin_bit_cast(OpT, *(const uint4*)(la + (16 * mf + r16) * 256 + 16 * ((4 * g + s) ^ r16)));
#pragma unroll
            for (int j = 0; j < NFW; ++j) {
              if constexpr (F16) acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, b[j], acc[mf][j], 0, 0, 0);
              else acc[mf][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, b[j], acc[mf][j], 0, 0, 0);
            }
          }
        }
      } else {
        i32x8 bfr[NFW];
        int sb[NFW];
#pragma unroll
        for (int j = 0; j < NFW; ++j) {
          bfr[j] = i32x8{(int)bq[j].x, (int)bq[j].y, (int)bq[j].z, (int)bq[j].w, 0, 0, 0, 0};
          sb[j] = (int)((bs[j] >> (8 * (kf & 3))) & 0xFFu);
        }
#pragma unroll
        for (int mf = 0; mf < NMF; ++mf) {
          const int row = 16 * mf + r16;
          const uint4 x0 = *(const uint4*)(la + row * ROWB + 16 * g);
          const uint4 x1 = *(const uint4*)(la + row * ROWB + 64 + 16 * g);
          const i32x8 afr = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          const int sa = (int)((lds_s[par][row] >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int j = 0; j < NFW; ++j)
            acc[mf][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(afr, bfr[j], acc[mf][j], 0, 4, 0, sa, 0,
                                                                           sb[j]);
        }
      }
    };

    // ---- main loop.  A: global loads of step kf+2 are issued at step kf into
    // the register stage of that parity and written to LDS at the end of step
    // kf+1; B: loads of step kf+2 are issued after step kf's MFMAs.  No load
    // is conditional (steps past the end load zeros), so each wait covers only
    // the loads its step consumes.  The whole loop is instantiated per count
    // of 16-row blocks (9, or rounded up to even).
    const bool idle = nnf == 0;  // this wave has no fragments in a partial N tile
    auto kloop = [&](auto nmf_tag) {
      uint4 ra0[LOADS], ra1[LOADS];
      uint32_t rs0 = 0, rs1 = 0, rk0 = 0, rk1 = 0;
      uint4 bq0[NFW], bq1[NFW];
      uint32_t bs0[NFW], bs1[NFW];
      __syncthreads();  // the previous work item is done with LDS
      load_a(ra0, rs0, rk0, 0);
      store_a(ra0, rs0, rk0, 0);
      load_a(ra1, rs1, rk1, 1);
      load_b(bq0, bs0, 0);
      load_b(bq1, bs1, 1);
      for (int kf = 0; kf < p.KF; kf += 2) {
        // even step: LDS buffer 0, ra1 holds step kf+1
        __syncthreads();
        load_a(ra0, rs0, rk0, kf + 2);
        if (!idle) compute(nmf_tag, std::integral_constant<int, 0>{}, lds_a[0], bq0, bs0, kf);
        store_a(ra1, rs1, rk1, 1);
        load_b(bq0, bs0, kf + 2);
        if (kf + 1 >= p.KF) break;
        // odd step: LDS buffer 1, ra0 holds step kf+2
        __syncthreads();
        load_a(ra1, rs1, rk1, kf + 3);
        if (!idle) compute(nmf_tag, std::integral_constant<int, 1>{}, lds_a[1], bq1, bs1, kf + 1);
        store_a(ra0, rs0, rk0, 0);
        load_b(bq1, bs1, kf + 3);
      }
    };

    // ---- W4A16 main loop: activations global -> LDS by DMA (buffer_load ... lds) into
    // two stages, weights into two register stages, both loaded one K step ahead.  DMA
    // instruction j of wave w fills rows kRowsPerWave w + 4 j + lane/16 of a stage;
    // position lane%16 of a row holds its 16-byte chunk (lane%16) ^ (row & 15), so the
    // MFMA operand reads of 16 rows hit 16 different bank groups.  Step kf waits for
    // its loads (issued during step kf - 1), then a barrier makes every wave's DMA of
    // the stage visible and frees the other stage (read at step kf - 1), which the
    // loads of step kf + 1 then refill while step kf computes.  Steps past the end
    // reload the last fragment and are not computed.
    constexpr int kStages = 2;
    constexpr int kRowsPerWave = kTileRows / 4;
    constexpr int kDma = kRowsPerWave / 4;  // 1 KB DMA instructions per wave per step
    static_assert(kRowsPerWave % 4 == 0, "DMA rows");
    auto stage_lds = [&](auto st_tag) -> uint8_t* {
      constexpr int ST = decltype(st_tag)::value;
      if constexpr (ST == 0) return lds_st0;
      else return lds_st1;
    };
    auto fill_row_scales = [&]() {  // f16: 2^exponent of each row's token (read by the epilogue)
      if constexpr (F16) {
        if (tid < kTileRows) {
          int ex = 0;
          if (tid < nrows) {
            const int pair = p.sorted[row0 + tid];
            if (pair >= 0 && pair < p.n_pairs) ex = p.a_exp[pair / p.k_top];
          }
          lds_rs[tid] = bits_f32((uint32_t)(127 + ex) << 23);
        }
      }
    };
    auto kloop_dma = [&](auto nmf_tag) {
      // per-lane DMA source offsets (row and swizzled chunk); zeros past the tile; in a
      // ragged last K fragment, zeros past K as well
      uint32_t dvoff[kDma];
      uint32_t in_last = 0;  // bit j: the chunk of DMA j lies inside K in the last fragment
#pragma unroll
      for (int j = 0; j < kDma; ++j) {
        const int rr = kRowsPerWave * wave + 4 * j + (lane >> 4);
        const int chunk = (lane & 15) ^ (rr & 15);
        int sr = -1;
        if (rr < nrows) {
          if (p.sorted) {
            const int pair = p.sorted[row0 + rr];
            sr = (pair >= 0 && pair < p.n_pairs) ? pair / p.k_top : -1;
          } else {
            sr = row0 + rr;
          }
        }
        dvoff[j] = sr >= 0 ? (uint32_t)(sr * p.a_stride * 2 + 16 * chunk) : kBufOOB;
        if (8 * chunk < k_last) in_last |= 1u << j;
      }
      auto dma_a = [&](auto st_tag, int kf) {
        const int kfc = min(kf, p.KF - 1);
        const uint32_t soff = (uint32_t)(kfc * kFragK * 2);
        uint8_t* base = stage_lds(st_tag) + kRowsPerWave * wave * 256;
        if (ragged && kfc == p.KF - 1) {
#pragma unroll
          for (int j = 0; j < kDma; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void*)(base + 1024 * j),
                                                     16, ((in_last >> j) & 1u) ? dvoff[j] : kBufOOB, soff, 0, 0);
        } else {
#pragma unroll
          for (int j = 0; j < kDma; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (__attribute__((address_space(3))) void*)(base + 1024 * j),
                                                     16, dvoff[j], soff, 0, 0);
        }
      };
      uint4 bq[2][NFW];
      uint32_t bs[2][NFW];
      // step kf: stage ST = kf % 2 (LDS and registers; also the parity of kf)
      auto step = [&](auto st_tag, int kf) {
        constexpr int ST = decltype(st_tag)::value;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's loads
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma_a(std::integral_constant<int, ST ^ 1>{}, kf + 1);
        load_b(bq[ST ^ 1], bs[ST ^ 1], kf + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (kf < p.KF && !idle)
          compute(nmf_tag, std::integral_constant<int, ST>{}, stage_lds(st_tag), bq[ST], bs[ST], kf);
      };
      __syncthreads();  // the previous work item is done with LDS
      fill_row_scales();
      dma_a(std::integral_constant<int, 0>{}, 0);
      load_b(bq[0], bs[0], 0);
      for (int kf = 0; kf < p.KF; kf += 2) {
        step(std::integral_constant<int, 0>{}, kf);
        if (kf + 1 >= p.KF) break;
        step(std::integral_constant<int, 1>{}, kf + 1);
      }
    };
    static_assert(MF == 8, "the loops are instantiated for 8, 6, 4 and 2 row blocks");
    if constexpr (A8) {
      if (nmf > 6) kloop(std::integral_constant<int, 8>{});
      else if (nmf > 4) kloop(std::integral_constant<int, 6>{});
      else if (nmf > 2) kloop(std::integral_constant<int, 4>{});
      else kloop(std::integral_constant<int, 2>{});
    } else {
      static_assert(kStages == 2, "the loop body is written for two stages");
      if (nmf > 6) kloop_dma(std::integral_constant<int, 8>{});
      else if (nmf > 4) kloop_dma(std::integral_constant<int, 6>{});
      else if (nmf > 2) kloop_dma(std::integral_constant<int, 4>{});
      else kloop_dma(std::integral_constant<int, 2>{});
    }

    // ---- epilogue: lane holds column r16 of each fragment, rows 4 g + i of each 16-row block
    if constexpr (MODE == MODE_DENSE || MODE == MODE_DOWN) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (mf < nmf) {
#pragma unroll
          for (int j = 0; j < NFW; ++j) {
            if (j < nnf) {
              const int col = 16 * (f0 + j) + r16;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int64_t row = row0 + 16 * mf + 4 * g + i;
                // a routed tile writes all its rows (pads land in their own rows, never read)
                if (MODE == MODE_DOWN || 16 * mf + 4 * g + i < nrows)
                  p.out16[row * p.out_stride + col] = (uint16_t)bf16_rne(acc[mf][j][i] * gsc);
              }
            }
          }
        }
      }
    } else {
      // activation values: gated -> NFW/2 column blocks (gate/up pairs); relu2 -> NFW blocks
      constexpr int NH = MODE == MODE_SILU ? NFW / 2 : NFW;
      const int nh = MODE == MODE_SILU ? nnf / 2 : nnf;
      const int hcol0 = MODE == MODE_SILU ? 16 * (f0 / 2) : 16 * f0;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (mf < nmf) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int64_t row = row0 + 16 * mf + 4 * g + i;
            const float rsc = F16 ? gsc * lds_rs[F16 ? 16 * mf + 4 * g + i : 0] : gsc;  // f16: undo the row's 2^-e
            float hv[NH];
#pragma unroll
            for (int q = 0; q < NH; ++q) {
              if constexpr (MODE == MODE_SILU) {
                const float gt = acc[mf][2 * q][i] * rsc, up = acc[mf][2 * q + 1][i] * rsc;
                hv[q] = p.oai ? swiglu_oai(gt, up) : gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
              } else {
                const float z = acc[mf][q][i] * rsc;
                hv[q] = z > 0.f ? z * z : 0.f;
              }
            }
            if constexpr (NVRT) {
              // NVFP4 blocks of 16 columns = one column block (the 16 lanes of
              // a row); h is the bf16 value E2M1 * E4M3 of its round trip, the
              // expert's activation scale is applied by the down GEMM
              const float gh = p.hglobal[e];
#pragma unroll
              for (int q = 0; q < NH; ++q) {
                if (q < nh) {
                  float m = fabsf(hv[q]);
                  m = row16_max(m);
                  const float sc = nv_block_scale(m, gh), rc = nv_recip(sc, gh);
                  p.h16[row * p.h_stride + hcol0 + 16 * q + r16] = (uint16_t)bf16_rne(nv_roundtrip(hv[q], sc, gh, rc));
                }
              }
            } else if constexpr (RT) {
              // MXFP8 blocks of 32 columns = column blocks (2b, 2b+1); h is the
              // bf16 value of its round trip
              static_assert(NH % 2 == 0, "whole MXFP8 blocks per wave");
#pragma unroll
              for (int blk = 0; blk < NH / 2; ++blk) {
                if (2 * blk < nh) {
                  float m = fmaxf(fabsf(hv[2 * blk]), fabsf(hv[2 * blk + 1]));
                  m = row16_max(m);
                  const int sx = mx_scale_exp(f32_bits(m));
                  const int64_t col = hcol0 + 32 * blk + r16;
                  p.h16[row * p.h_stride + col] = (uint16_t)mx_roundtrip_bf16(hv[2 * blk], sx);
                  p.h16[row * p.h_stride + col + 16] = (uint16_t)mx_roundtrip_bf16(hv[2 * blk + 1], sx);
                }
              }
            } else if constexpr (!A8) {
#pragma unroll
              for (int q = 0; q < NH; ++q)
                if (q < nh) p.h16[row * p.h_stride + hcol0 + 16 * q + r16] = (uint16_t)bf16_rne(hv[q]);
            } else {
              // MXFP8 blocks of 32 columns = column blocks (2b, 2b+1)
#pragma unroll
              for (int blk = 0; blk < NH / 2; ++blk) {
                if (2 * blk < nh) {
                  float m = fmaxf(fabsf(hv[2 * blk]), fabsf(hv[2 * blk + 1]));
                  m = row16_max(m);
                  const int sx = mx_scale_exp(f32_bits(m));
                  const int64_t col = hcol0 + 32 * blk + r16;
                  p.h8[row * p.h_stride + col] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[2 * blk]), sx);
                  p.h8[row * p.h_stride + col + 16] = (uint8_t)e4m3_encode_scaled(f32_bits(hv[2 * blk + 1]), sx);
                  if (r16 == 0) p.hs[row * p.hs_stride + (hcol0 + 32 * blk) / 32] = (uint8_t)(sx + 127);
                }
              }
            }
          }
        }
      }
    }
  }
  // no DMA into LDS may still be in flight when the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

constexpr int kGemmNFW = 4;  // weight fragments per wave: workgroup tile 128 rows x 256 columns

// Persistent grid: two workgroups per CU, a multiple of 8 (one share per XCD).
// Defined here, instantiated for each (weight format, activation format,
// mode) in the gemm_inst_*.hip sources so that they compile in parallel.
template <int WF, int AF, int MODE>
int launch_gemm_t(const GemmParams& p, int64_t max_work, hipStream_t s) {
  int64_t grid = 2 * (int64_t)device_cu_count();
  if (max_work < grid) grid = (max_work + 7) / 8 * 8;
  grid = grid / 8 * 8;
  if (grid <= 0) grid = 8;
  hipLaunchKernelGGL((moe_gemm_kernel<WF, AF, MODE, kGemmNFW>), dim3((unsigned)grid), dim3(kGemmThreads), 0, s, p);
  return (int)hipGetLastError();
}

#define B12X_GEMM_EXTERN(WF, AF, MODE) extern template int launch_gemm_t<WF, AF, MODE>(const GemmParams&, int64_t, hipStream_t);
#define B12X_GEMM_INST(WF, AF, MODE) template int launch_gemm_t<WF, AF, MODE>(const GemmParams&, int64_t, hipStream_t);

}  // namespace b12x
