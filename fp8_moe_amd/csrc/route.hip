// Integer routing stage of the grouped path (b12x README "Using it": the op
// binds caller-supplied topk_ids / topk_weights; "What's in here": routed
// experts run on a persistent grid).  Produces, for pair p = t*k + j:
// per-expert counts, exclusive offsets, offsets of rows padded per expert to
// kRowPad, the stable expert-major permutation of the pairs (padding rows -1),
// each pair's row and the list of (expert, first row, rows) GEMM tiles (each
// expert's rows split evenly into the fewest tiles of at most kTileRows).
// Three launches: per-chunk histograms, one scan workgroup, per-chunk scatter.
// Integer atomics only touch LDS counters whose final values are
// order-independent; every written position is deterministic.
#include "device_common.h"

namespace b12x {

constexpr int kRouteThreads = 256;
constexpr int kPairsPerThread = kRouteChunk / kRouteThreads;

__device__ __forceinline__ int valid_expert(int e, int E) { return e >= 0 && e < E; }

// chunk[c * E + e] = number of valid pairs of chunk c routed to e.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* __restrict__ ids, LiveT lv,
                                                                     int E, int32_t* __restrict__ chunk) {
  const int64_t T = lv.tokens();
  if (!lv.on()) return;
  const int64_t P = T * lv.k;
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk;
  for (int i = 0; i < kPairsPerThread; ++i) {
    const int64_t p = base + i * kRouteThreads + threadIdx.x;
    if (p < P) {
      const int e = ids[p];
      if (valid_expert(e, E)) atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads) chunk[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Block-wide exclusive scans of three ints per thread (blockDim.x = 1024):
// inclusive scans within each wave, then the wave totals in LDS (one
// barrier).  ex and tot receive the exclusive prefixes and the block totals.
__device__ void block_exclusive_scan3(const int (&v)[3], int (*wsum)[3], int (&ex)[3], int (&tot)[3]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int t = __shfl_up(incl[q], off);
      if (lane >= off) incl[q] += t;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int q = 0; q < 3; ++q) wsum[wave][q] = incl[q];
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    int before = 0, all = 0;
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[w][q];
      before += w < wave ? x : 0;
      all += x;
    }
    ex[q] = before + incl[q] - v[q];
    tot[q] = all;
  }
}

// One workgroup of 1024 threads, thread e = expert e.
__global__ __launch_bounds__(1024) void route_scan_kernel(int E, int n_chunks, int32_t* __restrict__ chunk,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ poff, int32_t* __restrict__ sorted,
                                                          int32_t* __restrict__ tiles, int32_t* __restrict__ ntiles,
                                                          LiveT lv) {
  if (!lv.on()) return;
  __shared__ int wsum[16][3];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    // chunk counts -> exclusive per-chunk bases, eight chunks' loads in flight at a time
    for (int c0 = 0; c0 < n_chunks; c0 += 8) {
      int h[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) h[u] = c0 + u < n_chunks ? chunk[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < n_chunks) chunk[(int64_t)(c0 + u) * E + e] = cnt;
        cnt += h[u];
      }
    }
  }
  const int padded = (cnt + kRowPad - 1) / kRowPad * kRowPad;
  // balanced tiles: the expert's 16-row blocks split as evenly as possible into
  // the fewest tiles of at most kTileRows rows (larger tiles first)
  constexpr int kTileBlocks = kTileRows / kRowPad;
  const int nb = padded / kRowPad;
  const int n_t = (nb + kTileBlocks - 1) / kTileBlocks;
  const int vals[3] = {cnt, padded, n_t};
  int ex[3], tot[3];
  block_exclusive_scan3(vals, wsum, ex, tot);
  const int off = ex[0], poffe = ex[1], toff = ex[2];
  const int tot_cnt = tot[0], tot_pad = tot[1], tot_tiles = tot[2];
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    poff[e] = poffe;
    for (int r = poffe + cnt; r < poffe + padded; ++r) sorted[r] = -1;
    const int q = n_t ? nb / n_t : 0, rem = n_t ? nb % n_t : 0;
    for (int i = 0; i < n_t; ++i) {
      const int r0 = poffe + (i * q + min(i, rem)) * kRowPad;
      const int rows = (q + (i < rem ? 1 : 0)) * kRowPad;
      *(int4*)(tiles + 4 * (toff + i)) = make_int4(e, r0, rows, 0);
    }
  }
  if (e == 0) {
    offsets[E] = tot_cnt;
    poff[E] = tot_pad;
    *(int4*)ntiles = make_int4(tot_tiles, tot_pad, 0, 0);
  }
}

// Stable scatter: each wave takes 256 consecutive pairs of the chunk in four
// rounds of 64; a lane's rank among equal experts of its round comes from
// ballots (the lanes below it with the same expert, found with one ballot per
// bit of the expert id), and LDS counters carry the count across rounds.  Waves are then ordered by a prefix over their counts.
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(const int32_t* __restrict__ ids, LiveT lv,
                                                                       int E, const int32_t* __restrict__ chunk,
                                                                       const int32_t* __restrict__ poff,
                                                                       int32_t* __restrict__ sorted,
                                                                       int32_t* __restrict__ pos) {
  const int64_t T = lv.tokens();
  if (!lv.on()) return;
  const int64_t P = T * lv.k;
  __shared__ int cnt[4][kMaxExperts];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * kMaxExperts; i += kRouteThreads) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kRouteChunk + wave * 256;
  int my_e[4], my_rank[4];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int id_bits = E > 1 ? 32 - __builtin_clz((unsigned)(E - 1)) : 0;  // bits of the largest id
  for (int r = 0; r < 4; ++r) {
    const int64_t p = base + r * 64 + lane;
    int e = p < P ? ids[p] : -1;
    const bool v = valid_expert(e, E);
    if (!v) e = -1;
    my_e[r] = e;
    my_rank[r] = -1;
    // lanes with this lane's expert: the valid lanes that agree with it on
    // every bit of the id (one ballot per bit)
    uint64_t same = __ballot(v);
    for (int b = 0; b < id_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    if (v) {
      // every lane of the group reads the counter, then the group's lowest
      // lane advances it (the wave's LDS reads and writes run in program order)
      const int before = cnt[wave][e];
      my_rank[r] = before + __builtin_popcountll(same & below);
      __builtin_amdgcn_wave_barrier();
      if ((same & below) == 0) cnt[wave][e] = before + __builtin_popcountll(same);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int r = 0; r < 4; ++r) {
    const int64_t p = base + r * 64 + lane;
    if (p >= P) continue;
    const int e = my_e[r];
    if (e < 0) {
      pos[p] = -1;
      continue;
    }
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += cnt[w][e];
    const int row = poff[e] + chunk[(int64_t)blockIdx.x * E + e] + wbase + my_rank[r];
    sorted[row] = (int32_t)p;
    pos[p] = row;
  }
}

// Grids cover the binding's capacity (its T, or the live binding's largest T);
// with a live token count the chunks past the live pairs count nothing.
int launch_route(const BindingImpl& b, hipStream_t s) {
  const int64_t P = b.T * b.k;
  const int n_chunks = (int)((P + kRouteChunk - 1) / kRouteChunk);
  const LiveT lv = b.live();
  hipLaunchKernelGGL(route_count_kernel, dim3(n_chunks), dim3(kRouteThreads), 0, s, b.ids, lv, b.E, b.chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, s, b.E, n_chunks, b.chunk, b.counts, b.offsets,
                     b.poff, b.sorted, b.tiles, b.ntiles, lv);
  e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(route_scatter_kernel, dim3(n_chunks), dim3(kRouteThreads), 0, s, b.ids, lv, b.E, b.chunk,
                     b.poff, b.sorted, b.pos);
  return (int)hipGetLastError();
}

}  // namespace b12x
