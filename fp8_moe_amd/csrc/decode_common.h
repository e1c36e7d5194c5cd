// Device helpers shared by the decode-path kernels (decode.hip,
// decode_sk.hip): routing rebuilt in LDS from topk_ids by every workgroup.
#pragma once
#include "device_common.h"

namespace b12x {

constexpr int kDecThreads = 256;
constexpr int kBitWords = kMaxExperts / 32;
static_assert(kBitWords <= 64, "one wave scans the expert bitmap");

// topk_ids -> LDS (invalid ids as -1), the bitmap of valid experts and the
// exclusive prefix popcounts of its words; returns the number of distinct
// valid experts.  All threads call it.
__device__ inline int decode_prep(const int32_t* ids, int P, int E, int* s_ids, uint32_t* s_bits, int* s_wpre) {
  const int tid = threadIdx.x;
  const int words = (E + 31) >> 5;
  for (int i = tid; i < words; i += kDecThreads) s_bits[i] = 0;
  __syncthreads();
  for (int q = tid; q < P; q += kDecThreads) {
    const int e = ids[q];
    const bool v = e >= 0 && e < E;
    s_ids[q] = v ? e : -1;
    if (v) atomicOr(&s_bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (tid < 64) {  // wave 0: words <= 64
    const int c = tid < words ? __builtin_popcount(s_bits[tid]) : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (tid >= off) incl += t;
    }
    if (tid < words) s_wpre[tid] = incl - c;
    if (tid == 63) s_wpre[kBitWords] = incl;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_wpre[kBitWords]);
}

// Expert of touched slot `slot` (the slot-th smallest distinct valid id) and
// its pairs in ascending pair order into s_rows; returns the pair count.
// All threads call it; it starts with a barrier, so the caller may reuse
// s_rows and s_info right after its own last reads.
__device__ inline int decode_expert(int P, int E, int slot, const int* s_ids, const uint32_t* s_bits,
                                    const int* s_wpre, int* s_rows, int* s_info, int& e_out) {
  const int tid = threadIdx.x;
  const int words = (E + 31) >> 5;
  __syncthreads();
  if (tid < words && slot >= s_wpre[tid] && slot < s_wpre[tid] + __builtin_popcount(s_bits[tid])) {
    uint32_t b = s_bits[tid];
    for (int r = slot - s_wpre[tid]; r > 0; --r) b &= b - 1;  // drop the lower set bits
    s_info[0] = tid * 32 + __builtin_ctz(b);
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_info[0]);
  e_out = e;
  // stable list of e's pairs: ballots per wave, waves ordered by a prefix
  const int wave = tid >> 6, lane = tid & 63;
  const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
  int total = 0;
  for (int base = 0; base < P; base += kDecThreads) {
    const int q = base + tid;
    const bool hit = q < P && s_ids[q] == e;
    const uint64_t bal = __ballot(hit);
    if (lane == 0) s_info[4 + wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += s_info[4 + w];
    if (hit) s_rows[off + __builtin_popcountll(bal & below)] = q;
    total += s_info[4] + s_info[5] + s_info[6] + s_info[7];
    __syncthreads();
  }
  return __builtin_amdgcn_readfirstlane(total);
}

struct DecodeLds {
  int ids[kDecodePairs];
  int rows[kDecodePairs];
  uint32_t bits[kBitWords];
  int wpre[kBitWords + 1];
  int info[8];
};

// Workgroups the device holds at once for one kernel (per device, cached by
// the caller: one cache per kernel).
template <typename Kernel>
static int resident_workgroups(Kernel kernel, int (&cache)[64]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cache[dev]) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kDecThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    cache[dev] = per_cu * device_cu_count();
  }
  return cache[dev];
}

}  // namespace b12x
