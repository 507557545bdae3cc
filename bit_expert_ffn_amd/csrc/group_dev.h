// Device helpers of the stable counting sort by expert (internal header): used by the
// grouping kernels and by the fused routing kernel.
#pragma once
#include "common.h"

namespace moe {

__device__ inline uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

// Rank of this lane among the lanes of `valid` holding the same expert, and that group's mask.
__device__ inline uint64_t same_expert_mask(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bal = __ballot(bit);
    m &= ((e >> b) & 1) ? bal : ~bal;
  }
  return m;
}

__device__ inline int expert_bits(int E) {
  int nb = 0;
  while ((1 << nb) < E) ++nb;
  return nb;
}

// Per-wavefront histogram of slots [s0, s1) into hist[E] (LDS).
__device__ inline void wave_hist(const int32_t* __restrict__ ids, int s0, int s1, int* hist) {
  const int lane = threadIdx.x & 63;
  for (int s = s0 + lane; s < s1; s += 64) atomicAdd(&hist[ids[s]], 1);
}

// Scatter slots [s0, s1) of one wavefront; run[e] holds the next row of expert e for it.
__device__ inline void wave_scatter(const int32_t* __restrict__ ids, int s0, int s1, int E,
                                    int* run, int32_t* __restrict__ sorted_slot,
                                    int32_t* __restrict__ slot_row) {
  const int lane = threadIdx.x & 63;
  const int nb = expert_bits(E);
  for (int base = s0; base < s1; base += 64) {
    const int s = base + lane;
    const bool valid = s < s1;
    const int e = valid ? ids[s] : 0;
    const uint64_t m = same_expert_mask(e, valid, nb);
    const int rank = __popcll(m & lanemask_lt(lane));
    int pos = 0;
    if (valid) pos = run[e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (valid) {
      sorted_slot[pos] = s;
      slot_row[s] = pos;
      const int last = 63 - __clzll(m);
      if (lane == last) run[e] = pos + 1;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Exclusive scan of cnt[0..E) into off[0..E] by wavefront 0 (4 experts per lane).
__device__ inline void wave_scan_offsets(const int* cnt, int E, int* off) {
  const int lane = threadIdx.x & 63;
  int c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    c[i] = e < E ? cnt[e] : 0;
    sum += c[i];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane * 4 + i;
    if (e < E) off[e] = run;
    run += c[i];
  }
  if (lane == 63) off[E] = incl;
}

// Active experts by (count desc, id asc); thread e places expert e.  Needs >= E threads and
// cnt[] zero-filled up to kMaxExperts (read 4 at a time).
__device__ inline void place_active(const int* cnt, int E, int32_t* __restrict__ active,
                                    int32_t* __restrict__ n_active) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int c = cnt[e];
  int rank = 0, nact = 0;
  const int4* c4 = reinterpret_cast<const int4*>(cnt);
  const int n4 = (E + 3) >> 2;
#pragma unroll 8
  for (int j4 = 0; j4 < n4; ++j4) {
    const int4 v = c4[j4];
    const int j = j4 * 4;
    nact += (v.x > 0) + (v.y > 0) + (v.z > 0) + (v.w > 0);
    rank += (v.x > c) || (v.x == c && j < e);
    rank += (v.y > c) || (v.y == c && j + 1 < e);
    rank += (v.z > c) || (v.z == c && j + 2 < e);
    rank += (v.w > c) || (v.w == c && j + 3 < e);
  }
  if (c > 0) active[rank] = e;
  if (e >= nact) active[e] = -1;
  if (e == 0) *n_active = nact;
}

}  // namespace moe
