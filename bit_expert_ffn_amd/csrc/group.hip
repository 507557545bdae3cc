// Token-to-expert grouping on the device: a stable counting sort of the T*k (token, slot) rows
// by expert, plus the active experts sorted by row count.  Index building stays on the device
// with no host round trip ("Day-0 Inference Adaptation for Ultra-Large Sparse Models",
// "Operator Layer", Index Pipeline); sorting a step's experts by row count feeds the split into
// few-row and busy experts ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU",
// section 5 "Keeping register pressure off the common path").
//
// Stability without order-dependent atomics: each wavefront owns a contiguous range of slots,
// counts it per expert in LDS, and a per-expert exclusive scan over the wavefronts (in order)
// gives each wavefront its base.  Inside a wavefront, slots are taken 64 at a time; a lane's
// rank among the earlier lanes holding the same expert comes from 8 ballots (one per bit of the
// expert id).  Outputs are therefore bit-exact and identical from run to run.
//
// Small problems (T*k <= 16384) run as one 1024-thread block.  Larger ones run in three passes:
// per-wavefront histograms, a per-expert scan, and the scatter.
#include "common.h"

namespace moe {

constexpr int kGroupWaves = 16;  // wavefronts per block

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

// Active experts by (count desc, id asc); thread e places expert e.  Needs >= E threads.
__device__ inline void place_active(const int* cnt, int E, int32_t* __restrict__ active,
                                    int32_t* __restrict__ n_active) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int c = cnt[e];
  int rank = 0, nact = 0;
  for (int j = 0; j < E; ++j) {
    const int cj = cnt[j];
    nact += cj > 0;
    rank += (cj > c) || (cj == c && j < e);
  }
  if (c > 0) active[rank] = e;
  if (e >= nact) active[e] = -1;
  if (e == 0) *n_active = nact;
}

__global__ __launch_bounds__(1024) void group_small_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ count,
    int32_t* __restrict__ offset, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ active, int32_t* __restrict__ n_active) {
  __shared__ int wcnt[kGroupWaves][kMaxExperts];
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  for (int i = tid; i < kGroupWaves * kMaxExperts; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int per = (n + kGroupWaves - 1) / kGroupWaves;
  const int s0 = min(n, wv * per), s1 = min(n, s0 + per);
  wave_hist(ids, s0, s1, wcnt[wv]);
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < kGroupWaves; ++w) {
      const int c = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += c;
    }
    cnt[tid] = run;
  }
  __syncthreads();
  if (wv == 0) wave_scan_offsets(cnt, E, off);
  __syncthreads();
  if (tid < E) {
    for (int w = 0; w < kGroupWaves; ++w) wcnt[w][tid] += off[tid];
    count[tid] = cnt[tid];
    offset[tid] = off[tid];
    if (tid == 0) offset[E] = off[E];
  }
  __syncthreads();
  wave_scatter(ids, s0, s1, E, wcnt[wv], sorted_slot, slot_row);
  place_active(cnt, E, active, n_active);
}

// Pass 1: per-wavefront histograms of each block's kGroupChunk slots -> whist[blk*16+w][E].
__global__ __launch_bounds__(1024) void group_hist_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int32_t* __restrict__ whist) {
  __shared__ int wcnt[kGroupWaves][kMaxExperts];
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int i = tid; i < kGroupWaves * kMaxExperts; i += 1024) (&wcnt[0][0])[i] = 0;
  __syncthreads();
  const int per = kGroupChunk / kGroupWaves;
  const int s0 = min(n, blockIdx.x * kGroupChunk + wv * per), s1 = min(n, s0 + per);
  wave_hist(ids, s0, s1, wcnt[wv]);
  __syncthreads();
  for (int i = tid; i < kGroupWaves * E; i += 1024) {
    const int w = i / E, e = i % E;
    whist[((size_t)blockIdx.x * kGroupWaves + w) * E + e] = wcnt[w][e];
  }
}

// Pass 2 (one block): per-expert exclusive scan over all wavefronts, offsets, active list.
// whist entries become each wavefront's first row for the expert.
__global__ __launch_bounds__(256) void group_scan_kernel(int32_t* __restrict__ whist, int nw,
                                                         int E, int32_t* __restrict__ count,
                                                         int32_t* __restrict__ offset,
                                                         int32_t* __restrict__ active,
                                                         int32_t* __restrict__ n_active) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  const int tid = threadIdx.x;
  if (tid < E) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int c = whist[(size_t)w * E + tid];
      whist[(size_t)w * E + tid] = run;
      run += c;
    }
    cnt[tid] = run;
  }
  __syncthreads();
  if (tid < 64) wave_scan_offsets(cnt, E, off);
  __syncthreads();
  if (tid < E) {
    count[tid] = cnt[tid];
    offset[tid] = off[tid];
    if (tid == 0) offset[E] = off[E];
    for (int w = 0; w < nw; ++w) whist[(size_t)w * E + tid] += off[tid];
  }
  place_active(cnt, E, active, n_active);
}

// Pass 3: scatter each wavefront's slots from its per-expert first rows.
__global__ __launch_bounds__(1024) void group_scatter_kernel(const int32_t* __restrict__ ids,
                                                             int n, int E,
                                                             const int32_t* __restrict__ whist,
                                                             int32_t* __restrict__ sorted_slot,
                                                             int32_t* __restrict__ slot_row) {
  __shared__ int wcnt[kGroupWaves][kMaxExperts];
  const int tid = threadIdx.x, wv = tid >> 6;
  for (int i = tid; i < kGroupWaves * E; i += 1024) {
    const int w = i / E, e = i % E;
    wcnt[w][e] = whist[((size_t)blockIdx.x * kGroupWaves + w) * E + e];
  }
  __syncthreads();
  const int per = kGroupChunk / kGroupWaves;
  const int s0 = min(n, blockIdx.x * kGroupChunk + wv * per), s1 = min(n, s0 + per);
  wave_scatter(ids, s0, s1, E, wcnt[wv], sorted_slot, slot_row);
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* count,
                        int32_t* offset, int32_t* sorted_slot, int32_t* slot_row,
                        int32_t* active, int32_t* n_active, int32_t* whist, hipStream_t s) {
  const int n = T * k;
  if (n <= kGroupSmallMax) {
    group_small_kernel<<<1, 1024, 0, s>>>(ids, n, E, count, offset, sorted_slot, slot_row,
                                          active, n_active);
  } else {
    const int nblk = (n + kGroupChunk - 1) / kGroupChunk;
    group_hist_kernel<<<nblk, 1024, 0, s>>>(ids, n, E, whist);
    group_scan_kernel<<<1, 256, 0, s>>>(whist, nblk * kGroupWaves, E, count, offset, active,
                                        n_active);
    group_scatter_kernel<<<nblk, 1024, 0, s>>>(ids, n, E, whist, sorted_slot, slot_row);
  }
  return hipGetLastError();
}

}  // namespace moe
