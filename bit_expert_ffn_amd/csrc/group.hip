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
#include "group_dev.h"

namespace moe {

constexpr int kGroupWaves = 16;  // wavefronts per block

__global__ __launch_bounds__(1024) void group_small_kernel(
    const int32_t* __restrict__ ids, int n, int E, int32_t* __restrict__ count,
    int32_t* __restrict__ offset, int32_t* __restrict__ sorted_slot,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
    GroupPlan plan) {
  __shared__ int wcnt[kGroupWaves][kMaxExperts];
  __shared__ __attribute__((aligned(16))) uint32_t key[kMaxExperts];
  __shared__ int act_l[kMaxExperts];  // the active list, for the tile plan
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int rank[kMaxExperts];
  __shared__ int s_nact;
  __shared__ int32_t sids[kGroupSmallMax];  // the expert ids, read from global memory once
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  for (int i = tid; i < n; i += 1024) sids[i] = ids[i];
  for (int i = tid; i < kGroupWaves * kMaxExperts; i += 1024) (&wcnt[0][0])[i] = 0;
  if (tid < kMaxExperts) {
    cnt[tid] = 0;
    rank[tid] = 0;
    key[tid] = 0;
  }
  if (tid == 0) s_nact = 0;
  __syncthreads();
  const int per = (n + kGroupWaves - 1) / kGroupWaves;
  const int s0 = min(n, wv * per), s1 = min(n, s0 + per);
  wave_hist(sids, s0, s1, wcnt[wv]);
  __syncthreads();
  // per expert: exclusive scan of the 16 wavefront counts.  Thread (e, q) owns wavefronts
  // 4q..4q+3 of expert e; the 4 threads of an expert are adjacent lanes.
  const int q = tid & 3, ex = tid >> 2;
  {
    int c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = ex < E ? wcnt[4 * q + i][ex] : 0;
      sum += c[i];
    }
    int incl = sum;
    int v = __shfl_up(incl, 1, 4);
    if (q >= 1) incl += v;
    v = __shfl_up(incl, 2, 4);
    if (q >= 2) incl += v;
    const int total = __shfl(incl, 3, 4);
    int run = incl - sum;
    if (ex < E) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        wcnt[4 * q + i][ex] = run;
        run += c[i];
      }
      if (q == 0) cnt[ex] = total;
    }
  }
  __syncthreads();
  if (wv == 0) wave_scan_offsets(cnt, E, off);
  __syncthreads();
  if (ex < E) {
#pragma unroll
    for (int i = 0; i < 4; ++i) wcnt[4 * q + i][ex] += off[ex];
    if (q == 0) {
      count[ex] = cnt[ex];
      offset[ex] = off[ex];
      // ranking key: larger key = earlier in the active list (count desc, then id asc);
      // counts are <= n <= 16384 < 2^24
      key[ex] = ((uint32_t)cnt[ex] << 8) | (uint32_t)(255 - ex);
      if (ex == 0) offset[E] = off[E];
    }
  }
  __syncthreads();
  wave_scatter(sids, s0, s1, E, wcnt[wv], sorted_slot, slot_row);
  // rank of expert e = number of larger keys; thread (e, seg) counts over 64 keys
  {
    const int e = tid & 255, seg = tid >> 8;
    const uint32_t ke = key[e];
    int r = 0, na = 0;
    const uint4* k4 = reinterpret_cast<const uint4*>(key + seg * 64);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint4 kk = k4[j];
      r += (kk.x > ke) + (kk.y > ke) + (kk.z > ke) + (kk.w > ke);
      na += (kk.x > 255u) + (kk.y > 255u) + (kk.z > 255u) + (kk.w > 255u);
    }
    if (e < E && ke > 255u) atomicAdd(&rank[e], r);
    if (e == 0) atomicAdd(&s_nact, na);
  }
  __syncthreads();
  if (tid < E) {
    const int nact = s_nact;
    if (key[tid] > 255u) {
      active[rank[tid]] = tid;
      act_l[rank[tid]] = tid;
    }
    if (tid >= nact) active[tid] = -1;
    if (tid == 0) *n_active = nact;
  }
  if (plan.MT > 0) {  // uniform over the block
    __syncthreads();
    if (wv == 0)
      ffn_plan_n(cnt, off, act_l, s_nact, plan.MT, plan.min_rows, plan.tiles, plan.max_tiles,
                 plan.n_tiles);
  }
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

// Pass 2 (one block of 1024 threads): per-expert exclusive scan over all wavefronts, offsets,
// active list.  Thread (q, e) takes quarter q of the wavefront range of expert e, with up to 64
// loads in flight: first its quarter's total, then (after the offsets) each wavefront's first
// row.  whist entries become each wavefront's first row for the expert.
__global__ __launch_bounds__(1024) void group_scan_kernel(int32_t* __restrict__ whist, int nw,
                                                          int E, int32_t* __restrict__ count,
                                                          int32_t* __restrict__ offset,
                                                          int32_t* __restrict__ active,
                                                          int32_t* __restrict__ n_active) {
  constexpr int kB = 64;  // loads in flight per thread
  __shared__ __attribute__((aligned(16))) int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int part[4][kMaxExperts];
  const int tid = threadIdx.x;
  // q is the same for the four wavefronts of a quarter: made uniform, the row offsets below are
  // scalar and each load takes one scalar base plus the lane's expert offset
  const int e = tid & (kMaxExperts - 1), q = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int per = (nw + 3) / 4, w0 = min(nw, q * per), w1 = min(nw, w0 + per);
  if (tid < kMaxExperts) cnt[tid] = 0;
  int tot = 0;
  if (e < E) {
    for (int wb = w0; wb < w1; wb += kB) {
      // unconditional loads (past w1 clamped, not added), so that all of them are in flight
      int c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = (whist + (size_t)min(wb + u, w1 - 1) * E)[e];
#pragma unroll
      for (int u = 0; u < kB; ++u) tot += wb + u < w1 ? c[u] : 0;
    }
  }
  part[q][e] = tot;
  __syncthreads();
  if (tid < E) cnt[tid] = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
  __syncthreads();
  if (tid < 64) wave_scan_offsets(cnt, E, off);
  __syncthreads();
  if (e < E) {
    int run = off[e];
    for (int j = 0; j < q; ++j) run += part[j][e];
    for (int wb = w0; wb < w1; wb += kB) {
      int c[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) c[u] = (whist + (size_t)min(wb + u, w1 - 1) * E)[e];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        if (wb + u < w1) {
          (whist + (size_t)(wb + u) * E)[e] = run;
          run += c[u];
        }
      }
    }
  }
  if (tid < E) {
    count[tid] = cnt[tid];
    offset[tid] = off[tid];
    if (tid == 0) offset[E] = off[E];
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
                        int32_t* active, int32_t* n_active, int32_t* whist, hipStream_t s,
                        const GroupPlan* plan) {
  const int n = T * k;
  if (n <= kGroupSmallMax) {
    GroupPlan p{0, 0, 0, nullptr, nullptr};
    if (plan) p = *plan;
    group_small_kernel<<<1, 1024, 0, s>>>(ids, n, E, count, offset, sorted_slot, slot_row,
                                          active, n_active, p);
  } else {
    if (plan && plan->MT > 0) return hipErrorInvalidValue;  // the three-pass grouping plans nothing
    const int nblk = (n + kGroupChunk - 1) / kGroupChunk;
    group_hist_kernel<<<nblk, 1024, 0, s>>>(ids, n, E, whist);
    group_scan_kernel<<<1, 1024, 0, s>>>(whist, nblk * kGroupWaves, E, count, offset, active,
                                         n_active);
    group_scatter_kernel<<<nblk, 1024, 0, s>>>(ids, n, E, whist, sorted_slot, slot_row);
  }
  return hipGetLastError();
}

}  // namespace moe
