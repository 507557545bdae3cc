// Single-launch layer for one or two tokens: router, top-k + softmax, grouping, gate/up +
// SwiGLU, down and the weighted combine in one persistent kernel.
//
// Sources: at small batch a step does little math per weight and is bound by HBM streaming, so
// the whole step runs as one program with no launch gaps, and each chosen expert's weights are
// requested the moment routing ends ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", section 1 "A megakernel" and section 2 "Pipelining everything inside the
// megakernel"); per expert gate/up, SwiGLU, down and a weighted sum read once (same page,
// section 8, "The fused MoE kernel and the pair exchange", "A one-pass combine").
//
// One block of 256 threads per CU; every block is resident (the host checks occupancy), so
// blocks can wait for each other.  Phases:
//   A  router partial logits.  Item = (1/32 of the hidden rows, 32 experts); each block's
//      partial sums go out with device-scope stores; every block then arrives on counter A and
//      stages the x rows in LDS while the others finish.
//   B  every block waits for counter A, adds the 32 slices in order, adds the bias, ranks the
//      experts, takes the softmax over the top k and groups the T*k (token, slot) rows by
//      expert: redundantly and in LDS, so that no second barrier is needed.  Block 0 also
//      writes the routing and grouping arrays.
//   C  gate/up + SwiGLU.  Item = (active expert, 16 features) per wavefront over the whole
//      hidden dimension; rows of h (f16) go out with device-scope stores; then counter C.
//   D  down + combine.  A block takes two 16-feature tiles of the output, each split over two
//      halves of the intermediate dimension (one wavefront each).  A wavefront issues the loads
//      of its first expert's weights, then waits for counter C, stages its half of every h row
//      in LDS and streams the down weights of every active expert;
//      out[t][f] = sum over the token's rows of w * ts_d * (W_d h), the halves added in LDS.
//   Per-XCD mode (one token with k = 8, the grid a multiple of 8): group g of blocks (index mod
//   8, which the hardware places on one XCD) runs slot g's expert alone.  In C its wavefronts take
//   that expert's 16-feature tiles; barrier C becomes one barrier per group (32 arrivals instead
//   of 256, and no wait for the other experts); D stages only slot g's h row and computes that
//   expert's down projection over every output feature, block j of the group taking range j of
//   the tiles.  Each block writes w_g * (W_d h) for its range to row g of a partial buffer; the
//   eighth block of range j to arrive at the range's counter adds the 8 rows in slot order and
//   writes out.  (Measured at decode: 50.4 -> 47.4 us.)
//   Exit: counter X; the last block to arrive resets the counters and flags for the next call.
//   A block arrives there once it has passed its last wait (barrier C, for a block with output
//   tiles), before its down phase, so that the reset overlaps the down phase.
//   In the per-XCD mode every block's last act is its arrival at its range's counter, so the
//   eighth arrival of each range also adds one to a count of finished ranges, and the arrival
//   that completes that count resets everything: no exit barrier behind the sums.
// A barrier: every block adds one to the barrier's counter; the block that completes it raises
// 16 copies of a flag, and each block polls its own copy.
// Failure: every wait is bounded (word kLsSyncSpin of the sync region, if non-zero, sets the
// number of polls; else kLsSpin, about 2 s).  A block whose wait gives up sets the error word,
// writes NaN over its output tiles, skips the rest of its work and still arrives at counter X,
// so the last block to exit resets the counters and flags whether or not the call succeeded: a
// failed call leaves NaN in out and the error word set, but cannot leave a barrier
// half-counted for the next call.  In the per-XCD mode a block that gives up writes NaN over
// its features of h (at barrier A) and over its row of the partial buffer, and still makes
// every arrival it has left (group barrier C, its range), so every range's sum is NaN where a
// block gave up and the count of finished ranges still completes.
// Data that crosses blocks (partial logits, h) is written with device-scope stores, which write
// through the per-XCD L2s (not coherent with each other) to memory, and read after the barrier
// with device-scope loads (global_load sc1), which do not take a possibly stale line from the
// reader's L2; the counters are relaxed device-scope atomics issued after a full s_waitcnt, so
// each block's stores are complete before its arrival.  No cache-wide release or acquire fence
// is needed.  (Measured at decode: the device-scope loads cost under 0.2 us against plain
// loads; a cooperative launch, which would refuse a grid that cannot be co-resident, took
// 70.3 against 52.9 us for the plain launch, so the host's occupancy check stays.)
#include <mutex>

#include "common.h"
#include "dot.h"
#include "select_dev.h"
#include "sync.h"

namespace moe {

// Profiling builds only (compiled with -DMOE_TIMELINE): each block's first thread records the
// 100 MHz real-time counter at the phase boundaries of the last call, read back with
// moe_timeline_layer_small.  Slots: 0 entry, 1 router partials stored, 2 barrier A passed,
// 3 routing published (gate/up starts), 4 gate/up done, 5 barrier C passed, 6 h staged, 7 exit;
// inside the routing: 8 logits summed, 9 first-level ranks, 10 candidate ranks, 11 first gate/up
// sets issued (one token); in the per-XCD down phase: 12 first set used, 13 last set used,
// 14 range counter passed.
#ifdef MOE_TIMELINE
__device__ unsigned long long g_ls_timeline[1024][16];
#define LS_STAMP(i)                                                                 \
  do {                                                                              \
    if (threadIdx.x == 0 && blockIdx.x < 1024)                                      \
      g_ls_timeline[blockIdx.x][i] = __builtin_amdgcn_s_memrealtime();              \
  } while (0)
#else
#define LS_STAMP(i) \
  do {              \
  } while (0)
#endif

constexpr int kLsNS = 32;                 // router: slices of the hidden dimension
constexpr int kLsEG = 32;                 // router: experts per item
constexpr int kLsSetC = 4;                // gate/up: chunks per load set
constexpr int kLsSetD = 8;                // down: chunks per load set
constexpr int kLsXTiles = 8;              // per-XCD mode: output tiles per wavefront, at most
// A block that gave up waiting writes NaN over its output tiles (the 32-feature tiles
// blockIdx.x + m * G of every token), so a failed call shows in out: a give-up at barrier A
// keeps barrier A or C from completing for everyone, so every block with output tiles gives up.
__device__ inline void ls_fail_out(const LayerSmallArgs& a, int G) {
  const float nan = __builtin_nanf("");
  for (int ftp = blockIdx.x; ftp < a.H / 32; ftp += G)
    for (int i = threadIdx.x; i < a.T * 32; i += 256)
      a.out[(size_t)(i >> 5) * a.H + ftp * 32 + (i & 31)] = nan;
}

// Wavefront sum of the device library (ockl): the sum over all active lanes, in every lane.
extern "C" __device__ __attribute__((const)) float __ockl_wfred_add_f32(float);

// Orders the LDS accesses of one wavefront (its lanes read what other lanes just wrote).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <int TT, bool VEC>
__global__ __launch_bounds__(256, 2) void layer_small_kernel(LayerSmallArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];  // x rows, later h halves
  __shared__ float red[32][TT][kLsEG];
  __shared__ uint64_t cand[TT][4 * kLsMaxSlots];
  __shared__ uint64_t wkey[4][64];                    // per wavefront: its 64 selection keys
  __shared__ uint64_t wsel[4][TT][kLsMaxSlots];      // per wavefront: the selected slots
  __shared__ int slot_e[kLsMaxSlots], slot_cnt[kLsMaxSlots], slot_first[kLsMaxSlots];
  __shared__ int slot_pos[kLsMaxSlots];
  __shared__ float slot_w[kLsMaxSlots];
  __shared__ float act_tsd[kLsMaxSlots];  // down tensor scale of each active expert
  __shared__ int act_e[kLsMaxSlots], act_cnt[kLsMaxSlots], act_off[kLsMaxSlots];
  __shared__ int srow_tok[kLsMaxSlots];
  __shared__ float srow_w[kLsMaxSlots];
  __shared__ float dred[4][TT][16];
  __shared__ float xred[4][kLsXTiles][16];  // per-XCD mode: each wavefront's half-sums per tile
  __shared__ int s_nact, s_flag, s_last;

  LS_STAMP(0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int G = gridDim.x;
  const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k;
  const int nq = T * k;
  // Per-XCD mode (one token, k = 8 slots): group g = blockIdx.x % 8 (the hardware puts those
  // blocks on one XCD; nothing depends on it for correctness) runs slot g's expert alone: its
  // gate/up tiles, a barrier among the group only, its h row, and its down projection over every
  // output feature, split over the group's blocks; block j of every group covers the same range
  // of features, and that range's eighth arrival adds the 8 weighted rows in slot order.
  const int xgs = G / kLsGroups;  // blocks per group
  const bool xm = TT == 1 && k == kLsGroups && G % kLsGroups == 0 && xgs <= kLsXRanges &&
                  (H / 16 + xgs - 1) / xgs <= 2 * kLsXTiles;
  const int xg = blockIdx.x % kLsGroups, xj = blockIdx.x / kLsGroups;
  const uint32_t spin_cfg = a.sync[kLsSyncSpin];  // written by the host before the launch
  const uint32_t spin = spin_cfg != 0 ? spin_cfg : kLsSpin;

  uint16_t* xs = reinterpret_cast<uint16_t*>(dyn);  // x rows (bf16), staged during barrier A

  // ---- A: router partial logits ----
  {
    const int NEG = (E + kLsEG - 1) / kLsEG;
    const int e4 = tid & 7, rp = tid >> 3;  // 4 experts per thread, 32 row phases
    for (int it = blockIdx.x; it < kLsNS * NEG; it += G) {
      const int sl = it / NEG, eg = it - sl * NEG;
      const int r0 = sl * H / kLsNS, r1 = (sl + 1) * H / kLsNS;
      const int eb = eg * kLsEG + e4 * 4;
      float acc[TT][4];
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[t][j] = 0.f;
      for (int rb = r0 + rp; rb < r1; rb += 32 * 8) {
        float w[8][4];
        uint16_t xb[8][TT];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = min(rb + 32 * i, r1 - 1);  // clamped rows multiply nothing (below)
          if (VEC) {
            const float4 v = *reinterpret_cast<const float4*>(a.wr + (size_t)r * E + min(eb, E - 4));
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) w[i][j] = a.wr[(size_t)r * E + min(eb + j, E - 1)];
          }
#pragma unroll
          for (int t = 0; t < TT; ++t) xb[i][t] = a.x[(size_t)min(t, T - 1) * H + r];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = rb + 32 * i;
          if (r < r1) {
#pragma unroll
            for (int t = 0; t < TT; ++t) {
              const float xv = t < T ? bf16_to_f32(xb[i][t]) : 0.f;
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[t][j] = fmaf(xv, w[i][j], acc[t][j]);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[rp][t][e4 * 4 + j] = acc[t][j];
      __syncthreads();
      if (tid < TT * kLsEG) {
        const int t = tid / kLsEG, el = tid - t * kLsEG, e = eg * kLsEG + el;
        float s = 0.f;
#pragma unroll 8
        for (int p = 0; p < 32; ++p) s += red[p][t][el];
        if (t < T && e < E) st_dev(reinterpret_cast<uint32_t*>(a.partial) + ((size_t)sl * T + t) * E + e, __float_as_uint(s));
      }
      __syncthreads();
    }
  }
  LS_STAMP(1);
  ls_arrive(a.sync, kLsSyncA, kLsFlagA, (uint32_t)G);
  // x rows into LDS for the gate/up phase, while barrier A completes
  for (int i = tid; i < T * H / 8; i += 256)
    reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(a.x)[i];

  // ---- gate/up plan, set up while barrier A completes.  Item = (expert, 16-feature tile) per
  // wavefront.  With one token the items follow the token's slots (largest logit first), so
  // that the first weights can be requested as soon as the ranks are known; with two tokens
  // they follow the active list. ----
  const int nch = H / kChunk;  // chunks along the hidden dimension
  const int ntile = I / 16;
  const int W = G * 4, gw = blockIdx.x * 4 + wv;
  const int nspi = (nch + kLsSetC - 1) / kLsSetC;  // load sets per item
  const size_t mq = (size_t)I * H / 2, ms = (size_t)I * H / 16;
  const int* c_e = TT == 1 ? slot_e : act_e;      // item's expert
  const int* c_off = TT == 1 ? slot_pos : act_off;  // item's first row in the grouped order
  int na = 0, n_items = 0, nsets = 0, Wc = W, it_end = 0;
  auto plan = [&](int nact) {
    na = nact;
    n_items = na * ntile;
    it_end = n_items;
    const int my_items = gw < n_items ? (n_items - 1 - gw) / W + 1 : 0;
    nsets = my_items * nspi;
  };
  // per-XCD mode: the group's wavefronts take tiles lw, lw + 4 xgs, ... of slot xg's expert
  const int xlw = xj * 4 + wv;
  auto plan_xcd = [&]() {
    na = k;
    n_items = k * ntile;
    Wc = 4 * xgs;
    it_end = (xg + 1) * ntile;
    const int my_items = xlw < ntile ? (ntile - 1 - xlw) / Wc + 1 : 0;
    nsets = my_items * nspi;
  };
  // A cursor walks the wavefront's load sets: set j of item it = gw + m W (item-list index ai,
  // 16-feature tile rt).  Past the last set it stays there (loads re-read it, unused).
  struct Cur {
    int j, it, ai, rt;
  };
  auto cur_item = [&](Cur& c, int it) {
    c.j = 0;
    c.it = it;
    c.ai = it / ntile;
    c.rt = it - c.ai * ntile;
  };
  auto cur_next = [&](Cur& c) {
    if (c.j + 1 < nspi) {
      ++c.j;
    } else if (c.it + Wc < it_end) {
      cur_item(c, c.it + Wc);
    }
  };
  uint4 qgA[kLsSetC], quA[kLsSetC], qgB[kLsSetC], quB[kLsSetC];
  uint32_t sgA[kLsSetC], suA[kLsSetC], sgB[kLsSetC], suB[kLsSetC];
  auto load_set = [&](uint4* qg, uint4* qu, uint32_t* sg, uint32_t* su, const Cur& c, int e) {
    const int cs = c.j * kLsSetC;
    const size_t tq = (size_t)e * mq + ((size_t)c.rt * nch) * 1024 + lane * 16;
    const size_t ts_ = (size_t)e * ms + ((size_t)c.rt * nch) * 128 + (lane >> 1) * 4;
#pragma unroll
    for (int u = 0; u < kLsSetC; ++u) {
      const int ch = min(cs + u, nch - 1);
      qg[u] = load_stream16(a.gq + tq + (size_t)ch * 1024);
      qu[u] = load_stream16(a.uq + tq + (size_t)ch * 1024);
      sg[u] = load_scale_dword(a.gs + ts_ + (size_t)ch * 128);
      su[u] = load_scale_dword(a.us + ts_ + (size_t)ch * 128);
    }
  };
  Cur lc, uc;
  if constexpr (TT == 1) {
    if (xm) {
      plan_xcd();
      cur_item(lc, xg * ntile + xlw);
    } else {
      plan(k);  // one token: k distinct experts
      cur_item(lc, gw);
    }
    uc = lc;
  }

  // Per-XCD mode: range xj of the output tiles, [xt0, xt1).
  const int xtpb = (H / 16 + xgs - 1) / xgs;
  const int xt0 = min(xj * xtpb, H / 16), xt1 = min(xt0 + xtpb, H / 16);
  // Per-XCD mode, the end of every block, also of one that gave up: once its row of the partial
  // buffer is complete, it arrives at range xj's counter; the range's eighth arrival adds the 8
  // rows in slot order, writes out and counts the range as done, and the arrival that completes
  // the last range resets the counters and flags.  A block arrives there after its last wait and
  // after its flag stores are complete, so no exit barrier is needed.
  auto xm_finish = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    lds_barrier();
    if (tid == 0)
      s_last = __hip_atomic_fetch_add(ls_xr_ctr(a.sync, xj), 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == kLsGroups - 1;
    lds_barrier();
    LS_STAMP(14);
    if (s_last) {
      uint32_t done = 0;
      if (tid == 0)
        done = __hip_atomic_fetch_add(ls_xdone(a.sync), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t* xa = reinterpret_cast<const uint32_t*>(a.xpart);
      for (int f = xt0 * 16 + tid; f < xt1 * 16; f += 256) {
        float sum = 0.f;
#pragma unroll
        for (int gg = 0; gg < kLsGroups; ++gg) sum += __uint_as_float(ld_dev(xa + (size_t)gg * H + f));
        a.out[f] = sum;
      }
      if (tid == 0 && done == (uint32_t)xgs - 1) ls_reset(a.sync);
    }
  };
  // Per-XCD mode, a block that gave up: NaN over its row of the partial buffer in range xj, so
  // that the range's sum is NaN.
  auto xm_fail_part = [&]() {
    for (int f = xt0 * 16 + tid; f < xt1 * 16; f += 256)
      st_dev(reinterpret_cast<uint32_t*>(a.xpart) + (size_t)xg * H + f, 0x7fc00000u);
  };

  // ---- B: logits, top-k, softmax, grouping (every block) ----
  if (!ls_wait(a.sync, kLsFlagA, &s_flag, spin)) {
    if (xm) {
      // NaN over this block's gate/up features in every row of h (the rows' order is not known),
      // so that every block of the group computes NaN; then its arrivals at barrier C and at its
      // range, as if it had finished
      for (int rt = xlw; rt < ntile; rt += Wc)
        for (int r = g; r < k; r += 4)
          if ((n & 1) == 0) st_dev(a.h + ((size_t)r * I + rt * 16 + n) / 2, 0x7e007e00u);
      ls_arrive_group(a.sync, xg, (uint32_t)xgs);
      xm_fail_part();
      xm_finish();
      return;
    }
    ls_fail_out(a, G);
    ls_exit(a.sync, (uint32_t)G);
    return;
  }
  LS_STAMP(2);
  // logits of expert e = tid (slices added in order), kept in registers
  float lg[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    lg[t] = -__builtin_inff();
    if (tid < E) {
      float v[kLsNS];
#pragma unroll
      for (int sl = 0; sl < kLsNS; ++sl)
        v[sl] = __uint_as_float(ld_dev(reinterpret_cast<const uint32_t*>(a.partial) + ((size_t)sl * T + t) * E + tid));
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < kLsNS; ++sl) sum += v[sl];
      if (a.bias) sum += a.bias[tid];
      if (blockIdx.x == 0 && a.logits) a.logits[(size_t)t * E + tid] = sum;
      lg[t] = sum;
    }
  }
  LS_STAMP(8);
  // top-k in two levels, by rank: an expert's rank is the number of experts with a larger
  // selection key (a larger logit, or an equal logit and a lower id).  Each lane first ranks
  // its expert among the 64 of its wavefront; those of rank < k are the candidates (the overall
  // top k are among them).  Then every wavefront (redundantly, so that no second barrier is
  // needed) ranks the 4k candidates among each other.  All comparisons are independent, so the
  // wavefront issues them back to back.
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const uint64_t key = tid < E ? sel_key(lg[t], tid) : 0;
    wkey[wv][lane] = key;
    if (lane < k) cand[t][wv * k + lane] = 0;
    wave_lds_sync();
    int rank = 0;
    const uint4* kp = reinterpret_cast<const uint4*>(wkey[wv]);
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const uint4 v = kp[j];
      rank += (((uint64_t)v.y << 32) | v.x) > key;
      rank += (((uint64_t)v.w << 32) | v.z) > key;
    }
    if (key != 0 && rank < k) cand[t][wv * k + rank] = key;
    wave_lds_sync();
  }
  lds_barrier();
  LS_STAMP(9);
  // candidate keys (two per lane) and their ranks among the candidates
  uint64_t cc0[TT], cc1[TT];
  int rr0[TT], rr1[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int nc = 4 * k;
    cc0[t] = lane < nc ? cand[t][lane] : 0;
    cc1[t] = lane + 64 < nc ? cand[t][lane + 64] : 0;
    int r0 = 0, r1 = 0;
    const uint4* cp = reinterpret_cast<const uint4*>(cand[t]);
    for (int j = 0; j < nc / 2; ++j) {  // nc is even
      const uint4 v = cp[j];
      const uint64_t v0 = ((uint64_t)v.y << 32) | v.x, v1 = ((uint64_t)v.w << 32) | v.z;
      r0 += (v0 > cc0[t]) + (v1 > cc0[t]);
      r1 += (v0 > cc1[t]) + (v1 > cc1[t]);
    }
    rr0[t] = r0;
    rr1[t] = r1;
  }
  LS_STAMP(10);
  if constexpr (TT == 1) {
    // the first two gate/up load sets are requested now: the expert of slot r is the candidate
    // of rank r
    auto slot_expert = [&](int r) {
      const uint64_t m0 = __ballot(cc0[0] != 0 && rr0[0] == r);
      const uint64_t m1 = __ballot(cc1[0] != 0 && rr1[0] == r);
      const int i0 = __builtin_amdgcn_readlane(sel_id(cc0[0]) , m0 ? (int)__builtin_ctzll(m0) : 0);
      const int i1 = __builtin_amdgcn_readlane(sel_id(cc1[0]), m1 ? (int)__builtin_ctzll(m1) : 0);
      return m0 ? i0 : (m1 ? i1 : 0);
    };
    if (nsets > 0) {
      load_set(qgA, quA, sgA, suA, lc, slot_expert(lc.ai));
      cur_next(lc);
      load_set(qgB, quB, sgB, suB, lc, slot_expert(lc.ai));
      cur_next(lc);
    }
    LS_STAMP(11);
  }
  // each token's slots into lanes (lane r < k: slot r), through this wavefront's LDS
  uint64_t sk[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (lane < k) wsel[wv][t][lane] = 0;
    wave_lds_sync();
    if (cc0[t] != 0 && rr0[t] < k) wsel[wv][t][rr0[t]] = cc0[t];
    if (cc1[t] != 0 && rr1[t] < k) wsel[wv][t][rr1[t]] = cc1[t];
    wave_lds_sync();
    sk[t] = lane < k ? wsel[wv][t][lane] : 0;
  }
  // softmax over each token's k selected logits (lanes r < k)
  float sw[TT];
  int se[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const float l = sel_value(sk[t]);
    const float l0 = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(l)));  // slot 0
    const float ex = lane < k ? expf(l - l0) : 0.f;
    sw[t] = ex / __ockl_wfred_add_f32(ex);
    se[t] = lane < k ? sel_id(sk[t]) : 0;
  }
  if constexpr (TT == 1) {
    // one token: its k experts are distinct, each with one row; the grouped order (and the
    // active order: count descending, id ascending) is expert id ascending
    int pos = 0;  // lane r < k: position of slot r in the grouped order
    const uint4* sp = reinterpret_cast<const uint4*>(wsel[wv][0]);
    for (int j = 0; j < (k + 1) / 2; ++j) {
      const uint4 v = sp[j];
      pos += (2 * j < k) & (sel_id(((uint64_t)v.y << 32) | v.x) < se[0]);
      pos += (2 * j + 1 < k) & (sel_id(((uint64_t)v.w << 32) | v.z) < se[0]);
    }
    if (wv == 0 && lane < k) {
      slot_e[lane] = se[0];
      slot_pos[lane] = pos;
      act_e[pos] = se[0];
      act_cnt[pos] = 1;
      act_off[pos] = pos;
      srow_tok[pos] = 0;
      srow_w[pos] = sw[0];
      if (blockIdx.x == 0) {
        a.topk_id[lane] = se[0];
        a.topk_w[lane] = sw[0];
        a.sorted_slot[pos] = lane;
        a.slot_row[lane] = pos;
      }
    }
    if (blockIdx.x == 0) {
      for (int e = tid; e < E; e += 256) {
        int c = 0, o = 0, act = -1;
        for (int r = 0; r < k; ++r) {
          const int er = __builtin_amdgcn_readlane(se[0], r);
          c += er == e;
          o += er < e;
          if (__builtin_amdgcn_readlane(pos, r) == e) act = er;
        }
        a.count[e] = c;
        a.offset[e] = o;
        a.active[e] = act;
      }
      if (tid == 0) {
        a.offset[E] = k;
        *a.n_active = k;
      }
    }
    lds_barrier();
  } else {
    if (wv == 0 && lane < k) {
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t < T) {
          slot_e[t * k + lane] = se[t];
          slot_w[t * k + lane] = sw[t];
          if (blockIdx.x == 0) {
            a.topk_id[t * k + lane] = se[t];
            a.topk_w[t * k + lane] = sw[t];
          }
        }
      }
    }
    __syncthreads();
    if (tid < nq) {
      // stable counting sort of the slots by expert: position = slots of smaller experts + earlier
      // slots of the same expert
      const int e = slot_e[tid];
      int cnt = 0, r = 0, off = 0;
      for (int q = 0; q < nq; ++q) {
        const int eq = slot_e[q];
        cnt += eq == e;
        r += (eq == e) & (q < tid);
        off += eq < e;
      }
      const int pos = off + r;
      slot_cnt[tid] = cnt;
      slot_first[tid] = r == 0;
      slot_pos[tid] = pos;
      srow_tok[pos] = tid / k;
      srow_w[pos] = slot_w[tid];
      if (blockIdx.x == 0) {
        a.sorted_slot[pos] = tid;
        a.slot_row[tid] = pos;
      }
    }
    __syncthreads();
    if (tid < nq && slot_first[tid]) {
      // active order: count descending, then expert id ascending
      const int e = slot_e[tid], cnt = slot_cnt[tid];
      int ar = 0;
      for (int q = 0; q < nq; ++q) {
        if (slot_first[q]) {
          const int c2 = slot_cnt[q], e2 = slot_e[q];
          ar += (c2 > cnt) | ((c2 == cnt) & (e2 < e));
        }
      }
      act_e[ar] = e;
      act_cnt[ar] = cnt;
      act_off[ar] = slot_pos[tid];
    }
    if (tid == 0) {
      int nact = 0;
      for (int q = 0; q < nq; ++q) nact += slot_first[q];
      s_nact = nact;
    }
    __syncthreads();
    plan(s_nact);
    if (blockIdx.x == 0) {
      for (int e = tid; e < E; e += 256) {
        int c = 0, o = 0;
        for (int q = 0; q < nq; ++q) {
          c += slot_e[q] == e;
          o += slot_e[q] < e;
        }
        a.count[e] = c;
        a.offset[e] = o;
        a.active[e] = e < na ? act_e[e] : -1;
      }
      if (tid == 0) {
        a.offset[E] = nq;
        *a.n_active = na;
      }
    }
    cur_item(lc, gw);
    uc = lc;
    if (nsets > 0) {
      load_set(qgA, quA, sgA, suA, lc, act_e[lc.ai]);
      cur_next(lc);
      load_set(qgB, quB, sgB, suB, lc, act_e[lc.ai]);
      cur_next(lc);
    }
  }

  LS_STAMP(3);
  // ---- C: gate/up + SwiGLU; rows of h (f16) go out with device-scope stores ----
  {
    // per-XCD mode: the one expert's tensor scales, read before the loop (a load in the item's
    // epilogue would wait for every weight load in flight)
    float tsg_x = 0.f, tsu_x = 0.f;
    if (xm) {
      tsg_x = a.ts[slot_e[xg] * 3 + 0];
      tsu_x = a.ts[slot_e[xg] * 3 + 1];
    }
    float ag[TT], au[TT];
#pragma unroll
    for (int r = 0; r < TT; ++r) ag[r] = au[r] = 0.f;
    auto use_set = [&](const uint4* qg, const uint4* qu, const uint32_t* sg, const uint32_t* su,
                       const Cur& cu) {
      const int ai = cu.ai, rt = cu.rt;
      const int rows = TT == 1 ? 1 : act_cnt[ai], off = c_off[ai];
      const int cs = cu.j * kLsSetC;
#pragma unroll
      for (int u = 0; u < kLsSetC; ++u) {
        const int c = cs + u;
        if (c < nch) {
          Dec32bf dg, du;  // decoded once, dotted with every row
          decode32(qg[u], scale_pair(sg[u], lane), dg);
          decode32(qu[u], scale_pair(su[u], lane), du);
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            if (r < rows) {
              const uint4* xv = reinterpret_cast<const uint4*>(
                  xs + (size_t)srow_tok[off + r] * H + c * kChunk + g * 32);
              ag[r] += dot32(dg, xv);
              au[r] += dot32(du, xv);
            }
          }
        }
      }
      if (cu.j == nspi - 1) {  // the item's last set: SwiGLU and store two features per lane
        const int e = c_e[ai];
        const float tsg = xm ? tsg_x : a.ts[e * 3 + 0], tsu = xm ? tsu_x : a.ts[e * 3 + 1];
#pragma unroll
        for (int r = 0; r < TT; ++r) {
          if (r < rows) {
            const float gv = sum_groups(ag[r]) * tsg, uv = sum_groups(au[r]) * tsu;
            const _Float16 hv = (_Float16)(gv / (1.0f + expf(-gv)) * uv);
            const uint32_t bits = __builtin_bit_cast(uint16_t, hv);
            const uint32_t nb = __shfl_down(bits, 1);
            if (g == 0 && (n & 1) == 0)
              st_dev(a.h + ((size_t)(off + r) * I + rt * 16 + n) / 2, bits | (nb << 16));
          }
          ag[r] = au[r] = 0.f;
        }
      }
    };

    // two load sets in flight: set s + 1 is requested before set s is used.  The loop runs while
    // two more sets exist and the tail takes the last one or two, so that no set past the end is
    // requested: its loads would be waited for at the barrier arrival, a full memory latency
    if (nsets > 0) {
      use_set(qgA, quA, sgA, suA, uc);
      cur_next(uc);
      if (2 < nsets) {
        load_set(qgA, quA, sgA, suA, lc, c_e[lc.ai]);
        cur_next(lc);
      }
      if (1 < nsets) {
        use_set(qgB, quB, sgB, suB, uc);
        cur_next(uc);
      }
      int s = 2;
      for (; s + 2 < nsets; s += 2) {  // sets s (in A), s + 1 and s + 2 exist
        load_set(qgB, quB, sgB, suB, lc, c_e[lc.ai]);
        cur_next(lc);
        use_set(qgA, quA, sgA, suA, uc);
        cur_next(uc);
        load_set(qgA, quA, sgA, suA, lc, c_e[lc.ai]);
        cur_next(lc);
        use_set(qgB, quB, sgB, suB, uc);
        cur_next(uc);
      }
      if (s + 1 < nsets) {  // the last two sets
        load_set(qgB, quB, sgB, suB, lc, c_e[lc.ai]);
        cur_next(lc);
        use_set(qgA, quA, sgA, suA, uc);
        cur_next(uc);
        use_set(qgB, quB, sgB, suB, uc);
        cur_next(uc);
      } else if (s < nsets) {  // the last set
        use_set(qgA, quA, sgA, suA, uc);
        cur_next(uc);
      }
    }
  }
  LS_STAMP(4);
  // the down phase's tensor scales, read here: a load inside its loop would wait for every
  // weight load in flight before it
  if (!xm && tid < na) act_tsd[tid] = a.ts[act_e[tid] * 3 + 2];
  if (xm)
    ls_arrive_group(a.sync, xg, (uint32_t)xgs);
  else
    ls_arrive(a.sync, kLsSyncC, kLsFlagC, (uint32_t)G);

  // ---- D: down + combine ----
  if (xm) {
    // per-XCD mode: slot xg's down projection over the output tiles [t0, t1) of range xj.  A
    // wavefront takes the tiles t0 + par + 2 m (par = wv / 2) over one half of I (kh = wv % 2);
    // each tile's load set is its 8 chunks of 1 KB along I.
    const int nci = I / kChunk;
    const int kh = wv & 1, par = wv >> 1;
    const int cbeg = kh * nci / 2, nck = (kh + 1) * nci / 2 - cbeg;  // this half's chunks
    const int hw_row = ((nci + 1) / 2) * (kChunk / 2);                 // LDS words per h row
    const int t0 = xt0, t1 = xt1;
    const int nmine = t1 - t0 > par ? (t1 - t0 - par + 1) / 2 : 0;
    const int nspe = (nck + kLsSetD - 1) / kLsSetD;  // load sets per tile
    const int nsets = nmine * nspe;
    const int e = slot_e[xg], hrow = slot_pos[xg];
    const float wgt = srow_w[hrow], tsd = a.ts[e * 3 + 2];
    const size_t mq = (size_t)H * I / 2, ms = (size_t)H * I / 16;
    uint4 qA[kLsSetD], qB[kLsSetD];
    uint32_t sA[kLsSetD], sB[kLsSetD];
    auto load_set = [&](uint4* q, uint32_t* sc, int s) {
      s = min(s, nsets - 1);  // past the end: re-read the last set (unused)
      const int m = s / nspe, cs = (s % nspe) * kLsSetD;
      const int ft = t0 + par + 2 * m;
      const size_t tq = (size_t)e * mq + ((size_t)ft * nci + cbeg) * 1024 + lane * 16;
      const size_t ts_ = (size_t)e * ms + ((size_t)ft * nci + cbeg) * 128 + (lane >> 1) * 4;
#pragma unroll
      for (int u = 0; u < kLsSetD; ++u) {
        const int c = min(cs + u, nck - 1);
        q[u] = load_stream16(a.dq + tq + (size_t)c * 1024);
        sc[u] = load_scale_dword(a.ds + ts_ + (size_t)c * 128);
      }
    };
    const bool has_k = nck > 0 && nsets > 0;
    if (has_k && wv != 0) load_set(qA, sA, 0);
    if (!ls_wait_at(a.sync, ls_xc_flag(a.sync, xg), &s_flag, spin)) {
      xm_fail_part();
      xm_finish();
      return;
    }
    LS_STAMP(5);
    // slot xg's h row, both halves: LDS [half][hw_row words], device-scope 64-bit loads
    uint32_t* hs0 = dyn;
    const int rq = I / 8;  // 16-byte pieces of the row
    for (int i = tid; i < rq; i += 256) {
      const int half = i >= (nci / 2) * (kChunk / 8) ? 1 : 0;
      const int pl = i - half * (nci / 2) * (kChunk / 8);
      const uint64_t* src = reinterpret_cast<const uint64_t*>(a.h) + 2 * ((size_t)hrow * rq + i);
      const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *reinterpret_cast<uint4*>(hs0 + (size_t)half * hw_row + pl * 4) =
          make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
    }
    if (has_k && wv == 0) load_set(qA, sA, 0);
    lds_barrier();
    LS_STAMP(6);
    const uint32_t* hs = dyn;
    float racc = 0.f;
    if (g == 0)  // a half with no chunks (I = 128) adds zero
#pragma unroll
      for (int m = 0; m < kLsXTiles; ++m) xred[wv][m][n] = 0.f;
    auto use_set = [&](const uint4* q, const uint32_t* sc, int s) {
      const int m = s / nspe, cs = (s % nspe) * kLsSetD;
#pragma unroll
      for (int u = 0; u < kLsSetD; ++u) {
        const int c = cs + u;
        if (c < nck) {
          Dec32h d;
          decode32(q[u], scale_pair(sc[u], lane), d);
          racc += dot32(d, reinterpret_cast<const uint4*>(hs + (size_t)kh * hw_row + c * (kChunk / 2) + g * 16));
        }
      }
      if (s % nspe == nspe - 1) {  // the tile's last set: this half's weighted sum
        const float y = sum_groups(racc) * tsd;
        if (g == 0) xred[wv][m][n] = wgt * y;
        racc = 0.f;
      }
    };
    if (has_k) {  // the loop runs while two more sets exist; the tail requests nothing past the end
      int s = 0;
      for (; s + 2 < nsets; s += 2) {
        load_set(qB, sB, s + 1);
        use_set(qA, sA, s);
        if (s == 0) LS_STAMP(12);
        load_set(qA, sA, s + 2);
        use_set(qB, sB, s + 1);
      }
      if (s + 1 < nsets) {
        load_set(qB, sB, s + 1);
        use_set(qA, sA, s);
        use_set(qB, sB, s + 1);
      } else {
        use_set(qA, sA, s);
      }
    }
    LS_STAMP(13);
    lds_barrier();
    // the two halves of each tile, added in order, into the group's row of the partial buffer
    float* xp = a.xpart + (size_t)xg * H;
    if (kh == 0 && g == 0)
      for (int m = 0; m < nmine; ++m)
        st_dev(reinterpret_cast<uint32_t*>(xp) + (t0 + par + 2 * m) * 16 + n,
               __float_as_uint(xred[wv][m][n] + xred[wv + 1][m][n]));
    LS_STAMP(7);
    xm_finish();
    return;
  } else {
    const int nci = I / kChunk;
    const int kh = wv & 1, ftl = wv >> 1;
    const int cbeg = kh * nci / 2, nck = (kh + 1) * nci / 2 - cbeg;  // this half's chunks
    const int hw_row = ((nci + 1) / 2) * (kChunk / 2);                 // LDS words per h row
    const int nspe = (nck + kLsSetD - 1) / kLsSetD;  // load sets per expert
    const int nsets = na * nspe;
    const int npairs = H / 32;
    const size_t mq = (size_t)H * I / 2, ms = (size_t)H * I / 16;
    uint4 qA[kLsSetD], qB[kLsSetD];
    uint32_t sA[kLsSetD], sB[kLsSetD];
    int ftp = blockIdx.x;
    auto load_set = [&](uint4* q, uint32_t* sc, int s) {
      s = min(s, nsets - 1);  // past the end: re-read the last set (unused)
      const int ai = s / nspe, cs = (s % nspe) * kLsSetD;
      const int e = act_e[ai];
      const int ft = ftp * 2 + ftl;
      const size_t tq = (size_t)e * mq + ((size_t)ft * nci + cbeg) * 1024 + lane * 16;
      const size_t ts_ = (size_t)e * ms + ((size_t)ft * nci + cbeg) * 128 + (lane >> 1) * 4;
#pragma unroll
      for (int u = 0; u < kLsSetD; ++u) {
        const int c = min(cs + u, nck - 1);
        q[u] = load_stream16(a.dq + tq + (size_t)c * 1024);
        sc[u] = load_scale_dword(a.ds + ts_ + (size_t)c * 128);
      }
    };
    const bool has_k = nck > 0;
    bool exited = false;
    // a block with no output tile neither waits nor stages h
    if (ftp < npairs) {
      // the first weights are requested before waiting for h (not by the polling wavefront,
      // whose poll would queue behind them)
      if (has_k && wv != 0) load_set(qA, sA, 0);
      if (!ls_wait(a.sync, kLsFlagC, &s_flag, spin)) {
        ls_fail_out(a, G);
        ls_exit(a.sync, (uint32_t)G);
        return;
      }
      LS_STAMP(5);
      // the block's last wait is over and its flag stores are complete: it arrives at the exit
      // barrier now, so that the reset overlaps the down phase instead of following it
      ls_exit(a.sync, (uint32_t)G);
      exited = true;
      if (has_k && wv == 0) load_set(qA, sA, 0);
      // both halves of every h row: LDS [half][row][hw_row words], read with device-scope
      // 64-bit loads (the rows were written by other blocks)
      uint32_t* hs0 = dyn;
      const int rq = I / 8;  // 16-byte pieces per h row
      for (int i = tid; i < nq * rq; i += 256) {
        const int p = i / rq, pc = i - p * rq;
        const int half = pc >= (nci / 2) * (kChunk / 8) ? 1 : 0;
        const int pl = pc - half * (nci / 2) * (kChunk / 8);
        const uint64_t* src = reinterpret_cast<const uint64_t*>(a.h) + 2 * (size_t)i;
        const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *reinterpret_cast<uint4*>(hs0 + ((size_t)half * nq + p) * hw_row + pl * 4) =
            make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32));
      }
      lds_barrier();
      LS_STAMP(6);
    }
    const uint32_t* hs = dyn;
    for (; ftp < npairs; ftp += G) {
      float acc_t[TT], racc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) acc_t[t] = racc[t] = 0.f;
      auto use_set = [&](const uint4* q, const uint32_t* sc, int s) {
        const int ai = s / nspe, cs = (s % nspe) * kLsSetD;
        const int rows = act_cnt[ai], off = act_off[ai];
#pragma unroll
        for (int u = 0; u < kLsSetD; ++u) {
          const int c = cs + u;
          if (c < nck) {
            Dec32h d;  // decoded once, dotted with every row
            decode32(q[u], scale_pair(sc[u], lane), d);
#pragma unroll
            for (int r = 0; r < TT; ++r) {
              if (r < rows) {
                const uint4* hv = reinterpret_cast<const uint4*>(
                    hs + ((size_t)kh * nq + off + r) * hw_row + c * (kChunk / 2) + g * 16);
                racc[r] += dot32(d, hv);
              }
            }
          }
        }
        if (s % nspe == nspe - 1) {  // the expert's last set: weight its rows into the tokens
          const float tsd = act_tsd[ai];
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            if (r < rows) {
              const float y = sum_groups(racc[r]) * tsd;
              const int tok = srow_tok[off + r];
              const float w = srow_w[off + r];
#pragma unroll
              for (int t = 0; t < TT; ++t)
                if (t == tok) acc_t[t] = fmaf(w, y, acc_t[t]);
            }
            racc[r] = 0.f;
          }
        }
      };
      if (has_k) {  // the loop runs while two more sets exist; the tail requests nothing past the end
        if (ftp != (int)blockIdx.x) load_set(qA, sA, 0);
        int s = 0;
        for (; s + 2 < nsets; s += 2) {
          load_set(qB, sB, s + 1);
          use_set(qA, sA, s);
          load_set(qA, sA, s + 2);
          use_set(qB, sB, s + 1);
        }
        if (s + 1 < nsets) {
          load_set(qB, sB, s + 1);
          use_set(qA, sA, s);
          use_set(qB, sB, s + 1);
        } else {
          use_set(qA, sA, s);
        }
      }
      // add the two halves of each feature in LDS, in order
      if (g == 0)
#pragma unroll
        for (int t = 0; t < TT; ++t) dred[wv][t][n] = acc_t[t];
      lds_barrier();
      if (kh == 0 && g == 0) {
        const int f = (ftp * 2 + ftl) * 16 + n;
#pragma unroll
        for (int t = 0; t < TT; ++t)
          if (t < T) a.out[(size_t)t * H + f] = dred[wv][t][n] + dred[wv + 1][t][n];
      }
      lds_barrier();
    }
    // ---- exit: a block that has not arrived at the exit barrier yet (no output tile) ----
    LS_STAMP(7);
    if (!exited) ls_exit(a.sync, (uint32_t)G);
  }
}

size_t layer_small_lds(int T, int H, int I, int k) {
  const size_t xb = (size_t)T * H * 2;
  const size_t hw_row = (size_t)((I / kChunk + 1) / 2) * (kChunk / 2);
  const size_t hb = 2 * (size_t)T * k * hw_row * 4;
  return xb > hb ? xb : hb;
}

bool layer_small_fits(int T, int H, int I, int E, int k) {
  (void)E;
  return T >= 1 && T <= 2 && T * k <= kLsMaxSlots && layer_small_lds(T, H, I, k) <= 65536;
}

// Blocks of the single-launch kernel on this device: one per CU, provided that at least one
// block fits per CU (every block must be resident); 0 if not.  The answer depends only on the
// device and the kernel's LDS size, so it is computed once per (device, kernel, LDS size) and
// cached for the life of the process.
static int layer_small_grid(int T, bool vec, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int var = (T == 1 ? 0 : 2) + (vec ? 1 : 0);
  struct Entry {
    size_t lds;
    int grid;
  };
  static std::mutex mu;
  static Entry cache[64][4][4];  // [device][kernel][slot]: a few LDS sizes per kernel
  static int next[64][4];
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& c : cache[dev][var])
      if (c.grid > 0 && c.lds == lds) return c.grid;
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int occ = 0;
  const void* f = T == 1 ? (vec ? (const void*)layer_small_kernel<1, true>
                                : (const void*)layer_small_kernel<1, false>)
                         : (vec ? (const void*)layer_small_kernel<2, true>
                                : (const void*)layer_small_kernel<2, false>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, 256, lds) != hipSuccess) return 0;
  const int grid = occ >= 1 ? ncu : 0;
  if (grid > 0) {
    std::lock_guard<std::mutex> lock(mu);
    cache[dev][var][next[dev][var]++ % 4] = Entry{lds, grid};
  }
  return grid;
}

hipError_t launch_layer_small(const LayerSmallArgs& a, hipStream_t s) {
  const size_t lds = layer_small_lds(a.T, a.H, a.I, a.k);
  const bool vec = (a.E & 3) == 0;
  const int grid = layer_small_grid(a.T, vec, lds);
  if (grid == 0) return hipErrorInvalidConfiguration;
  if (a.T == 1) {
    if (vec) layer_small_kernel<1, true><<<grid, 256, lds, s>>>(a);
    else layer_small_kernel<1, false><<<grid, 256, lds, s>>>(a);
  } else {
    if (vec) layer_small_kernel<2, true><<<grid, 256, lds, s>>>(a);
    else layer_small_kernel<2, false><<<grid, 256, lds, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_TIMELINE
extern "C" __attribute__((visibility("default"))) int moe_timeline_layer_small(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(moe::g_ls_timeline), sizeof(moe::g_ls_timeline),
                                  0, hipMemcpyDeviceToHost);
}
#endif
