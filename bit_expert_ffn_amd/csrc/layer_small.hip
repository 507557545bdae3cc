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
//   Exit: counter X; the last block to arrive resets the counters and flags for the next call.
// A barrier: every block adds one to the barrier's counter; the block that completes it raises
// 16 copies of a flag, and each block polls its own copy.
// Data that crosses blocks (partial logits, h) is written with device-scope stores, which write
// through the per-XCD L2s (not coherent with each other) to memory, and the counters are relaxed
// device-scope atomics issued after a full s_waitcnt, so no cache-wide release or acquire is
// needed.  The readers use plain cached loads: every kernel starts with invalidated caches and
// no block reads those lines before the counter says they are complete, so the first read on
// each XCD fetches them from memory and the other blocks of the XCD hit its L2.  Every wait is
// bounded: on a timeout the block sets the error word and returns.
#include "common.h"
#include "dot.h"

namespace moe {

constexpr int kLsNS = 32;                 // router: slices of the hidden dimension
constexpr int kLsEG = 32;                 // router: experts per item
constexpr int kLsSetC = 4;                // gate/up: chunks per load set
constexpr int kLsSetD = 8;                // down: chunks per load set
constexpr uint32_t kLsSpin = 1u << 21;    // polls before a wait gives up (about 2 s)
// Sync region (kSyncBytes at the start of the workspace), in 32-bit words: arrival counters A,
// C, X and the error word, 64 bytes apart; then kLsFlags copies of the "all arrived" flags of
// barriers A and C, 4 KB apart so that the pollers of different copies hit different memory
// channels.
constexpr int kLsSyncA = 0, kLsSyncC = 16, kLsSyncX = 32, kLsSyncErr = 48;
constexpr int kLsFlags = 16, kLsFlagBase = 64, kLsFlagStride = 1024;
constexpr int kLsFlagA = 0, kLsFlagC = 16;
static_assert((kLsFlagBase + (kLsFlags - 1) * kLsFlagStride + kLsFlagC + 1) * 4 <= kSyncBytes,
              "flags must fit in the sync region");

__device__ inline uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every earlier store of this block is complete, then thread 0 adds one to the counter; the
// block that brings it to G raises every copy of the barrier's flag.
__device__ inline void ls_arrive(uint32_t* sync, int ctr, int flag, uint32_t G) {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  lds_barrier();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(sync + ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1)
      for (int i = 0; i < kLsFlags; ++i) st_dev(sync + kLsFlagBase + i * kLsFlagStride + flag, 1u);
  }
}

// Thread 0 polls this block's copy of the flag; the other wavefronts wait at an LDS-only
// barrier, keeping their own loads in flight.  false (for every thread) after a timeout.
__device__ inline bool ls_wait(uint32_t* sync, int flag, int* s_ok) {
  if (threadIdx.x == 0) {
    const uint32_t* f = sync + kLsFlagBase + (blockIdx.x % kLsFlags) * kLsFlagStride + flag;
    uint32_t spins = 0;
    int ok = 1;
    while (ld_dev(f) == 0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins > kLsSpin) {
        ok = 0;
        __hip_atomic_fetch_or(sync + kLsSyncErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    *s_ok = ok;
  }
  lds_barrier();
  const bool ok = *s_ok != 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return ok;
}

template <int TT, bool VEC>
__global__ __launch_bounds__(256, 2) void layer_small_kernel(LayerSmallArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];  // x rows, later h halves
  __shared__ float red[32][TT][kLsEG];
  __shared__ __attribute__((aligned(16))) float lv[TT][kMaxExperts];
  __shared__ float2 cand[TT][4 * kLsMaxSlots];
  __shared__ int sel_e[kLsMaxSlots];
  __shared__ float sel_l[kLsMaxSlots];
  __shared__ int slot_e[kLsMaxSlots], slot_cnt[kLsMaxSlots], slot_first[kLsMaxSlots];
  __shared__ int slot_pos[kLsMaxSlots];
  __shared__ float slot_w[kLsMaxSlots];
  __shared__ int act_e[kLsMaxSlots], act_cnt[kLsMaxSlots], act_off[kLsMaxSlots];
  __shared__ int srow_tok[kLsMaxSlots];
  __shared__ float srow_w[kLsMaxSlots];
  __shared__ float dred[4][TT][16];
  __shared__ int s_nact, s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int G = gridDim.x;
  const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k;
  const int nq = T * k;

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
  ls_arrive(a.sync, kLsSyncA, kLsFlagA, (uint32_t)G);
  // x rows into LDS for the gate/up phase, while barrier A completes
  for (int i = tid; i < T * H / 8; i += 256)
    reinterpret_cast<uint4*>(xs)[i] = reinterpret_cast<const uint4*>(a.x)[i];

  // ---- B: logits, top-k, softmax, grouping (every block) ----
  if (!ls_wait(a.sync, kLsFlagA, &s_flag)) return;
  {
    const int e = tid;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= T) break;
      if (e < E) {
        float v[kLsNS];
#pragma unroll
        for (int sl = 0; sl < kLsNS; ++sl)
          v[sl] = a.partial[((size_t)sl * T + t) * E + e];
        float s = 0.f;
#pragma unroll
        for (int sl = 0; sl < kLsNS; ++sl) s += v[sl];
        if (a.bias) s += a.bias[e];
        if (blockIdx.x == 0 && a.logits) a.logits[(size_t)t * E + e] = s;
        lv[t][e] = s;
      } else {
        lv[t][e] = -__builtin_inff();  // never larger than a real logit
      }
    }
  }
  __syncthreads();
  // top-k in two levels.  An expert's rank is the number of experts with a larger logit plus
  // those with an equal logit and a lower id.  Each wavefront first ranks its 64 experts among
  // themselves; those of local rank < k are the candidates (the overall top k are among them),
  // and the 4k candidates are then ranked among each other.
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t >= T) break;
    const float le = lv[t][tid];
    const f32x4* lp = reinterpret_cast<const f32x4*>(&lv[t][wv * 64]);
    int rl = 0;
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const f32x4 v = lp[j];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        rl += (v[c] > le) | ((v[c] == le) & (wv * 64 + 4 * j + c < tid));
    }
    // candidates as (logit, id) pairs; missing ones (fewer than k experts in the wavefront)
    // are (-inf, INT_MAX), which never count as larger
    if (tid < E && rl < k) cand[t][wv * k + rl] = make_float2(le, __int_as_float(tid));
    if (lane < k && wv * 64 + lane >= E)
      cand[t][wv * k + lane] = make_float2(-__builtin_inff(), __int_as_float(0x7fffffff));
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if (t >= T) break;
    const int nc = 4 * k;
    if (tid < nc) {
      const float2 me = cand[t][tid];
      const float le = me.x;
      const int e = __float_as_int(me.y);
      int r = 0;
      for (int c0 = 0; c0 < nc; c0 += 8) {
        float2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = cand[t][min(c0 + u, nc - 1)];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (c0 + u < nc)
            r += (v[u].x > le) | ((v[u].x == le) & (__float_as_int(v[u].y) < e));
      }
      if (r < k && e != 0x7fffffff) {
        sel_e[t * k + r] = e;
        sel_l[t * k + r] = le;
      }
    }
  }
  __syncthreads();
  if (tid < nq) {
    const int t = tid / k;
    const float m = sel_l[t * k];
    float den = 0.f;
    for (int i = 0; i < k; ++i) den += expf(sel_l[t * k + i] - m);
    const float w = expf(sel_l[tid] - m) / den;
    slot_e[tid] = sel_e[tid];
    slot_w[tid] = w;
    if (blockIdx.x == 0) {
      a.topk_id[tid] = sel_e[tid];
      a.topk_w[tid] = w;
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
    int na = 0;
    for (int q = 0; q < nq; ++q) na += slot_first[q];
    s_nact = na;
  }
  __syncthreads();
  const int na = s_nact;
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

  // ---- C: gate/up + SwiGLU; item = (active expert, 16-feature tile) per wavefront ----
  {
    const int nch = H / kChunk;  // chunks along the hidden dimension
    const int ntile = I / 16;
    const int n_items = na * ntile;
    const int W = G * 4, gw = blockIdx.x * 4 + wv;
    const int nspi = (nch + kLsSetC - 1) / kLsSetC;  // load sets per item
    const int my_items = gw < n_items ? (n_items - 1 - gw) / W + 1 : 0;
    const int nsets = my_items * nspi;
    const size_t mq = (size_t)I * H / 2, ms = (size_t)I * H / 16;
    uint4 qgA[kLsSetC], quA[kLsSetC], qgB[kLsSetC], quB[kLsSetC];
    uint32_t sgA[kLsSetC], suA[kLsSetC], sgB[kLsSetC], suB[kLsSetC];
    auto load_set = [&](uint4* qg, uint4* qu, uint32_t* sg, uint32_t* su, int s) {
      s = min(s, nsets - 1);  // past the end: re-read the last set (unused)
      const int it = gw + (s / nspi) * W;
      const int ai = it / ntile, rt = it - ai * ntile;
      const int e = act_e[ai];
      const int cs = (s % nspi) * kLsSetC;
      const size_t tq = (size_t)e * mq + ((size_t)rt * nch) * 1024 + lane * 16;
      const size_t ts_ = (size_t)e * ms + ((size_t)rt * nch) * 128 + lane * 2;
#pragma unroll
      for (int u = 0; u < kLsSetC; ++u) {
        const int c = min(cs + u, nch - 1);
        qg[u] = *reinterpret_cast<const uint4*>(a.gq + tq + (size_t)c * 1024);
        qu[u] = *reinterpret_cast<const uint4*>(a.uq + tq + (size_t)c * 1024);
        sg[u] = load_u16(a.gs + ts_ + (size_t)c * 128);
        su[u] = load_u16(a.us + ts_ + (size_t)c * 128);
      }
    };
    float ag[TT], au[TT];
#pragma unroll
    for (int r = 0; r < TT; ++r) ag[r] = au[r] = 0.f;
    auto use_set = [&](const uint4* qg, const uint4* qu, const uint32_t* sg, const uint32_t* su,
                       int s) {
      const int it = gw + (s / nspi) * W;
      const int ai = it / ntile, rt = it - ai * ntile;
      const int rows = act_cnt[ai], off = act_off[ai];
      const int cs = (s % nspi) * kLsSetC;
#pragma unroll
      for (int u = 0; u < kLsSetC; ++u) {
        const int c = cs + u;
        if (c < nch) {
          Dec32bf dg, du;  // decoded once, dotted with every row
          decode32(qg[u], sg[u], dg);
          decode32(qu[u], su[u], du);
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
      if (s % nspi == nspi - 1) {  // the item's last set: SwiGLU and store two features per lane
        const int e = act_e[ai];
        const float tsg = a.ts[e * 3 + 0], tsu = a.ts[e * 3 + 1];
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
    if (nsets > 0) {
      load_set(qgA, quA, sgA, suA, 0);
      for (int s = 0; s < nsets; s += 2) {
        load_set(qgB, quB, sgB, suB, s + 1);
        use_set(qgA, quA, sgA, suA, s);
        load_set(qgA, quA, sgA, suA, s + 2);
        if (s + 1 < nsets) use_set(qgB, quB, sgB, suB, s + 1);
      }
    }
  }
  ls_arrive(a.sync, kLsSyncC, kLsFlagC, (uint32_t)G);

  // ---- D: down + combine ----
  {
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
      const size_t ts_ = (size_t)e * ms + ((size_t)ft * nci + cbeg) * 128 + lane * 2;
#pragma unroll
      for (int u = 0; u < kLsSetD; ++u) {
        const int c = min(cs + u, nck - 1);
        q[u] = *reinterpret_cast<const uint4*>(a.dq + tq + (size_t)c * 1024);
        sc[u] = load_u16(a.ds + ts_ + (size_t)c * 128);
      }
    };
    const bool has_k = nck > 0;
    // a block with no output tile neither waits nor stages h
    if (ftp < npairs) {
      // the first weights are requested before waiting for h (not by the polling wavefront,
      // whose poll would queue behind them)
      if (has_k && wv != 0) load_set(qA, sA, 0);
      if (!ls_wait(a.sync, kLsFlagC, &s_flag)) return;
      if (has_k && wv == 0) load_set(qA, sA, 0);
      // both halves of every h row: LDS [half][row][hw_row words].  Plain (cached) loads: no
      // block of this kernel read these lines before counter C, and the caches hold nothing
      // from earlier kernels.
      uint32_t* hs0 = dyn;
      const int rq = I / 8;  // 16-byte pieces per h row
      for (int i = tid; i < nq * rq; i += 256) {
        const int p = i / rq, pc = i - p * rq;
        const int half = pc >= (nci / 2) * (kChunk / 8) ? 1 : 0;
        const int pl = pc - half * (nci / 2) * (kChunk / 8);
        *reinterpret_cast<uint4*>(hs0 + ((size_t)half * nq + p) * hw_row + pl * 4) =
            reinterpret_cast<const uint4*>(a.h)[i];
      }
      lds_barrier();
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
            decode32(q[u], sc[u], d);
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
          const float tsd = a.ts[act_e[ai] * 3 + 2];
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
      if (has_k) {
        if (ftp != (int)blockIdx.x) load_set(qA, sA, 0);
        for (int s = 0; s < nsets; s += 2) {
          load_set(qB, sB, s + 1);
          use_set(qA, sA, s);
          load_set(qA, sA, s + 2);
          if (s + 1 < nsets) use_set(qB, sB, s + 1);
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
  }

  // ---- exit: the last block resets the counters and flags for the next call ----
  if (tid == 0) {
    __builtin_amdgcn_s_waitcnt(0);  // this block's flag stores are complete
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t old =
        __hip_atomic_fetch_add(a.sync + kLsSyncX, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old == (uint32_t)G - 1) {
      // every block has passed both barriers: nobody polls these words any more
      st_dev(a.sync + kLsSyncA, 0u);
      st_dev(a.sync + kLsSyncC, 0u);
      for (int i = 0; i < kLsFlags; ++i) {
        st_dev(a.sync + kLsFlagBase + i * kLsFlagStride + kLsFlagA, 0u);
        st_dev(a.sync + kLsFlagBase + i * kLsFlagStride + kLsFlagC, 0u);
      }
      st_dev(a.sync + kLsSyncX, 0u);
    }
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
// block fits per CU (every block must be resident).  0 if not.
static int layer_small_grid(int T, bool vec, size_t lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  int occ = 0;
  const void* f = T == 1 ? (vec ? (const void*)layer_small_kernel<1, true>
                                : (const void*)layer_small_kernel<1, false>)
                         : (vec ? (const void*)layer_small_kernel<2, true>
                                : (const void*)layer_small_kernel<2, false>);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, 256, lds) != hipSuccess) return 0;
  return occ >= 1 ? ncu : 0;
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
