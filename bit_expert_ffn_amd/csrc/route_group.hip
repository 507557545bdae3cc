// Fused routing for a small batch (3..128 tokens): router logits, top-k + softmax, the grouping
// of the (token, slot) rows by expert and the grouped GEMM's tile plan, in ONE persistent kernel.
//
// Sources: at small batch the routing steps are short and bound by latency, so they run as one
// program with no launch gaps between them ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", section 1 "A megakernel" and section 2 "Pipelining everything inside the
// megakernel"); every token is routed to k of E experts (same page, Background / "The model");
// index building stays on the device with no host round trip ("Day-0 Inference Adaptation for
// Ultra-Large Sparse Models", "Operator Layer", Index Pipeline).
//
// One block of 256 threads per CU, every block resident (the host checks occupancy); blocks
// wait for each other at the grid barriers of sync.h.  Phases:
//   A  router partial logits on the matrix cores.  Item = (1/32 of the hidden steps, 32
//      experts); its four wavefronts take interleaved 16-position steps.  Each fp32 router
//      weight is split in registers into three bf16 pieces whose sum is exactly the weight
//      (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid); x is bf16, so every product
//      x * piece is exact in fp32 and the logits differ from the fp32 definition only in the
//      order of the fp32 additions.  v_mfma_f32_32x32x16_bf16 takes 32 tokens x 16 positions
//      of x and 16 positions x 32 experts of one piece.  The wavefronts' sums are added in LDS
//      in a fixed order and the item's partials [slice][token][expert] go out with
//      device-scope stores.  Barrier A.
//   B  block t takes token t: adds its 32 partial slices in order (device-scope loads), adds
//      the bias, sorts the experts by selection key (larger logit, or equal logit and lower id;
//      a bitonic network over the block) and writes the k best in descending order with the
//      softmax over them; each of the k experts gets this token's bit in its token mask (an
//      atomic OR, cleared before barrier A).  Barrier C.
//   C  grouping without a serial pass: every token block reads the E token masks; an expert's
//      row count is the popcount of its mask, the offsets are their exclusive scan, and token
//      t's row for expert e is offset[e] plus the number of earlier tokens in e's mask (the
//      stable order: by token, and a token's k experts are distinct).  Each token block writes
//      its own k rows; block 0 also writes the counts and offsets, the active experts sorted by
//      (count desc, id asc) (a bitonic sort of count << 8 | (255 - id)) and the grouped GEMM's
//      row tiles.
//   Exit barrier X (its last arrival resets the counters and flags): a token block arrives as
//   soon as it has passed barrier C, its last wait, and before its stores of phase C, so that
//   the reset overlaps them; the other blocks arrive after barrier C's arrival.
// A wait that gives up sets the error word (as in the single-launch layer); block 0 then writes
// a grouping with no active expert, identity slot rows and NaN weights, so the kernels that
// follow stay inside their buffers and out shows NaN.
// Results are the same as moe_route + moe_group for the same logits: the grouping is bit-exact
// and deterministic; the logits differ from the fp32-slice router only in summation order.
#include <mutex>

#include "common.h"
#include "group_dev.h"
#include "select_dev.h"
#include "sync.h"

namespace moe {

// Profiling builds only (compiled with -DMOE_TIMELINE): each block's first thread records the
// 100 MHz real-time counter at the phase boundaries of the last call, read back with
// moe_timeline_route_group.  Slots: 0 entry, 1 router partials stored, 2 barrier A passed (token
// blocks), 3 top-k done, 4 barrier C passed, 5 rows placed, 6 block 0: active list sorted,
// 7 exit; inside phase A: 8 first loads issued, 9 products done, 10 sums in LDS.
#ifdef MOE_TIMELINE
__device__ unsigned long long g_rg_timeline[1024][16];
#define RG_STAMP(i)                                                                 \
  do {                                                                              \
    if (threadIdx.x == 0 && blockIdx.x < 1024)                                      \
      g_rg_timeline[blockIdx.x][i] = __builtin_amdgcn_s_memrealtime();              \
  } while (0)
#else
#define RG_STAMP(i) \
  do {              \
  } while (0)
#endif

constexpr int kRgSlices = 32;  // phase A: slices of the hidden dimension
constexpr int kRgEG = 32;      // phase A: experts per item
constexpr int kRgBatch = 4;    // phase A: steps per wavefront whose loads are in flight together
constexpr int kRgMaskWords = kRgMaxT / 32;  // phase C: token-mask words per expert

typedef __attribute__((ext_vector_type(8))) __bf16 rg_bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t rg_u32x4;

// Sorts the 256 keys of a 256-thread block in descending order (a bitonic network: partners
// within a wavefront exchange through lane shuffles, the strides of 64 and 128 through LDS);
// returns the key at this thread's position.  buf: 256 keys of LDS scratch.
template <typename K>
__device__ inline K block_sort_desc(K v, K* buf) {
  const int i = threadIdx.x;
  for (int size = 2; size <= 256; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      K pv;
      if (stride >= 64) {
        buf[i] = v;
        __syncthreads();
        pv = buf[i ^ stride];
        __syncthreads();
      } else if (sizeof(K) == 8) {
        const uint64_t u = (uint64_t)v;
        const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, stride);
        const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), stride);
        pv = (K)(((uint64_t)hi << 32) | lo);
      } else {
        pv = (K)(uint32_t)__shfl_xor((int)(uint32_t)v, stride);
      }
      // the pair (i, i ^ stride) runs descending where (i & size) == 0, ascending elsewhere
      // (all descending in the last merge); the lower position keeps the larger key in a
      // descending run
      const bool lower = (i & stride) == 0;
      const bool keep_max = ((i & size) == 0) == lower;
      v = keep_max ? (v > pv ? v : pv) : (v < pv ? v : pv);
    }
  }
  return v;
}

// Block 0 after a wait gave up: a grouping that no later kernel can misuse -- no active expert
// and no GEMM tile (the expert-FFN kernels then do nothing), slot rows that stay inside y, and
// NaN routing weights, so the combine's out shows the failure.
__device__ inline void route_group_fail(const RouteGroupArgs& a) {
  const int n = a.T * a.k;
  for (int i = threadIdx.x; i < n; i += 256) {
    a.sorted_slot[i] = i;
    a.slot_row[i] = i;
    st_dev(reinterpret_cast<uint32_t*>(a.topk_w) + i, 0x7fc00000u);
  }
  for (int e = threadIdx.x; e < a.E; e += 256) {
    a.count[e] = 0;
    a.offset[e] = 0;
    a.active[e] = -1;
  }
  if (threadIdx.x == 0) {
    a.offset[a.E] = 0;
    *a.n_active = 0;
    if (a.plan_MT > 0) *a.n_tiles = 0;
  }
}

template <int TTT>  // 32-token tiles: T <= 32 * TTT
__global__ __launch_bounds__(256, 1) void route_group_kernel(RouteGroupArgs a) {
  // every LDS array is a __shared__ object, so that its accesses compile to LDS instructions
  // (through a generic pointer they become flat accesses, each of which also waits for the
  // block's outstanding global stores)
  __shared__ __attribute__((aligned(16))) float red[4][TTT * 32][kRgEG];  // A
  __shared__ uint64_t sortbuf[kMaxExperts];                               // B, C
  __shared__ float lgs[kMaxExperts];                                       // B
  __shared__ float selv[kMaxExperts];
  __shared__ int selid[kMaxExperts];
  __shared__ float s_den;
  __shared__ int s_flag, s_nact;
  __shared__ uint32_t masks[kMaxExperts][kRgMaskWords];                   // C
  __shared__ __attribute__((aligned(16))) int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 4];
  __shared__ int act_l[kMaxExperts];

  RG_STAMP(0);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = gridDim.x;
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  const uint32_t spin_cfg = a.sync[kLsSyncSpin];
  const uint32_t spin = spin_cfg != 0 ? spin_cfg : kLsSpin;
  uint32_t* part = reinterpret_cast<uint32_t*>(a.partial);
  // the experts' token masks start zero: cleared before barrier A, set in phase B
  if (blockIdx.x == 0)
    for (int i = tid; i < E * kRgMaskWords; i += 256) st_dev(a.masks + i, 0u);

  // ---- A: router partial logits on the matrix cores ----
  {
    const int NEG = (E + kRgEG - 1) / kRgEG;
    const int nst = H / 16;  // 16-position steps of the hidden dimension
    const int r32 = lane & 31, kg = lane >> 5;
    for (int it = blockIdx.x; it < kRgSlices * NEG; it += G) {
      // item it -> (slice, expert group): the NEG items of one slice get the same it % 8, so
      // they run on one XCD and share the slice's x rows in its L2
      const int j8 = it >> 3;
      const int sl = (it & 7) + 8 * (j8 / NEG), eg = j8 % NEG;
      const int s0 = sl * nst / kRgSlices, s1 = (sl + 1) * nst / kRgSlices;
      const int e = min(eg * kRgEG + r32, E - 1);  // clamped columns are not stored
      f32x16 acc[TTT];
#pragma unroll
      for (int i = 0; i < TTT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;
      // this wavefront's steps s0 + wv, s0 + wv + 4, ..., kRgBatch at a time: every load of a
      // batch is issued before the first product (steps past s1 re-read step s1 - 1 and are
      // not multiplied)
      for (int sb = s0 + wv; sb < s1; sb += 4 * kRgBatch) {
        float w[kRgBatch][8];
        rg_u32x4 xa[kRgBatch][TTT];
#pragma unroll
        for (int b = 0; b < kRgBatch; ++b) {
          const int st = min(sb + 4 * b, s1 - 1);
          const int h0 = st * 16 + kg * 8;  // this lane's 8 hidden positions
#pragma unroll
          for (int j = 0; j < 8; ++j) w[b][j] = a.wr[(size_t)(h0 + j) * E + e];
#pragma unroll
          for (int i = 0; i < TTT; ++i) {
            const int t = min(i * 32 + r32, T - 1);  // rows past T are not stored
            xa[b][i] = *reinterpret_cast<const rg_u32x4*>(a.x + (size_t)t * H + h0);
          }
        }
        if (sb == s0 + wv) RG_STAMP(8);
#pragma unroll
        for (int b = 0; b < kRgBatch; ++b) {
          if (sb + 4 * b < s1) {
            // exact three-piece split of every weight
            rg_bf16x8 p[3];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const __bf16 hi = (__bf16)w[b][j];
              const float r1 = w[b][j] - (float)hi;
              const __bf16 mid = (__bf16)r1;
              const float r2 = r1 - (float)mid;
              p[0][j] = hi;
              p[1][j] = mid;
              p[2][j] = (__bf16)r2;
            }
#pragma unroll
            for (int q = 2; q >= 0; --q)  // small pieces first
#pragma unroll
              for (int i = 0; i < TTT; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(rg_bf16x8, xa[b][i]), p[q], acc[i], 0, 0, 0);
          }
        }
      }
      RG_STAMP(9);
      // accumulator element v of lane l: token (v / 4) * 8 + (l / 32) * 4 + v % 4 of its tile,
      // expert l % 32 of the item
#pragma unroll
      for (int i = 0; i < TTT; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[wv][i * 32 + (v >> 2) * 8 + kg * 4 + (v & 3)][r32] = acc[i][v];
      __syncthreads();
      RG_STAMP(10);
      for (int q = tid; q < TTT * 32 * kRgEG; q += 256) {
        const int t = q / kRgEG, el = q - t * kRgEG, ee = eg * kRgEG + el;
        const float s = ((red[0][t][el] + red[1][t][el]) + red[2][t][el]) + red[3][t][el];
        if (t < T && ee < E) st_dev(part + ((size_t)sl * T + t) * E + ee, __float_as_uint(s));
      }
      __syncthreads();
    }
  }
  RG_STAMP(1);
  ls_arrive(a.sync, kLsSyncA, kLsFlagA, (uint32_t)G);

  // ---- B: one token per block: logits, top-k, softmax ----
  const int t = blockIdx.x;
  if (t < T) {
    if (!ls_wait(a.sync, kLsFlagA, &s_flag, spin)) {
      if (blockIdx.x == 0) route_group_fail(a);
      ls_exit(a.sync, (uint32_t)G);
      return;
    }
    RG_STAMP(2);
    float lg = 0.f;
    uint64_t key = 0;  // below every real key
    if (tid < E) {
      float v[kRgSlices];
#pragma unroll
      for (int sl = 0; sl < kRgSlices; ++sl)
        v[sl] = __uint_as_float(ld_dev(part + ((size_t)sl * T + t) * E + tid));
      float sum = 0.f;
#pragma unroll
      for (int sl = 0; sl < kRgSlices; ++sl) sum += v[sl];
      if (a.bias) sum += a.bias[tid];
      if (a.logits) a.logits[(size_t)t * E + tid] = sum;
      lg = sum;
      key = sel_key(sum, tid);
    }
    lgs[tid] = lg;
    // the experts in selection order: position j holds the expert of rank j
    key = block_sort_desc(key, sortbuf);
    if (tid < k) {
      const int id = sel_id(key);
      selid[tid] = id;
      selv[tid] = lgs[id];
    }
    __syncthreads();
    if (tid == 0) {
      const float m = selv[0];
      float den = 0.f;
      for (int j = 0; j < k; ++j) den += expf(selv[j] - m);
      s_den = den;
    }
    __syncthreads();
    if (tid < k) {
      const int e = selid[tid];
      st_dev(reinterpret_cast<uint32_t*>(a.topk_id) + (size_t)t * k + tid, (uint32_t)e);
      st_dev(reinterpret_cast<uint32_t*>(a.topk_w) + (size_t)t * k + tid,
             __float_as_uint(expf(selv[tid] - selv[0]) / s_den));
      // this token in expert e's mask (the k experts of a token are distinct)
      __hip_atomic_fetch_or(a.masks + e * kRgMaskWords + (t >> 5), 1u << (t & 31),
                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  RG_STAMP(3);
  ls_arrive(a.sync, kLsSyncC, kLsFlagC, (uint32_t)G);

  // ---- C: every token block places its own k rows; block 0 also writes the per-expert
  // arrays, the active list and the GEMM tiles.  The grouped order is stable: within expert e
  // the rows follow the token order, so the row of (t, j) is offset[e] plus the number of
  // earlier tokens in e's mask. ----
  if (t < T) {
    if (!ls_wait(a.sync, kLsFlagC, &s_flag, spin)) {
      if (blockIdx.x == 0) route_group_fail(a);
      ls_exit(a.sync, (uint32_t)G);
      return;
    }
    // this block's last wait is over and its flag stores are complete: it arrives at the exit
    // barrier now, so that the reset overlaps the stores below instead of following them
    ls_exit(a.sync, (uint32_t)G);
    RG_STAMP(4);
    const int mw = (T + 31) >> 5;  // mask words in use
    int c = 0;
    if (tid < E) {
#pragma unroll
      for (int w = 0; w < kRgMaskWords; ++w) {
        const uint32_t m = w < mw ? ld_dev(a.masks + tid * kRgMaskWords + w) : 0u;
        masks[tid][w] = m;
        c += __popc(m);
      }
    }
    cnt[tid] = c;
    __syncthreads();
    if (wv == 0) wave_scan_offsets(cnt, E, off);
    __syncthreads();
    if (tid < k) {
      const int e = selid[tid];
      int below = __popc(masks[e][t >> 5] & ((1u << (t & 31)) - 1u));
#pragma unroll
      for (int w = 0; w < kRgMaskWords; ++w) below += w < (t >> 5) ? __popc(masks[e][w]) : 0;
      const int pos = off[e] + below;
      const int slot = t * k + tid;
      a.slot_row[slot] = pos;
      a.sorted_slot[pos] = slot;
    }
    RG_STAMP(5);
    if (blockIdx.x == 0) {
      if (tid < E) {
        a.count[tid] = cnt[tid];
        a.offset[tid] = off[tid];
        if (tid == 0) a.offset[E] = off[E];
      }
      // active experts by (count desc, id asc): sort the keys count << 8 | (255 - id) of the
      // experts with rows; inactive experts have key 0 and sort last
      const uint32_t akey =
          tid < E && cnt[tid] > 0 ? ((uint32_t)cnt[tid] << 8) | (uint32_t)(255 - tid) : 0u;
      const int nact = __syncthreads_count(akey != 0);
      const uint32_t sk = block_sort_desc(akey, reinterpret_cast<uint32_t*>(sortbuf));
      act_l[tid] = sk != 0 ? 255 - (int)(sk & 255u) : -1;
      if (tid < E) a.active[tid] = act_l[tid];
      if (tid == 0) {
        *a.n_active = nact;
        s_nact = nact;
      }
      __syncthreads();
      RG_STAMP(6);
      if (a.plan_MT > 0 && wv == 0)
        ffn_plan_n(cnt, off, act_l, s_nact, a.plan_MT, a.plan_min_rows, a.tiles, a.max_tiles,
                   a.n_tiles);
    }
  }
  RG_STAMP(7);
  if (t >= T) ls_exit(a.sync, (uint32_t)G);
}

bool route_group_fits(int T, int k) {
  return T >= 1 && T <= kRgMaxT && (size_t)T * k <= (size_t)kRgMaxSlots;
}

// Blocks: one per CU if one block fits per CU (every block must be resident), else 0.  Cached
// per (device, kernel), computed on the first launch there.
static int route_group_grid(int ttt) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int var = ttt == 1 ? 0 : ttt == 2 ? 1 : 2;
  static std::mutex mu;
  static int cache[64][3];
  {
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev][var] > 0) return cache[dev][var];
  }
  int ncu = 0;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const void* f = ttt == 1 ? (const void*)route_group_kernel<1>
                           : ttt == 2 ? (const void*)route_group_kernel<2>
                                      : (const void*)route_group_kernel<4>;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, f, 256, 0) != hipSuccess) return 0;
  const int grid = occ >= 1 ? ncu : 0;
  if (grid > 0) {
    std::lock_guard<std::mutex> lock(mu);
    cache[dev][var] = grid;
  }
  return grid;
}

hipError_t launch_route_group(const RouteGroupArgs& a, hipStream_t s) {
  const int ttt = a.T <= 32 ? 1 : a.T <= 64 ? 2 : 4;
  const int grid = route_group_grid(ttt);
  // phase B gives every token a block of its own
  if (grid == 0 || grid < a.T) return hipErrorInvalidConfiguration;
  if (ttt == 1)
    route_group_kernel<1><<<grid, 256, 0, s>>>(a);
  else if (ttt == 2)
    route_group_kernel<2><<<grid, 256, 0, s>>>(a);
  else
    route_group_kernel<4><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_TIMELINE
extern "C" __attribute__((visibility("default"))) int moe_timeline_route_group(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(moe::g_rg_timeline), sizeof(moe::g_rg_timeline),
                                  0, hipMemcpyDeviceToHost);
}
#endif
