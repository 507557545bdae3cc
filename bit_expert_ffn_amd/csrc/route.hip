// Router GEMV/GEMM, top-k and softmax over the selected logits.
// The layer routes every token to k of E experts ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", Background / "The model"); the routing weights are the softmax over the k
// selected logits.
//
// Two kernels:
//   router_slices_kernel  grid (token tiles of TT, KS slices of the hidden dimension).  Lane l
//       owns experts 4l..4l+3 (one 16-byte load per router-weight row, a whole 1 KB row per
//       wavefront); the RG wavefronts of a block take interleaved rows in batches of kRows
//       unconditional loads, and their sums are added in LDS in a fixed order.  Each block
//       writes fp32 partial logits of its tokens over its slice.  Splitting the hidden
//       dimension lets a single token spread over many CUs.
//   router_select_kernel  one block per token: adds the KS slices in slice order (so the logits
//       are deterministic), adds the bias, writes the logits, then ranks the experts: expert
//       e's rank is the number of experts with a larger key (logit, then lower id first), all
//       counted in parallel, and the experts of rank < k are the top-k in order.  The weights
//       are the softmax over the selected logits.
// The kernel boundary between the two makes the partials visible without device-scope
// fences inside a kernel.
//
// Many tokens (T >= kRouteMfmaMinT): the slices come from the matrix cores instead.
//   router_split_kernel   writes each fp32 router weight as the exact sum of three bf16 values
//       (hi = bf16(w), mid = bf16(w - hi), lo = w - hi - mid), in the order the matrix-core
//       operand reads them (1 KB per 32 experts x 16 hidden positions).
//   router_mfma_kernel    block = 128 tokens x 256 experts (4 wavefronts of 64 experts) over one
//       slice of the hidden dimension, x staged in LDS; logits += x * hi + x * mid + x * lo on
//       v_mfma_f32_32x32x16_bf16.  x is bf16, so every product is exact in fp32 and the result
//       differs from the fp32 definition only in the order of the fp32 additions.
#include "common.h"

namespace moe {

constexpr int kRows = 16;  // router-weight rows per wavefront per batch of loads

RoutePlan route_plan(int T, int H, int E) {
  (void)E;
  RoutePlan p;
  if (T >= kRouteMfmaMinT) {
    // matrix-core router: 128-token tiles; split the hidden dimension until there are at least
    // 512 blocks (two per CU), in slices that are multiples of 128
    p.mfma = true;
    p.TT = 128;
    p.RG = 4;
    p.tiles = (T + 127) / 128;
    const int ks = (512 + p.tiles - 1) / p.tiles;
    int kc = (H + ks - 1) / ks;
    kc = (kc + 127) / 128 * 128;
    if (kc > H) kc = H;
    p.kc = kc;
    p.KS = (H + kc - 1) / kc;
    return p;
  }
  p.mfma = false;
  // 4-token tiles on 8 wavefronts from 2 tokens up: two wavefronts per SIMD hide the LDS and
  // load latency of the FMA loop (measured faster than 8- or 16-token tiles on 4 wavefronts at
  // 64 and 128 tokens)
  p.TT = T <= 1 ? 1 : 4;
  p.RG = p.TT <= 4 ? 8 : 4;
  const int tiles = (T + p.TT - 1) / p.TT;
  int kc;
  if (tiles >= 128) {
    kc = H;  // enough token tiles to fill the chip: no split of the hidden dimension
  } else {
    // ~256 blocks in total; slices of at least one batch of loads per wavefront
    const int ks = (256 + tiles - 1) / tiles;
    kc = (H + ks - 1) / ks;
    const int minkc = kRows * p.RG;
    kc = (kc + minkc - 1) / minkc * minkc;
  }
  if (kc > H) kc = H;
  p.kc = kc;
  p.KS = (H + kc - 1) / kc;
  p.tiles = tiles;
  return p;
}

template <int TT, int RG, bool VEC>
__global__ __launch_bounds__(RG * 64) void router_slices_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ wr, int T, int H, int E, int kc,
    float* __restrict__ partial) {
  constexpr int NT = RG * 64;
  __shared__ float xs[TT][256];
  __shared__ float red[RG][TT][kMaxExperts];
  const int tile = blockIdx.x, ks = blockIdx.y;
  const int t0 = tile * TT;
  const int lane = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int e0 = lane * 4;
  const int k_begin = ks * kc, k_end = min(H, k_begin + kc);
  float acc[TT][4];
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = 0.f;

  for (int kb = k_begin; kb < k_end; kb += 256) {
    const int len = min(256, k_end - kb);
    __syncthreads();
    for (int i = threadIdx.x; i < TT * 256; i += NT) {
      const int t = i >> 8, h = i & 255;
      float v = 0.f;
      if (t0 + t < T && h < len) v = bf16_to_f32(x[(size_t)(t0 + t) * H + kb + h]);
      xs[t][h] = v;
    }
    __syncthreads();
    if (e0 < E) {
      // rows rg, rg + RG, ... of the staged chunk.  Every load is unconditional (row index
      // clamped into the chunk; a clamped row multiplies a zero x value), so a batch's loads
      // are all in flight together.
      const float* wrow = wr + (size_t)kb * E;
      for (int hb = 0; hb < len; hb += RG * kRows) {
        float w[kRows][4];
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
          const int h = min(hb + rg + RG * i, len - 1);
          if (VEC) {
            const float4 v = *reinterpret_cast<const float4*>(wrow + (size_t)h * E + e0);
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) w[i][j] = wrow[(size_t)h * E + min(e0 + j, E - 1)];
          }
        }
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
          const int h = hb + rg + RG * i;
#pragma unroll
          for (int t = 0; t < TT; ++t) {
            const float xv = h < len ? xs[t][h] : 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[t][j] = fmaf(xv, w[i][j], acc[t][j]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + j < E) red[rg][t][e0 + j] = acc[t][j];
  __syncthreads();
  // this slice's partial logits: the row groups added in order
  for (int i = threadIdx.x; i < TT * E; i += NT) {
    const int t = i / E, e = i - t * E;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += red[r][t][e];
    if (t0 + t < T) partial[((size_t)ks * T + t0 + t) * E + e] = s;
  }
}

// bf16 nearest-even of a finite float (NaN stays NaN)
__device__ inline uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// wr [H][E] fp32 -> wsplit: three bf16 planes with w = hi + mid + lo exactly: hi keeps the leading
// 8 significant bits (rounded), the residual w - hi is exact in fp32 and has at most 16
// significant bits, mid keeps 8 of them and the remaining w - hi - mid fits in lo.
// Each plane is stored in the order the matrix-core operand reads it: for the 32-expert tile et
// and the 16-position step st, 1 KB holds lane l's 8 values at byte 16 l (expert 32 et + l % 32,
// positions 16 st + 8 (l / 32) .. + 7), so one wavefront's operand of one step is one coalesced
// 1 KB load.  Element offset (((p NET + et) NST + st) 64 + l) 8 + j, NET = ceil(E / 32), NST =
// H / 16; the experts past E in the last tile are zero.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ wr, int H,
                                                           int E, uint16_t* __restrict__ wsplit) {
  __shared__ float tile[64][65];  // [position][expert]
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int hh = i >> 6, ee = i & 63;
    float v = 0.f;
    if (h0 + hh < H && e0 + ee < E) v = wr[(size_t)(h0 + hh) * E + e0 + ee];
    tile[hh][ee] = v;
  }
  __syncthreads();
  const int NET = (E + 31) / 32, NST = H / 16;
  const size_t plane = (size_t)NET * 32 * H;
  // item = (expert ee of the tile, 8-position group hg): two per thread
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int ee = i & 63, hg = i >> 6;
    const int e = e0 + ee, h = h0 + hg * 8;
    if (e >= NET * 32 || h >= H) continue;
    uint32_t pk[3][4];
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      uint32_t q[3] = {0u, 0u, 0u};
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float v = tile[hg * 8 + j + jj][ee];
        const uint16_t hi = f32_to_bf16_rne(v);
        const float r1 = v - bf16_to_f32(hi);
        const uint16_t mid = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_to_f32(mid);
        const uint16_t lo = f32_to_bf16_rne(r2);
        q[0] |= (uint32_t)hi << (16 * jj);
        q[1] |= (uint32_t)mid << (16 * jj);
        q[2] |= (uint32_t)lo << (16 * jj);
      }
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) pk[pp][j / 2] = q[pp];
    }
    const int et = e >> 5, st = h >> 4, l = ((h >> 3) & 1) * 32 + (e & 31);
    const size_t o = (((size_t)et * NST + st) * 64 + l) * 8;
#pragma unroll
    for (int pp = 0; pp < 3; ++pp)
      *reinterpret_cast<uint4*>(wsplit + pp * plane + o) = make_uint4(pk[pp][0], pk[pp][1], pk[pp][2], pk[pp][3]);
  }
}

// Block: 4 wavefronts, 128 tokens; wavefront w takes experts 64 w .. 64 w + 63 (two 32-expert
// tiles) for all 128 tokens (four 32-token tiles), over hidden positions [ks kc, ks kc + kc).
// x goes through LDS: the block loads each 64-position chunk of its 128 token rows once, with
// coalesced 16-byte loads, double-buffered (the next chunk's loads are in flight during the
// current chunk's products), and every wavefront reads its A operands (lane l: token l % 32, 8
// positions from 8 (l / 32)) from there.  The split weights are read in operand order, one
// coalesced 1 KB load per operand, one step ahead.  Token rows past T are clamped and experts
// past E are zero; neither is stored.  A wavefront with no experts still loads x and meets the
// barriers.
constexpr int kRmChunk = 64;         // positions per x chunk in LDS
constexpr int kRmXS = kRmChunk + 8;  // bf16 per LDS row (padded: conflict-free 16-byte reads)
__global__ __launch_bounds__(256, 2) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wsplit,
                                                          int T, int H, int E, int kc,
                                                          float* __restrict__ partial) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][128 * kRmXS];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e_base = w * 64;
  const bool has_e = e_base < E;
  const int t0 = blockIdx.x * 128, ks = blockIdx.y;
  const int k_begin = ks * kc, k_end = min(H, k_begin + kc);
  const int nsteps = (k_end - k_begin) / 16;  // a multiple of 8: kc and H are multiples of 128
  const int nchunks = nsteps / 4;
  const int r32 = lane & 31, kg = lane >> 5;
  const int NET = (E + 31) / 32, NST = H / 16;
  const size_t plane = (size_t)NET * 32 * H;
  const int et0 = min(2 * w, NET - 1), et1 = min(2 * w + 1, NET - 1);
  const uint16_t* wb0 = wsplit + ((size_t)et0 * NST + k_begin / 16) * 512 + lane * 8;
  const uint16_t* wb1 = wsplit + ((size_t)et1 * NST + k_begin / 16) * 512 + lane * 8;

  // x chunk c: piece q = tid + 256 u is row q / 8, 16-byte piece q % 8 of the chunk
  u32x4 xv[4];
  auto load_x = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u, row = q >> 3, pc = q & 7;
      xv[u] = *reinterpret_cast<const u32x4*>(x + (size_t)min(t0 + row, T - 1) * H + k_begin +
                                             c * kRmChunk + pc * 8);
    }
  };
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u, row = q >> 3, pc = q & 7;
      *reinterpret_cast<u32x4*>(&xs[buf][row * kRmXS + pc * 8]) = xv[u];
    }
  };
  struct Regs {
    u32x4 b[3][2];
  };
  auto load_b = [&](Regs& r, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < 3; ++pp) {
      r.b[pp][0] = *reinterpret_cast<const u32x4*>(wb0 + pp * plane + (size_t)st * 512);
      r.b[pp][1] = *reinterpret_cast<const u32x4*>(wb1 + pp * plane + (size_t)st * 512);
    }
  };
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][n][v] = 0.f;
  auto compute = [&](const Regs& r, int buf, int sc) __attribute__((always_inline)) {
    u32x4 a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const u32x4*>(&xs[buf][(i * 32 + r32) * kRmXS + sc * 16 + kg * 8]);
#pragma unroll
    for (int pp = 2; pp >= 0; --pp)  // small pieces first
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[i][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, a[i]), __builtin_bit_cast(bf16x8, r.b[pp][n]), acc[i][n], 0, 0, 0);
  };
  Regs r0, r1;
  load_x(0);
  if (has_e) load_b(r0, 0);
  store_x(0);
  if (nchunks > 1) load_x(1);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // chunk c is in xs[c & 1]; the other buffer's chunk has been used
    if (c + 1 < nchunks) {
      store_x((c + 1) & 1);
      if (c + 2 < nchunks) load_x(c + 2);
    }
    if (has_e) {
#pragma unroll
      for (int sc = 0; sc < 4; sc += 2) {
        const int st = c * 4 + sc;
        load_b(r1, st + 1);
        __builtin_amdgcn_sched_barrier(0);
        compute(r0, c & 1, sc);
        __builtin_amdgcn_sched_barrier(0);
        load_b(r0, min(st + 2, nsteps - 1));
        __builtin_amdgcn_sched_barrier(0);
        compute(r1, c & 1, sc + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (!has_e) return;
  // accumulator element v of a 32x32 tile: token (v/4)*8 + (lane/32)*4 + v%4, expert lane % 32
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e_base + n * 32 + r32;
    if (e >= E) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + i * 32 + (v >> 2) * 8 + kg * 4 + (v & 3);
        if (t < T) partial[((size_t)ks * T + t) * E + e] = acc[i][n][v];
      }
  }
}

// Order-preserving map of a float to an unsigned integer.
__device__ inline uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One block per token, P threads per expert (256 * P threads).
template <int P>
__global__ __launch_bounds__(256 * P) void router_select_kernel(
    const float* __restrict__ partial, int KS, const float* __restrict__ bias, int T, int E,
    int k, float* __restrict__ logits, int32_t* __restrict__ topk_id,
    float* __restrict__ topk_w) {
  __shared__ __attribute__((aligned(16))) uint64_t key[kMaxExperts];
  __shared__ __attribute__((aligned(16))) uint64_t cand[4 * 32];  // two-level selection (k <= 32)
  __shared__ float lv[kMaxExperts];
  __shared__ int rank[kMaxExperts];
  __shared__ float selv[kMaxExperts];
  __shared__ float s_den;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int q = tid & (P - 1), e = tid / P;
  // logits: slices added in order, P threads per expert then a fixed shuffle tree
  {
    float s = 0.f;
    if (e < E) {
      // slices q, q + P, ... in order, 8 unconditional (clamped) loads in flight per batch
      const float* p = partial + (size_t)t * E + e;
      const size_t stride = (size_t)T * E;
      for (int qb = q; qb < KS; qb += 8 * P) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[(size_t)min(qb + i * P, KS - 1) * stride];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (qb + i * P < KS) s += v[i];
      }
    }
    if (P >= 2) s += __shfl_xor(s, 1, P);
    if (P >= 4) s += __shfl_xor(s, 2, P);
    if (q == 0) {
      if (e < E) {
        if (bias) s += bias[e];
        if (logits) logits[(size_t)t * E + e] = s;
        lv[e] = s;
        // larger key = earlier: higher logit, then lower expert id
        key[e] = ((uint64_t)ordered_bits(s) << 32) | (uint32_t)(kMaxExperts - 1 - e);
      } else {
        key[e] = 0;  // below every real key
      }
      rank[e] = 0;
    }
  }
  __syncthreads();
  if (P == 1 && k <= 32) {
    // two levels: each expert is ranked among the 64 keys of its wavefront; those of rank < k
    // are the candidates (the overall top k are among them), which are then ranked among each
    // other.  rank[e] is the overall rank for the top k and at least k for the others.
    const int wv = tid >> 6, lane = tid & 63;
    const uint64_t ke = key[tid];
    if (tid < 4 * k) cand[tid] = 0;
    int r = 0;
    const uint4* kp = reinterpret_cast<const uint4*>(key + wv * 64);
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const uint4 v = kp[j];
      r += (((uint64_t)v.y << 32) | v.x) > ke;
      r += (((uint64_t)v.w << 32) | v.z) > ke;
    }
    __syncthreads();
    if (ke != 0 && r < k) cand[wv * k + r] = ke;
    if (e < E) rank[e] = k;
    __syncthreads();
    if (tid < 4 * k) {
      const uint64_t kc = cand[tid];
      int rc = 0;
      for (int j = 0; j < 4 * k; ++j) rc += cand[j] > kc;
      if (kc != 0 && rc < k) rank[kMaxExperts - 1 - (int)(uint32_t)kc] = rc;
    }
    (void)lane;
  } else {
    // rank: thread (e, q) counts the larger keys among 256/P of them
    if (e < E) {
      const uint64_t ke = key[e];
      int r = 0;
      constexpr int span = kMaxExperts / P;
#pragma unroll 8
      for (int j = q * span; j < q * span + span; ++j) r += key[j] > ke;
      if (P > 1)
        atomicAdd(&rank[e], r);
      else
        rank[e] = r;
    }
  }
  __syncthreads();
  if (q == 0 && e < E && rank[e] < k) selv[rank[e]] = lv[e];
  __syncthreads();
  if (tid == 0) {
    const float m = selv[0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf(selv[j] - m);
    s_den = den;
  }
  __syncthreads();
  if (q == 0 && e < E && rank[e] < k) {
    const int j = rank[e];
    topk_id[(size_t)t * k + j] = e;
    topk_w[(size_t)t * k + j] = expf(lv[e] - selv[0]) / s_den;
  }
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                        int E, int k, float* logits, int32_t* topk_id, float* topk_w,
                        float* partial, uint16_t* wsplit, hipStream_t s) {
  const RoutePlan p = route_plan(T, H, E);
  dim3 grid(p.tiles, p.KS);
  if (p.mfma) {
    router_split_kernel<<<dim3(H / 64, ((E + 31) / 32 * 32 + 63) / 64), 256, 0, s>>>(wr, H, E, wsplit);
    router_mfma_kernel<<<grid, 256, 0, s>>>(x, wsplit, T, H, E, p.kc, partial);
  } else {
#define MOE_SLICES(TT_, RG_)                                                                  \
  do {                                                                                        \
    if ((E & 3) == 0)                                                                         \
      router_slices_kernel<TT_, RG_, true><<<grid, RG_ * 64, 0, s>>>(x, wr, T, H, E, p.kc,   \
                                                                     partial);                \
    else                                                                                      \
      router_slices_kernel<TT_, RG_, false><<<grid, RG_ * 64, 0, s>>>(x, wr, T, H, E, p.kc,  \
                                                                      partial);               \
  } while (0)
  if (p.TT == 1)
    MOE_SLICES(1, 8);
  else
    MOE_SLICES(4, 8);
#undef MOE_SLICES
  }
  if (p.KS >= 8)
    router_select_kernel<4><<<T, 1024, 0, s>>>(partial, p.KS, bias, T, E, k, logits, topk_id,
                                               topk_w);
  else
    router_select_kernel<1><<<T, 256, 0, s>>>(partial, p.KS, bias, T, E, k, logits, topk_id,
                                              topk_w);
  return hipGetLastError();
}

}  // namespace moe
