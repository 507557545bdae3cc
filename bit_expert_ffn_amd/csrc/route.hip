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
#include "common.h"

namespace moe {

constexpr int kRows = 16;  // router-weight rows per wavefront per batch of loads

RoutePlan route_plan(int T, int H, int E) {
  (void)E;
  RoutePlan p;
  p.TT = T <= 1 ? 1 : T <= 4 ? 4 : T <= 64 ? 8 : 16;
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
                        float* partial, hipStream_t s) {
  const RoutePlan p = route_plan(T, H, E);
  dim3 grid(p.tiles, p.KS);
#define MOE_SLICES(TT_, RG_)                                                                  \
  do {                                                                                        \
    if ((E & 3) == 0)                                                                         \
      router_slices_kernel<TT_, RG_, true><<<grid, RG_ * 64, 0, s>>>(x, wr, T, H, E, p.kc,   \
                                                                     partial);                \
    else                                                                                      \
      router_slices_kernel<TT_, RG_, false><<<grid, RG_ * 64, 0, s>>>(x, wr, T, H, E, p.kc,  \
                                                                      partial);               \
  } while (0)
  switch (p.TT) {
    case 1: MOE_SLICES(1, 8); break;
    case 4: MOE_SLICES(4, 8); break;
    case 8: MOE_SLICES(8, 4); break;
    default: MOE_SLICES(16, 4); break;
  }
#undef MOE_SLICES
  if (p.KS >= 8)
    router_select_kernel<4><<<T, 1024, 0, s>>>(partial, p.KS, bias, T, E, k, logits, topk_id,
                                               topk_w);
  else
    router_select_kernel<1><<<T, 256, 0, s>>>(partial, p.KS, bias, T, E, k, logits, topk_id,
                                              topk_w);
  return hipGetLastError();
}

}  // namespace moe
