// Router GEMV/GEMM, top-k and softmax over the selected logits.
// The layer routes every token to k of E experts ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", Background / "The model"); the routing weights are the softmax over the k
// selected logits.
//
// Two kernels:
//   router_partial_kernel  fp32 partial logits over one slice of the hidden dimension
//                          (split-K so that a single token still spreads over many CUs);
//   router_topk_kernel     sums the slices in a fixed order (deterministic), adds the bias,
//                          writes the logits, then one wavefront per token runs k rounds of a
//                          wave-wide argmax (ties to the lower expert id) and the softmax.
#include "common.h"

namespace moe {

RoutePlan route_plan(int T, int H, int E) {
  (void)E;
  RoutePlan p;
  p.TT = T <= 1 ? 1 : T <= 4 ? 4 : T <= 64 ? 8 : 16;
  int tiles = (T + p.TT - 1) / p.TT;
  int ks = (256 + tiles - 1) / tiles;  // aim for ~256 blocks
  int max_ks = H / 64;
  if (ks > max_ks) ks = max_ks;
  if (ks < 1) ks = 1;
  int kc = (H + ks - 1) / ks;
  kc = (kc + 63) / 64 * 64;
  p.kc = kc;
  p.KS = (H + kc - 1) / kc;
  return p;
}

// Block: 256 threads, thread e owns expert e (E <= 256).  Grid: (ceil(T/TT), KS).
// x[t][h] of the block's tokens is staged in LDS as fp32, 256 hidden values at a time.
template <int TT>
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             int T, int H, int E, int kc,
                                                             float* __restrict__ partial) {
  __shared__ float xs[TT][256];
  const int ks = blockIdx.y;
  const int t0 = blockIdx.x * TT;
  const int e = threadIdx.x;
  const int k_begin = ks * kc;
  const int k_end = min(H, k_begin + kc);
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) acc[t] = 0.f;
  for (int kb = k_begin; kb < k_end; kb += 256) {
    const int len = min(256, k_end - kb);
    __syncthreads();
    for (int i = threadIdx.x; i < TT * 256; i += 256) {
      const int t = i >> 8, h = i & 255;
      float v = 0.f;
      if (t0 + t < T && h < len) v = bf16_to_f32(x[(size_t)(t0 + t) * H + kb + h]);
      xs[t][h] = v;
    }
    __syncthreads();
    if (e < E) {
      const float* wp = wr + (size_t)kb * E + e;
#pragma unroll 4
      for (int h = 0; h < len; ++h) {
        const float w = wp[(size_t)h * E];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = fmaf(xs[t][h], w, acc[t]);
      }
    }
  }
  if (e < E) {
#pragma unroll
    for (int t = 0; t < TT; ++t)
      if (t0 + t < T) partial[((size_t)ks * T + t0 + t) * E + e] = acc[t];
  }
}

// Block: 256 threads = 4 wavefronts = 4 tokens.  Lane l holds experts l, l+64, l+128, l+192.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial,
                                                          int KS, const float* __restrict__ bias,
                                                          int T, int E, int k,
                                                          float* __restrict__ logits,
                                                          int32_t* __restrict__ topk_id,
                                                          float* __restrict__ topk_w) {
  __shared__ float selv[4][kMaxExperts];
  __shared__ int sele[4][kMaxExperts];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wv;
  if (t >= T) return;
  float v[4];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    ok[i] = e < E;
    float s = 0.f;
    if (ok[i]) {
      for (int q = 0; q < KS; ++q) s += partial[((size_t)q * T + t) * E + e];
      if (bias) s += bias[e];
      if (logits) logits[(size_t)t * E + e] = s;
    }
    v[i] = s;
  }
  for (int j = 0; j < k; ++j) {
    float bv = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (ok[i] && (be == 0x7fffffff || v[i] > bv)) {  // e ascends with i: ties keep the lower id
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      const bool take = (oe != 0x7fffffff) &&
                        (be == 0x7fffffff || ov > bv || (ov == bv && oe < be));
      if (take) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (be == lane + 64 * i) ok[i] = false;
    if (lane == 0) {
      selv[wv][j] = bv;
      sele[wv][j] = be;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  const float m = selv[wv][0];
  float den = 0.f;
  for (int j = 0; j < k; ++j) den += expf(selv[wv][j] - m);
  for (int j = lane; j < k; j += 64) {
    topk_id[(size_t)t * k + j] = sele[wv][j];
    topk_w[(size_t)t * k + j] = expf(selv[wv][j] - m) / den;
  }
}

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                        int E, int k, float* logits, int32_t* topk_id, float* topk_w,
                        float* partial, hipStream_t s) {
  const RoutePlan p = route_plan(T, H, E);
  dim3 g1((T + p.TT - 1) / p.TT, p.KS);
  switch (p.TT) {
    case 1: router_partial_kernel<1><<<g1, 256, 0, s>>>(x, wr, T, H, E, p.kc, partial); break;
    case 4: router_partial_kernel<4><<<g1, 256, 0, s>>>(x, wr, T, H, E, p.kc, partial); break;
    case 8: router_partial_kernel<8><<<g1, 256, 0, s>>>(x, wr, T, H, E, p.kc, partial); break;
    default: router_partial_kernel<16><<<g1, 256, 0, s>>>(x, wr, T, H, E, p.kc, partial); break;
  }
  router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(partial, p.KS, bias, T, E, k, logits, topk_id,
                                                 topk_w);
  return hipGetLastError();
}

}  // namespace moe
