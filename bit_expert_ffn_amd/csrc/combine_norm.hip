// Combine variants: the routing-weighted sum of a token's expert outputs with
//   - a per-expert RMS norm of every expert output row before the weighted sum
//     ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", section 8, "The fused MoE
//     kernel and the pair exchange" and "A one-pass combine"), and/or
//   - an epilogue that applies the MoE output's own RMS factor s, adds the scaled residual
//     alpha * x + beta * s * f and RMS-normalises the result with a gain for the next layer
//     (same page, section 3, the residual stream of "What makes this possible is where Muse
//     Spark normalizes"; "A 501B sparse model gets day-one serving support": post-norm, scaled
//     residual and next pre-norm in one kernel).
// RMS norm of a row v: v / sqrt(mean(v^2) + eps).
//
// One block of 512 threads per token (1024 for hidden sizes above 32768, where registers
// spill); thread i owns the 4-feature groups i, i + NT, ... (G groups, features [4q, 4q + 4)
// of group q), so the block reads every row it needs once, coalesced.  Expert rows are loaded
// KC at a time into registers: their sums of squares are reduced over the block in one round
// (wavefront butterfly, then the wavefront totals through LDS, in a fixed order), and the same
// registers are then scaled into the fp32 accumulator, so y is read exactly once.  512-thread
// blocks keep three tokens resident per compute unit at hidden 7168.  The epilogue needs two
// more block reductions (f, then the new residual) and writes the residual (fp32) and the next
// input (bf16, round to nearest even) once each.
#include "common.h"

namespace moe {

namespace {


typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;

template <bool Y_F16>
struct RowVec;
template <>
struct RowVec<true> {
  typedef f16x4 type;
};
template <>
struct RowVec<false> {
  typedef f32x4 type;
};

typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// Buffer resource over `bytes` bytes at p: rows are addressed by a scalar base and a 32-bit
// per-lane offset, so no 64-bit address per load stays live in vector registers.  Every offset
// used here is in range (tail groups are clamped), so the hardware range check never applies.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ inline f16x4 load_vec(__amdgpu_buffer_rsrc_t r, uint32_t off, f16x4*) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ inline f32x4 load_vec(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4*) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ inline f32x4 to_f32(f16x4 v) { return __builtin_convertvector(v, f32x4); }
__device__ inline f32x4 to_f32(f32x4 v) { return v; }

// sum of squares of four values added to s (f16 pairs through the f32-accumulating dot)
__device__ inline float add_squares(f16x4 v, float s) {
  const f16x2 lo = {v.x, v.y}, hi = {v.z, v.w};
  s = __builtin_amdgcn_fdot2(lo, lo, s, false);
  return __builtin_amdgcn_fdot2(hi, hi, s, false);
}
__device__ inline float add_squares(f32x4 v, float s) {
  s = fmaf(v.x, v.x, s);
  s = fmaf(v.y, v.y, s);
  s = fmaf(v.z, v.z, s);
  return fmaf(v.w, v.w, s);
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
  return v;
}

// Sums v[0..N) over the block of NW wavefronts; every thread gets the totals.  Each wavefront
// reduces its own values (xor butterfly), lane 0 writes them to red; after the barrier lane l
// reads wavefront (l % NW)'s value and an NW-lane butterfly adds the wavefront totals.  Every
// lane ends with the same bits (xor butterflies add the same pairs on both sides).  red is
// [2][NW][N] floats, used alternately (phase toggles): a wavefront can only write a buffer
// again after passing the next reduction's barrier, which every reader of this one reaches
// only after reading.
template <int N, int NW>
__device__ inline void block_sum(float (&v)[N], float* red, int& phase) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float* buf = red + phase * (NW * N);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) buf[wave * N + i] = v[i];
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float s = buf[(lane & (NW - 1)) * N + i];
#pragma unroll
    for (int m = 1; m < NW; m <<= 1) s += __shfl_xor(s, m);
    v[i] = s;
  }
  phase ^= 1;
}

__device__ inline float rms_factor(float sum_sq, float inv_h, float eps) {
  return 1.0f / __builtin_sqrtf(sum_sq * inv_h + eps);
}

// Expert rows held in registers at a time: 16 groups of four f16 values, or 8 groups of four
// fp32 values (or of f16 values from G = 8 on), at most 8 rows, at least one.
constexpr int combine_norm_rows(bool f16, int G) {
  return (f16 && G < 8 ? 16 : 8) / G > 8 ? 8 : ((f16 && G < 8 ? 16 : 8) / G < 1 ? 1 : (f16 && G < 8 ? 16 : 8) / G);
}

}  // namespace

// NT threads per block (one token), G 4-feature groups per thread: H <= 4 NT G.
template <bool Y_F16, int G, int NT>
__global__ __launch_bounds__(NT) void combine_norm_kernel(CombineNormArgs a) {
  constexpr int NW = NT / 64;
  typedef typename RowVec<Y_F16>::type vec_t;
  constexpr int KC = combine_norm_rows(Y_F16, G);
  __shared__ float red[2 * NW * KC];
  const int t = blockIdx.x;
  const int H = a.H, k = a.k;
  const float inv_h = 1.0f / (float)H;
  const vec_t* y = reinterpret_cast<const vec_t*>(a.y);
  const int nq = H >> 2;  // groups per row
  const uint32_t vb = (uint32_t)sizeof(vec_t);
  int phase = 0;

  f32x4 acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A group past the row end (only in the last group of a row) reads a clamped in-range
  // offset and is zeroed; slots past k read the token's last row with weight zero.  So every
  // load is unconditional and all of a chunk's loads are in flight together.
  bool valid[G];
  uint32_t qi[G];  // group index (clamped)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int q = g * NT + threadIdx.x;
    valid[g] = q < nq;
    qi[g] = (uint32_t)(valid[g] ? q : nq - 1);
  }
  for (int j0 = 0; j0 < k; j0 += KC) {
    vec_t v[KC][G];
    float c[KC];
    __amdgpu_buffer_rsrc_t row[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int j = j0 + i < k ? j0 + i : k - 1;
      row[i] = rsrc(y + (size_t)a.slot_row[(size_t)t * k + j] * nq, (uint32_t)nq * vb);
      c[i] = j0 + i < k ? a.w[(size_t)t * k + j] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < KC; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) v[i][g] = load_vec(row[i], qi[g] * vb, (vec_t*)nullptr);
#pragma unroll
    for (int i = 0; i < KC; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) v[i][g] = valid[g] ? v[i][g] : vec_t{};
    if (a.expert_norm) {
      float ss[KC];
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        ss[i] = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) ss[i] = add_squares(v[i][g], ss[i]);
      }
      block_sum<KC, NW>(ss, red, phase);
#pragma unroll
      for (int i = 0; i < KC; ++i) c[i] *= rms_factor(ss[i], inv_h, a.eps);
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      if (j0 + i < k) {  // (slots past k add nothing; skipping keeps moe_combine's bits)
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const f32x4 f = to_f32(v[i][g]);
          acc[g].x = fmaf(c[i], f.x, acc[g].x);
          acc[g].y = fmaf(c[i], f.y, acc[g].y);
          acc[g].z = fmaf(c[i], f.z, acc[g].z);
          acc[g].w = fmaf(c[i], f.w, acc[g].w);
        }
      }
    }
  }

  // resid and out may be the same array (the residual stream updated in place): each thread
  // reads its own features of resid before it writes them.
  f32x4* out = reinterpret_cast<f32x4*>(a.out) + (size_t)t * nq;
  if (!a.epilogue) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (valid[g]) out[qi[g]] = acc[g];
    return;
  }
  float sf[1] = {0.f};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    sf[0] = fmaf(acc[g].x, acc[g].x, sf[0]);
    sf[0] = fmaf(acc[g].y, acc[g].y, sf[0]);
    sf[0] = fmaf(acc[g].z, acc[g].z, sf[0]);
    sf[0] = fmaf(acc[g].w, acc[g].w, sf[0]);
  }
  // for small G the residual and gain loads are issued before the reduction waits; the new
  // residual replaces f in acc
  const __amdgpu_buffer_rsrc_t resid = rsrc(a.resid + (size_t)t * H, (uint32_t)H * 4u);
  const __amdgpu_buffer_rsrc_t gain = rsrc(a.gain, (uint32_t)H * 4u);
  constexpr int NP = G <= 4 ? G : 1;
  f32x4 pre[NP], pgain[NP];
  if (G <= 4) {
#pragma unroll
    for (int g = 0; g < NP; ++g) {
      pre[g] = load_vec(resid, qi[g] * 16u, (f32x4*)nullptr);
      pgain[g] = load_vec(gain, qi[g] * 16u, (f32x4*)nullptr);
    }
  }
  block_sum<1, NW>(sf, red, phase);
  const float bs = a.beta * rms_factor(sf[0], inv_h, a.eps);
  float so[1] = {0.f};
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const f32x4 x =
        G <= 4 ? pre[g < NP ? g : 0] : load_vec(resid, qi[g] * 16u, (f32x4*)nullptr);
    f32x4 o;
    o.x = fmaf(bs, acc[g].x, a.alpha * x.x);
    o.y = fmaf(bs, acc[g].y, a.alpha * x.y);
    o.z = fmaf(bs, acc[g].z, a.alpha * x.z);
    o.w = fmaf(bs, acc[g].w, a.alpha * x.w);
    acc[g] = valid[g] ? o : f32x4{0.f, 0.f, 0.f, 0.f};
    so[0] = fmaf(acc[g].x, acc[g].x, so[0]);
    so[0] = fmaf(acc[g].y, acc[g].y, so[0]);
    so[0] = fmaf(acc[g].z, acc[g].z, so[0]);
    so[0] = fmaf(acc[g].w, acc[g].w, so[0]);
    if (valid[g]) out[qi[g]] = acc[g];
  }
  block_sum<1, NW>(so, red, phase);
  const float r = rms_factor(so[0], inv_h, a.eps);
  bf16x4_t* xn = reinterpret_cast<bf16x4_t*>(a.x_next) + (size_t)t * nq;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const f32x4 gv =
        G <= 4 ? pgain[g < NP ? g : 0] : load_vec(gain, qi[g] * 16u, (f32x4*)nullptr);
    if (valid[g]) xn[qi[g]] = __builtin_convertvector(gv * (acc[g] * r), bf16x4_t);
  }
}

// 512 threads per token up to H = 32768 (G = 1..16 groups per thread), 1024 above.
hipError_t launch_combine_norm(const CombineNormArgs& a, int y_f16, hipStream_t s) {
  int G = 1;
  while (G * 512 * 4 < a.H && G < 16) G <<= 1;
  const bool wide = a.H > 512 * 4 * 16;
  const dim3 grid((unsigned)a.T);
#define MOE_CN(F16_, G_, NT_) combine_norm_kernel<F16_, G_, NT_><<<grid, dim3(NT_), 0, s>>>(a)
#define MOE_CN_G(F16_)                 \
  if (wide) {                          \
    MOE_CN(F16_, 16, 1024);            \
  } else {                             \
    switch (G) {                       \
      case 1: MOE_CN(F16_, 1, 512); break; \
      case 2: MOE_CN(F16_, 2, 512); break; \
      case 4: MOE_CN(F16_, 4, 512); break; \
      case 8: MOE_CN(F16_, 8, 512); break; \
      default: MOE_CN(F16_, 16, 512); break; \
    }                                  \
  }
  if (y_f16) {
    MOE_CN_G(true)
  } else {
    MOE_CN_G(false)
  }
#undef MOE_CN_G
#undef MOE_CN
  return hipGetLastError();
}

}  // namespace moe
