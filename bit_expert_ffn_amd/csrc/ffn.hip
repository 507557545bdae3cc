// Expert FFN over NVFP4 weights: gate/up -> SwiGLU -> down for every routed row.
//
// Sources: per expert gate/up, SwiGLU, then down ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", section 8, "The fused MoE kernel and the pair exchange"); packed 4-bit
// weights are streamed and unpacked with their per-16 block scale in registers, never
// dequantised to HBM; a grouped GEMM runs over the active experts only ("Optimizing Models to
// Be Fast at Codegen", section 2 "Kernels optimized for latency or throughput"); a few-row
// expert fits in the same row tile as a single token (Muse Spark page, section 6).
//
// Matrix-core mapping (gfx950, v_mfma_f32_16x16x32_f16, 64-lane wavefronts):
//   one wavefront computes a 16 (rows) x 16 (features) tile over the full K.  K is walked in
//   chunks of 128.  Lane l = 16*g + n holds, for chunk c, weight row n's 32 values
//   K = [c*128 + g*32, +32): exactly one 16-byte load of packed codes plus two scale bytes.
//   Those 32 values feed four MFMAs (8 each).  The MFMA sums over its 32 k positions, so the
//   order of K inside the chunk is free; the A operand (activations) is read with the same
//   permutation: lane l = 16*g + m supplies row m's values [c*128 + g*32 + 8i, +8) to MFMA i.
// Decode: v_cvt_scalef32_pk_f16_fp4 turns one byte (two e2m1 codes) into two exact f16
//   values; the hardware uses only the exponent of its fp32 scale operand, so the e4m3 block
//   scale (converted to f16 by v_cvt_scalef32_pk_f16_fp8) is applied with one v_pk_mul_f16.
//   e2m1 * e4m3 needs at most 6 significant bits and lies in [2^-10, 2688], so the f16 weight
//   is exact.  The fp32 tensor scale multiplies the fp32 accumulator once.
// Activations: x (bf16) is converted once to f16 (exact for |x| in [2^-17, 65504]); h is
//   stored as f16.
#include "common.h"

namespace moe {

constexpr int kChunk = 128;         // K values per chunk
constexpr int kTileM = 16;          // rows per tile
constexpr int kWavesPerBlock = 4;   // one 16-feature tile per wavefront
constexpr int kFeatPerBlock = 16 * kWavesPerBlock;

__device__ inline f16x8 decode8(uint32_t q, f16x2 s) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * s;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// acc += A(16 x 128 chunk) * B(128 chunk x 16) for one chunk: 4 MFMAs.
__device__ inline f32x4 mma_chunk(f32x4 acc, const f16x8 a[4], uint4 q, uint32_t sbytes) {
  const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sbytes, 1.0f, false);
  const f16x2 s0 = {sc[0], sc[0]};
  const f16x2 s1 = {sc[1], sc[1]};
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], decode8(q.x, s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], decode8(q.y, s0), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[2], decode8(q.z, s1), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[3], decode8(q.w, s1), acc, 0, 0, 0);
  return acc;
}

__device__ inline void load_a(f16x8 a[4], const _Float16* p, bool valid) {
  if (valid) {
    const uint4* v = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(f16x8, v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

__device__ inline uint32_t load_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// x [T][H] bf16 -> f16, 8 values per thread.
__global__ __launch_bounds__(256) void x_to_f16_kernel(const uint16_t* __restrict__ x,
                                                       _Float16* __restrict__ x16, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  f16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (_Float16)__uint_as_float(w[j] << 16);
    o[2 * j + 1] = (_Float16)__uint_as_float(w[j] & 0xffff0000u);
  }
  reinterpret_cast<f16x8*>(x16)[i] = o;
}

// Gate/up + SwiGLU.  Grid: (I / 64, max active experts).  Block: 4 wavefronts, each one
// 16-feature tile of gate and of up for the same features, so h = silu(g) * u is formed in
// registers.  The block walks the expert's rows 16 at a time.
__global__ __launch_bounds__(256) void ffn_gateup_tile_kernel(
    const _Float16* __restrict__ x16, const uint8_t* __restrict__ gq,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ us, const float* __restrict__ ts,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ sorted_slot, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, int k, int H, int I, _Float16* __restrict__ h16) {
  const int slot = blockIdx.y;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int rows = count[e];
  const int base = offset[e];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int f0 = blockIdx.x * kFeatPerBlock + wv * 16;
  const size_t qrow = ((size_t)e * I + f0 + n);
  const uint8_t* gqp = gq + qrow * (H / 2) + g * 16;
  const uint8_t* uqp = uq + qrow * (H / 2) + g * 16;
  const uint8_t* gsp = gs + qrow * (H / 16) + g * 2;
  const uint8_t* usp = us + qrow * (H / 16) + g * 2;
  const float tsg = ts[e * 3 + 0], tsu = ts[e * 3 + 1];
  const int nchunk = H / kChunk;
  for (int m0 = 0; m0 < rows; m0 += kTileM) {
    const int ra = m0 + n;  // A row of this lane (m = lane & 15)
    const bool va = ra < rows;
    const int tok = va ? sorted_slot[base + ra] / k : 0;
    const _Float16* ap = x16 + (size_t)tok * H + g * 32;
    f32x4 accg = {0, 0, 0, 0}, accu = {0, 0, 0, 0};
    for (int c = 0; c < nchunk; ++c) {
      f16x8 a[4];
      load_a(a, ap + c * kChunk, va);
      const uint4 qg = *reinterpret_cast<const uint4*>(gqp + c * (kChunk / 2));
      const uint4 qu = *reinterpret_cast<const uint4*>(uqp + c * (kChunk / 2));
      const uint32_t sg = load_u16(gsp + c * (kChunk / 16));
      const uint32_t su = load_u16(usp + c * (kChunk / 16));
      accg = mma_chunk(accg, a, qg, sg);
      accu = mma_chunk(accu, a, qu, su);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + g * 4 + r;
      if (m < rows) {
        const float gv = accg[r] * tsg, uv = accu[r] * tsu;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        h16[(size_t)(base + m) * I + f0 + n] = (_Float16)hv;
      }
    }
  }
}

// Down projection.  Grid: (H / 64, max active experts).  A = h rows (grouped order, f16).
template <bool Y_F16>
__global__ __launch_bounds__(256) void ffn_down_tile_kernel(
    const _Float16* __restrict__ h16, const uint8_t* __restrict__ dq,
    const uint8_t* __restrict__ dsc, const float* __restrict__ ts,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int H, int I,
    void* __restrict__ y) {
  const int slot = blockIdx.y;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int rows = count[e];
  const int base = offset[e];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int f0 = blockIdx.x * kFeatPerBlock + wv * 16;
  const size_t qrow = ((size_t)e * H + f0 + n);
  const uint8_t* qp = dq + qrow * (I / 2) + g * 16;
  const uint8_t* sp = dsc + qrow * (I / 16) + g * 2;
  const float tsd = ts[e * 3 + 2];
  const int nchunk = I / kChunk;
  for (int m0 = 0; m0 < rows; m0 += kTileM) {
    const int ra = m0 + n;
    const bool va = ra < rows;
    const _Float16* ap = h16 + (size_t)(base + (va ? ra : 0)) * I + g * 32;
    f32x4 acc = {0, 0, 0, 0};
    for (int c = 0; c < nchunk; ++c) {
      f16x8 a[4];
      load_a(a, ap + c * kChunk, va);
      const uint4 q = *reinterpret_cast<const uint4*>(qp + c * (kChunk / 2));
      const uint32_t s = load_u16(sp + c * (kChunk / 16));
      acc = mma_chunk(acc, a, q, s);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + g * 4 + r;
      if (m < rows) {
        const float v = acc[r] * tsd;
        const size_t o = (size_t)(base + m) * H + f0 + n;
        if (Y_F16)
          reinterpret_cast<_Float16*>(y)[o] = (_Float16)v;
        else
          reinterpret_cast<float*>(y)[o] = v;
      }
    }
  }
}

hipError_t launch_ffn(const FfnArgs& a, hipStream_t s) {
  const int maxe = a.E < a.T * a.k ? a.E : a.T * a.k;
  const size_t n8 = (size_t)a.T * a.H / 8;
  x_to_f16_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(a.x, a.x16, n8);
  ffn_gateup_tile_kernel<<<dim3(a.I / kFeatPerBlock, maxe), 256, 0, s>>>(
      a.x16, a.gq, a.uq, a.gs, a.us, a.ts, a.count, a.offset, a.sorted_slot, a.active,
      a.n_active, a.k, a.H, a.I, a.h16);
  if (a.y_f16)
    ffn_down_tile_kernel<true><<<dim3(a.H / kFeatPerBlock, maxe), 256, 0, s>>>(
        a.h16, a.dq, a.ds, a.ts, a.count, a.offset, a.active, a.n_active, a.H, a.I, a.y);
  else
    ffn_down_tile_kernel<false><<<dim3(a.H / kFeatPerBlock, maxe), 256, 0, s>>>(
        a.h16, a.dq, a.ds, a.ts, a.count, a.offset, a.active, a.n_active, a.H, a.I, a.y);
  return hipGetLastError();
}

}  // namespace moe
