// NVFP4 dot-product helpers shared by the VALU expert kernels (internal).
//
// Tile-major layout: a 16-row x 128-column tile of an expert matrix is 1024 bytes of e2m1 codes
// and 128 bytes of e4m3 scales; lane l = 16 g + n of a wavefront holds row n's 32 codes of
// columns [32 g, 32 g + 32) of the chunk (16 bytes) and their two scale bytes.
// v_cvt_scalef32_pk_{bf16,f16}_fp4 turns one byte (two e2m1 codes) into two exact 16-bit
// values; each 16-value block's dot product is multiplied by its e4m3 scale in fp32.
#pragma once
#include "common.h"

namespace moe {

constexpr int kChunk = 128;  // K values per chunk (one tile-major column block)

// Lane l's two scale bytes are bytes 2 l and 2 l + 1 of a 128-byte scale block.  They are
// loaded as the aligned dword that holds them (p = block + 4 (l / 2); lanes 2 i and 2 i + 1 read
// the same dword) and taken out at the use with scale_pair().  A 16-bit load leaves the compiler
// a value to zero-extend, and where it placed that at a loop back edge or where two paths join,
// the wavefront waited there for the whole load set it had just issued.  One instruction reads
// the whole 128-byte block and nothing reads it again, so the load is non-temporal like the codes
// (measured at decode: 46.2 -> 46.0 us; the grouped GEMM, whose scale blocks serve two stages,
// keeps cached scale loads: non-temporal ones cost it 3.7% at T = 64 and 5% at T = 128).
__device__ inline uint32_t load_scale_dword(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ inline uint32_t scale_pair(uint32_t w, int lane) { return w >> ((lane & 1) * 16); }

// 16 bytes of weights that the kernel reads once: a non-temporal load, so that the streamed
// expert weights do not displace reused lines from the caches (measured: the few-row expert
// kernels at T = 64 stream 3.4% faster, the single-launch layer at T = 1 3.1%; the grouped GEMMs,
// whose weight slices are shared through L2 by an expert's row tiles, run slower with it).
__device__ inline uint4 load_stream16(const uint8_t* p) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// A lane's 32 weights decoded once (two 16-value scale blocks) and then dotted with any number
// of activation rows: each block's dot times its e4m3 scale.
struct Dec32bf {
  bf16x2_t v[16];
  float s0, s1;
};
struct Dec32h {
  f16x2 v[16];
  float s0, s1;
};

__device__ inline void decode32(uint4 q, uint32_t sbytes, Dec32bf& d) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d.v[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 0);
    d.v[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 1);
    d.v[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 2);
    d.v[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 3);
  }
  d.s0 = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 0);
  d.s1 = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 1);
}

__device__ inline void decode32(uint4 q, uint32_t sbytes, Dec32h& d) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d.v[4 * i + 0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0);
    d.v[4 * i + 1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1);
    d.v[4 * i + 2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2);
    d.v[4 * i + 3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3);
  }
  d.s0 = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 0);
  d.s1 = __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 1);
}

// xv: the 32 matching activations (four 16-byte pieces), in the order of the decoded values
__device__ inline float dot32(const Dec32bf& d, const uint4* xv) {
  float b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x0[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
    const uint32_t x1[4] = {xv[i + 2].x, xv[i + 2].y, xv[i + 2].z, xv[i + 2].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0 = __builtin_amdgcn_fdot2_f32_bf16(d.v[4 * i + j], __builtin_bit_cast(bf16x2_t, x0[j]),
                                           b0, false);
      b1 = __builtin_amdgcn_fdot2_f32_bf16(d.v[8 + 4 * i + j],
                                           __builtin_bit_cast(bf16x2_t, x1[j]), b1, false);
    }
  }
  return b0 * d.s0 + b1 * d.s1;
}

__device__ inline float dot32(const Dec32h& d, const uint4* xv) {
  float b0 = 0.f, b1 = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x0[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
    const uint32_t x1[4] = {xv[i + 2].x, xv[i + 2].y, xv[i + 2].z, xv[i + 2].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b0 = __builtin_amdgcn_fdot2(d.v[4 * i + j], __builtin_bit_cast(f16x2, x0[j]), b0, false);
      b1 = __builtin_amdgcn_fdot2(d.v[8 + 4 * i + j], __builtin_bit_cast(f16x2, x1[j]), b1, false);
    }
  }
  return b0 * d.s0 + b1 * d.s1;
}

// the four K-groups of feature n (lanes n, n+16, n+32, n+48), fixed order
__device__ inline float sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace moe
