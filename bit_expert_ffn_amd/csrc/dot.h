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

__device__ inline uint32_t load_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// 8 values of one code dword dotted with 8 activations (4 pairs), accumulated into acc
__device__ inline float dot8_bf16(uint32_t q, uint4 xx, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0),
                                        __builtin_bit_cast(bf16x2_t, xx.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1),
                                        __builtin_bit_cast(bf16x2_t, xx.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2),
                                        __builtin_bit_cast(bf16x2_t, xx.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3),
                                        __builtin_bit_cast(bf16x2_t, xx.w), acc, false);
  return acc;
}

__device__ inline float dot8_f16(uint32_t q, uint4 xx, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0),
                               __builtin_bit_cast(f16x2, xx.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1),
                               __builtin_bit_cast(f16x2, xx.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2),
                               __builtin_bit_cast(f16x2, xx.z), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3),
                               __builtin_bit_cast(f16x2, xx.w), acc, false);
  return acc;
}

// A lane's 32 values (two 16-value scale blocks): each block's dot times its e4m3 scale.
__device__ inline float dot32_bf16(uint4 q, uint32_t sbytes, const uint4* xv) {
  const float b0 = dot8_bf16(q.y, xv[1], dot8_bf16(q.x, xv[0], 0.f));
  const float b1 = dot8_bf16(q.w, xv[3], dot8_bf16(q.z, xv[2], 0.f));
  return b0 * __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 0) +
         b1 * __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 1);
}

__device__ inline float dot32_f16(uint4 q, uint32_t sbytes, const uint4* xv) {
  const float b0 = dot8_f16(q.y, xv[1], dot8_f16(q.x, xv[0], 0.f));
  const float b1 = dot8_f16(q.w, xv[3], dot8_f16(q.z, xv[2], 0.f));
  return b0 * __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 0) +
         b1 * __builtin_amdgcn_cvt_f32_fp8((int)sbytes, 1);
}

// the four K-groups of feature n (lanes n, n+16, n+32, n+48), fixed order
__device__ inline float sum_groups(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace moe
