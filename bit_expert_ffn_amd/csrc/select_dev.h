// Top-k selection keys (internal header): one 64-bit key per expert, so that "larger key" means
// a larger logit, or an equal logit and a lower expert id.
#pragma once
#include "common.h"

namespace moe {

// Selection key of a logit: larger key = larger logit, equal logits -> the lower expert id.  -0
// counts as +0 and NaN as -inf.  0 is below every key (an empty candidate).
__device__ inline uint64_t sel_key(float v, int id) {
  v = v == v ? v + 0.0f : -__builtin_inff();
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)id;
}
__device__ inline float sel_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}
__device__ inline int sel_id(uint64_t key) { return (int)~(uint32_t)key; }

}  // namespace moe
