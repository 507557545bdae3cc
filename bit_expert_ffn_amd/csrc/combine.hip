// Routing-weighted combine: out[t][n] = sum_{j<k} w[t][j] * y[slot_row[t*k+j]][n] in fp32.
// One pass that reads each expert output once and writes every output row exactly once, with
// no zero fill ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", section 8,
// "A one-pass combine" and "No zero fill, unrolled writes").
// Grid: T * ceil(H / 1024) blocks; each thread owns 4 consecutive features of one token.
#include "common.h"

namespace moe {

template <bool Y_F16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w, int k, int H,
                                                      int nhb, float* __restrict__ out) {
  const int t = blockIdx.x / nhb;
  const int h = ((blockIdx.x % nhb) * 256 + threadIdx.x) * 4;
  if (h >= H) return;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const size_t r = (size_t)slot_row[(size_t)t * k + j];
    const float wj = w[(size_t)t * k + j];
    float4 v;
    if (Y_F16) {
      const f16x4 hv = *reinterpret_cast<const f16x4*>(reinterpret_cast<const _Float16*>(y) + r * H + h);
      v = {(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
    } else {
      v = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + r * H + h);
    }
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  *reinterpret_cast<float4*>(out + (size_t)t * H + h) = acc;
}

hipError_t launch_combine(const void* y, int y_f16, const int32_t* slot_row, const float* w,
                          int T, int k, int H, float* out, hipStream_t s) {
  const int nhb = (H + 1023) / 1024;
  const unsigned grid = (unsigned)T * (unsigned)nhb;
  if (y_f16)
    combine_kernel<true><<<grid, 256, 0, s>>>(y, slot_row, w, k, H, nhb, out);
  else
    combine_kernel<false><<<grid, 256, 0, s>>>(y, slot_row, w, k, H, nhb, out);
  return hipGetLastError();
}

}  // namespace moe
