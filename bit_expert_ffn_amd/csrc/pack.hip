// Layout conversion of NVFP4 expert matrices: row-major -> tile-major.
//
// Row-major (how quantised checkpoints store a matrix [N][K]): codes [N][K/2], scales [N][K/16].
// Tile-major (what the FFN kernels read): the matrix is cut into 16-row x 128-column tiles,
// tile (r, c) = rows 16r..16r+15, columns 128c..128c+127, tiles ordered r-major.  Inside a
// tile, "lane" l = 16*g + i (i = row within the tile, g = 32-column group) owns the 32 codes
// of row 16r+i, columns 128c+32g..+32 (16 bytes) and their two scale bytes.  A tile's codes are
// 64 lanes x 16 B = 1 KB contiguous and its scales 64 x 2 B = 128 B contiguous, so one
// wavefront load instruction reads exactly one tile, and lane l receives the operand that
// lane l of a 16x16x32 MFMA needs (column n = l % 16 of B, k-group l / 16).
//   codes:  byte ((r*(K/128) + c)*64 + l)*16 + (k%32)/2, low nibble = even k
//   scales: byte ((r*(K/128) + c)*64 + l)*2  + (k%32)/16
// Expert e's matrix starts at e*N*K/2 (codes) and e*N*K/16 (scales), as in row-major.
#include "common.h"

namespace moe {

// One thread per (expert, tile, lane).
__global__ __launch_bounds__(256) void nvfp4_pack_kernel(const uint8_t* __restrict__ q_in,
                                                         const uint8_t* __restrict__ s_in,
                                                         size_t nlanes, int N, int K,
                                                         uint8_t* __restrict__ q_out,
                                                         uint8_t* __restrict__ s_out) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nlanes) return;
  const int l = (int)(idx & 63);
  const size_t tile_all = idx >> 6;  // e * tiles_per_matrix + tile
  const size_t tiles = (size_t)(N / 16) * (K / 128);
  const size_t e = tile_all / tiles;
  const size_t t = tile_all - e * tiles;
  const int r = (int)(t / (K / 128)), c = (int)(t % (K / 128));
  const int i = l & 15, g = l >> 4;
  const size_t row = e * N + (size_t)r * 16 + i;
  const uint4 q = *reinterpret_cast<const uint4*>(q_in + row * (K / 2) + c * 64 + g * 16);
  const uint16_t s = *reinterpret_cast<const uint16_t*>(s_in + row * (K / 16) + c * 8 + g * 2);
  *reinterpret_cast<uint4*>(q_out + e * ((size_t)N * K / 2) + (t * 64 + l) * 16) = q;
  *reinterpret_cast<uint16_t*>(s_out + e * ((size_t)N * K / 16) + (t * 64 + l) * 2) = s;
}

hipError_t launch_pack(const uint8_t* q_in, const uint8_t* s_in, int E, int N, int K,
                       uint8_t* q_out, uint8_t* s_out, hipStream_t s) {
  const size_t nlanes = (size_t)E * (N / 16) * (K / 128) * 64;
  nvfp4_pack_kernel<<<(unsigned)((nlanes + 255) / 256), 256, 0, s>>>(q_in, s_in, nlanes, N, K,
                                                                      q_out, s_out);
  return hipGetLastError();
}

}  // namespace moe
