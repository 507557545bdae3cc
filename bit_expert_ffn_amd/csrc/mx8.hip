// Low-precision variant of the expert FFN: fp8 compute with MXFP8 weights and activations on
// gfx950's scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// "Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU" serves its model with fp8 compute
// and NVFP4 expert weights (Figure 1); the MI355X form of that is OCP MX: e4m3 values with one
// power-of-two (e8m0) scale per 32 consecutive values, which the scaled MFMA applies itself.
//   - NVFP4 weights (e2m1 * e4m3 per 16 * fp32 tensor scale) are requantised to MXFP8 once, at
//     load time, in double precision (every dequantised weight is exact in double), into the
//     operand layout of the MFMA (below).
//   - x is quantised to MXFP8 per token row; h = silu(g) * u is quantised to MXFP8 in the
//     gate/up epilogue; y is written in f16.
// Quantiser (OCP MX v1.0): scale 2^E, E = floor(log2(amax)) - 8, clamped to [-127, 127]
// (amax = 0 gives E = -127 and zero codes); elements rounded to e4m3 to nearest, ties to even,
// saturated at 448.
//
// Operand layout of the scaled 32x32x64 fp8 MFMA (measured on gfx950): for a 64-wide K step,
// lane l (row or column l % 32, half hh = l / 32) holds 32 bytes: bytes 0..15 are K values
// 16 hh .. 16 hh + 15 and bytes 16..31 are K values 32 + 16 hh .. 32 + 16 hh + 15; its scale
// operand is the scale of the K block hh (values 32 hh .. 32 hh + 31) of its row.
//
// Weight layout (MX tile-major), per expert and matrix [N][K]: tiles of 32 rows x 64 K, each
// 2048 bytes with lane l's 32 bytes at 32 l, tiles ordered (row tile, K step); scales per row
// tile in groups of four K steps: 256 bytes, lane l's four scale bytes (steps 4g .. 4g + 3) at
// 4 l.  One 16-byte load pair and one dword per lane feed a whole MFMA operand.
#include "common.h"

namespace moe {

// ------------------------------------------------------------------------------------------------
// e4m3 (OCP E4M3FN) code of a double: nearest, ties to the even mantissa, saturated at 448; a
// negative value keeps its sign bit.
__device__ inline uint32_t e4m3_code_f64(double v) {
  const uint32_t sign = v < 0 ? 0x80u : 0u;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7Eu;
  if (a < 0x1p-6) return sign | (uint32_t)rint(a * 512.0);  // subnormals, step 2^-9
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  int m = (int)rint((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    ++e;
  }
  return sign | (uint32_t)((e + 7) << 3) | (uint32_t)m;
}

__device__ inline double e2m1_value(uint32_t c) {
  const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  return (c & 8u) ? -mag[c & 7u] : mag[c & 7u];
}

__device__ inline double e4m3_value(uint32_t c) {
  const int e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return (c & 0x80u) ? -v : v;
}

// MX shared exponent of a block's largest magnitude
__device__ inline int mx8_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  const int E = __builtin_amdgcn_frexp_expf(amax) - 1 - 8;  // frexp exponent - 1 = floor(log2)
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

// Four floats (already divided by the block scale) -> four e4m3 codes in one dword, by the
// hardware conversion (round to nearest even); values are clamped to +-448 first.
__device__ inline uint32_t e4m3_pack4(float a, float b, float c, float d) {
  auto cl = [](float v) { return fminf(fmaxf(v, -448.f), 448.f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true);
}

// ------------------------------------------------------------------------------------------------
// Load-time conversion: NVFP4 matrix (row-major codes [E][N][K/2], scales [E][N][K/16], tensor
// scales ts[e * 3 + tsi]) -> MXFP8 in the tile layout above.  One thread per 32-value block.
__global__ __launch_bounds__(256) void nvfp4_to_mx8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ s, const float* __restrict__ ts,
    int tsi, int E, int N, int K, uint8_t* __restrict__ q8, uint8_t* __restrict__ s8) {
  const size_t nblk = (size_t)E * N * (K / 32);
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  const int nb = K / 32;
  const size_t row = i / nb;
  const int b = (int)(i - row * nb);
  const int e = (int)(row / N), n = (int)(row - (size_t)e * N);
  const uint4 qv = *reinterpret_cast<const uint4*>(q + row * (K / 2) + 16 * b);
  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
  const double sc0 = e4m3_value(s[row * (K / 16) + 2 * b]);
  const double sc1 = e4m3_value(s[row * (K / 16) + 2 * b + 1]);
  const double t = (double)ts[(size_t)e * 3 + tsi];
  double w[32], amax = 0.0;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const uint32_t c = (qw[j >> 3] >> (4 * (j & 7))) & 15u;
    w[j] = e2m1_value(c) * (j < 16 ? sc0 : sc1) * t;
    amax = fmax(amax, fabs(w[j]));
  }
  int Ex = -127;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex);
    Ex = ex - 1 - 8;
    Ex = Ex < -127 ? -127 : (Ex > 127 ? 127 : Ex);
  }
  uint32_t cw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) cw[j] = 0;
  if (amax > 0.0) {
#pragma unroll
    for (int j = 0; j < 32; ++j) cw[j >> 2] |= e4m3_code_f64(ldexp(w[j], -Ex)) << (8 * (j & 3));
  }
  const int nst = K / 64, st = b >> 1, jb = b & 1;
  const size_t tile = (size_t)e * (N / 32) + n / 32;
  uint8_t* base = q8 + (tile * nst + st) * 2048;
  // values 0..15 -> lane n % 32, values 16..31 -> lane n % 32 + 32; bytes 16 jb .. 16 jb + 15
  *reinterpret_cast<uint4*>(base + (n % 32) * 32 + 16 * jb) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  *reinterpret_cast<uint4*>(base + (n % 32 + 32) * 32 + 16 * jb) =
      make_uint4(cw[4], cw[5], cw[6], cw[7]);
  s8[((tile * (nst / 4) + st / 4) * 64 + (n % 32) + 32 * jb) * 4 + (st & 3)] = (uint8_t)(Ex + 127);
}

hipError_t launch_nvfp4_to_mx8(const uint8_t* q, const uint8_t* s, const float* ts, int tsi,
                               int E, int N, int K, uint8_t* q8, uint8_t* s8, hipStream_t st) {
  const size_t nblk = (size_t)E * N * (K / 32);
  nvfp4_to_mx8_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, st>>>(q, s, ts, tsi, E, N, K,
                                                                        q8, s8);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------------
// x [T][H] bf16 -> MXFP8 (codes [T][H], scales [T][H/32]); one thread per 32-value block.  Block
// 0's first wavefront also lists the tiles of every active expert.
__global__ __launch_bounds__(256) void x_to_mx8_plan_kernel(
    const uint16_t* __restrict__ x, uint8_t* __restrict__ x8, uint8_t* __restrict__ xs,
    size_t nblk, const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int MT,
    int4* __restrict__ tiles, int max_tiles, int32_t* __restrict__ n_tiles) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < nblk) {
    const uint4* src = reinterpret_cast<const uint4*>(x) + i * 4;
    float v[32];
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint4 u = src[p];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * p + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * p + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const int E = mx8_exp(amax);
    uint32_t cw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      cw[j] = amax > 0.f ? e4m3_pack4(ldexpf(v[4 * j], -E), ldexpf(v[4 * j + 1], -E),
                                      ldexpf(v[4 * j + 2], -E), ldexpf(v[4 * j + 3], -E))
                         : 0u;
    uint4* dst = reinterpret_cast<uint4*>(x8) + i * 2;
    dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    xs[i] = (uint8_t)(E + 127);
  }
  if (blockIdx.x == 0 && threadIdx.x < 64)
    ffn_plan(count, offset, active, n_active, MT, 1, tiles, max_tiles, n_tiles);
}

// ------------------------------------------------------------------------------------------------
// Grouped GEMM over every active expert.  Block: NW wavefronts side by side in N, MT = 64 WM
// rows; each wavefront takes all MT rows against two 32-row weight tiles (gate/up: the gate and
// the up tile of the same 32 features; down: 64 consecutive output features).  K in steps of 64:
// the activation step (MT rows x 64 codes and two scale bytes per row) goes through LDS (double
// buffered); each lane loads its own weight bytes and scale dword.  Loads run one step ahead;
// a scheduling barrier after each step's products keeps the compiler from sinking them (and
// the LDS operands they hold live) towards the end of the unrolled loop.
template <bool GATEUP, int WM, int NW>
__global__ __launch_bounds__(64 * NW, 512 / (64 * NW)) void mx8_gemm_kernel(
    const uint8_t* __restrict__ a8, const uint8_t* __restrict__ as8,
    const uint8_t* __restrict__ q0, const uint8_t* __restrict__ s0,
    const uint8_t* __restrict__ q1, const uint8_t* __restrict__ s1,
    const int32_t* __restrict__ sorted_slot, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int k, int H, int I, void* __restrict__ out,
    uint8_t* __restrict__ hs_out) {
  constexpr int NTH = 64 * NW;
  constexpr int MT = 64 * WM;
  constexpr int MI = MT / 32;
  constexpr int LDA = 80;  // LDS row pitch in bytes (64 codes + padding)
  static_assert(MT * 4 == NTH, "one 16-byte activation piece per thread and step");
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  typedef __attribute__((ext_vector_type(8))) int i32x8;
  __shared__ __attribute__((aligned(16))) uint8_t As[2][MT][LDA];
  __shared__ __attribute__((aligned(4))) uint16_t Ass[2][NTH];  // entries >= MT unused

  // block order: as in the NVFP4 grouped GEMM (one contiguous range of the logical order per
  // XCD; experts one after another, in each the weight blocks, in each the expert's row tiles)
  const int NB = gridDim.x;
  const int ntl = *n_tiles;
  const int total = NB * ntl;
  const int bid = blockIdx.x + NB * blockIdx.y;
  if (bid >= total) return;
  int L;
  {
    constexpr int kX = 8;
    const int qx = bid % kX, loc = bid / kX;
    const int per = total / kX, rem = total % kX;
    L = qx * per + min(qx, rem) + loc;
  }
  const int4 td = tiles[L / NB];
  const int e = td.x, rows = td.z, base = td.w;
  const int ne = (rows + MT - 1) / MT;
  const int o = L - NB * td.y;
  const int fb = o / ne;
  const int m0 = (o - fb * ne) * MT;
  const int K = GATEUP ? H : I;
  const int N = GATEUP ? I : H;
  const int nst = K / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int r32 = lane & 31, hh = lane >> 5;

  // this thread's activation piece: row tid / 4 of the tile, bytes 16 (tid % 4) of each step;
  // rows past the expert's end repeat its last row (never stored)
  uint32_t aoff, soff;
  {
    const int r = min(m0 + (tid >> 2), rows - 1);
    const uint32_t src = GATEUP ? (uint32_t)(sorted_slot[base + r] / k) : (uint32_t)(base + r);
    aoff = src * (uint32_t)K + (uint32_t)(tid & 3) * 16u;
    const int rs = min(m0 + tid, rows - 1);  // scale row (threads tid >= MT: never read)
    const uint32_t srs = GATEUP ? (uint32_t)(sorted_slot[base + rs] / k) : (uint32_t)(base + rs);
    soff = srs * (uint32_t)(K / 32);
  }

  // this wavefront's two weight tiles (32-row tile indices, clamped to the matrix).  The lane
  // reads the operand bytes and scale dword of row pr of the tile (lane slot pr + 32 hh) rather
  // than row r32, so that, with the weights as the first MFMA operand, accumulator element v of
  // lane l is feature 16 (l / 32) + v of the tile: 16 consecutive features of one token row.
  const int pr = ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);
  const int slot = pr + 32 * hh;
  int feat[2];
  const uint8_t* qt[2];
  const uint8_t* stl[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row0 = GATEUP ? fb * (32 * NW) + wn * 32 : fb * (64 * NW) + wn * 64 + t * 32;
    feat[t] = row0;  // first feature of the tile
    const int tile = min(row0, N - 32) / 32;
    const size_t tix = (size_t)e * (N / 32) + tile;
    const uint8_t* qm = GATEUP && t == 1 ? q1 : q0;
    const uint8_t* sm = GATEUP && t == 1 ? s1 : s0;
    qt[t] = qm + tix * (size_t)nst * 2048 + slot * 32;
    stl[t] = sm + tix * (size_t)(nst / 4) * 256 + slot * 4;
  }

  struct Stage {
    u32x4 a;
    uint32_t as;
    u32x4 q[2][2];
    uint32_t sd[2];
  };
  auto load = [&](Stage& r, int st) __attribute__((always_inline)) {
    r.a = *reinterpret_cast<const u32x4*>(a8 + aoff + (uint32_t)st * 64u);
    r.as = *reinterpret_cast<const uint16_t*>(as8 + soff + 2u * (uint32_t)st);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint8_t* p = qt[t] + (size_t)st * 2048;
      r.q[t][0] = *reinterpret_cast<const u32x4*>(p);
      r.q[t][1] = *reinterpret_cast<const u32x4*>(p + 16);
      r.sd[t] = *reinterpret_cast<const uint32_t*>(stl[t] + (size_t)(st >> 2) * 256);
    }
  };
  auto store_a = [&](const Stage& r, int buf) __attribute__((always_inline)) {
    *reinterpret_cast<u32x4*>(&As[buf][tid >> 2][(tid & 3) * 16]) = r.a;
    Ass[buf][tid] = (uint16_t)r.as;
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][t][v] = 0.f;

  auto compute = [&](const Stage& r, int buf, auto jj_c) __attribute__((always_inline)) {
    constexpr int jj = decltype(jj_c)::value;  // step index modulo 4: byte of the scale dword
    i32x8 b[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
      b[t] = i32x8{(int)r.q[t][0].x, (int)r.q[t][0].y, (int)r.q[t][0].z, (int)r.q[t][0].w,
                   (int)r.q[t][1].x, (int)r.q[t][1].y, (int)r.q[t][1].z, (int)r.q[t][1].w};
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = i * 32 + r32;
      const u32x4 a0 = *reinterpret_cast<const u32x4*>(&As[buf][row][16 * hh]);
      const u32x4 a1 = *reinterpret_cast<const u32x4*>(&As[buf][row][32 + 16 * hh]);
      const i32x8 av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                        (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const int sa = (int)((Ass[buf][row] >> (8 * hh)) & 0xffu);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[t], av, acc[i][t], 0, 0, jj,
                                                                    (int)r.sd[t], 0, sa);
    }
  };

  // pipeline: two register sets, loads one step ahead; the step loop is unrolled by four (K is
  // a multiple of 256) so that the step index modulo 4, which selects the byte of the weight
  // scale dword, is a compile-time constant.  Loads past the last step re-read it (unused).
  Stage rs[2];
  const int last = nst - 1;
  // the prologue issues its loads in the loop's order (set 0, then set 1), so that the wait
  // counts the compiler derives at the loop head stay those of the steady state
  load(rs[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  load(rs[1], min(1, last));
  __builtin_amdgcn_sched_barrier(0);
  store_a(rs[0], 0);
  lds_barrier();
  // K >= 256 (checked by the caller): at least one pass, no guard branch for the compiler to
  // sink the prologue loads into
  int st = 0;
  do {
#define MOE_MX8_STEP(JJ)                                               \
    compute(rs[JJ & 1], JJ & 1, std::integral_constant<int, JJ>{});   \
    __builtin_amdgcn_sched_barrier(0);                                \
    store_a(rs[(JJ + 1) & 1], (JJ + 1) & 1);                          \
    load(rs[JJ & 1], min(st + JJ + 2, last));                         \
    lds_barrier();
    MOE_MX8_STEP(0)
    MOE_MX8_STEP(1)
    MOE_MX8_STEP(2)
    MOE_MX8_STEP(3)
#undef MOE_MX8_STEP
    st += 4;
  } while (st < nst);

  // epilogue.  The weights are the first operand and their rows are read in the order above:
  // lane l holds features 16 (l / 32) .. + 15 of its weight tile for token row l % 32 of each
  // 32-row sub-tile.
  if (GATEUP) {
    uint8_t* h8 = reinterpret_cast<uint8_t*>(out);
    const int f0 = feat[0];  // the gate tile and the up tile hold the same 32 features
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + i * 32 + r32;
      float hv[16], amax = 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float g = acc[i][0][v], u = acc[i][1][v];
        hv[v] = g / (1.0f + expf(-g)) * u;
        amax = fmaxf(amax, fabsf(hv[v]));
      }
      // the row's MXFP8 block: its 32 features, 16 in this lane and 16 in lane l ^ 32
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const int E = mx8_exp(amax);
      if (m < rows && f0 < N) {
        uint32_t w[4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          w[g4] = amax > 0.f ? e4m3_pack4(ldexpf(hv[4 * g4], -E), ldexpf(hv[4 * g4 + 1], -E),
                                          ldexpf(hv[4 * g4 + 2], -E), ldexpf(hv[4 * g4 + 3], -E))
                             : 0u;
        *reinterpret_cast<uint4*>(h8 + (size_t)(base + m) * I + f0 + hh * 16) =
            make_uint4(w[0], w[1], w[2], w[3]);
        if (hh == 0) hs_out[(size_t)(base + m) * (I / 32) + f0 / 32] = (uint8_t)(E + 127);
      }
    }
  } else {
    _Float16* y = reinterpret_cast<_Float16*>(out);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + i * 32 + r32;
      if (m >= rows) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int f0 = feat[t];
        if (f0 >= N) continue;  // N is a multiple of 32: a tile is wholly in or out
        f16x8 o[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) o[v >> 3][v & 7] = (_Float16)acc[i][t][v];
        f16x8* dst = reinterpret_cast<f16x8*>(y + (size_t)(base + m) * H + f0 + hh * 16);
        dst[0] = o[0];
        dst[1] = o[1];
      }
    }
  }
}

hipError_t launch_ffn_mx8(const Mx8Args& a, hipStream_t s) {
  const int MT = a.T >= 2048 ? 128 : 64;  // the kernel's tiles: 128 or 64 rows (max_tiles bounds both)
  const int max_tiles = (int)gemm_max_tiles(a.T, a.k, a.E);
  const size_t nblk = (size_t)a.T * a.H / 32;
  x_to_mx8_plan_kernel<<<(unsigned)((nblk + 255) / 256), 256, 0, s>>>(
      a.x, a.x8, a.xs, nblk, a.count, a.offset, a.active, a.n_active, MT, a.tiles, max_tiles,
      a.n_tiles);
#define MOE_MX8(GU_, WM_, A8_, AS_, Q0_, S0_, Q1_, S1_, OUT_, HS_)                             \
  do {                                                                                        \
    constexpr int NW_ = WM_ == 2 ? 8 : 4;                                                     \
    const dim3 g_(GU_ ? (a.I + 32 * NW_ - 1) / (32 * NW_) : (a.H + 64 * NW_ - 1) / (64 * NW_), \
                  max_tiles);                                                                 \
    mx8_gemm_kernel<GU_, WM_, NW_><<<g_, 64 * NW_, 0, s>>>(                                   \
        A8_, AS_, Q0_, S0_, Q1_, S1_, a.sorted_slot, a.tiles, a.n_tiles,                      \
        a.k, a.H, a.I, OUT_, HS_);                                                            \
  } while (0)
  if (MT == 128) {
    MOE_MX8(true, 2, a.x8, a.xs, a.gq, a.gs, a.uq, a.us, a.h8, a.hs);
    MOE_MX8(false, 2, a.h8, a.hs, a.dq, a.ds, a.dq, a.ds, a.y, nullptr);
  } else {
    MOE_MX8(true, 1, a.x8, a.xs, a.gq, a.gs, a.uq, a.us, a.h8, a.hs);
    MOE_MX8(false, 1, a.h8, a.hs, a.dq, a.ds, a.dq, a.ds, a.y, nullptr);
  }
#undef MOE_MX8
  return hipGetLastError();
}

}  // namespace moe
