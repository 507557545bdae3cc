// Grouped GEMM over the busy experts: gate/up (+ SwiGLU) and down on the matrix cores.
//
// Sources: per expert gate/up, SwiGLU, then down; one expert's weights are streamed while the
// rows routed to it are multiplied ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU",
// section 8, "The fused MoE kernel and the pair exchange"); a dequantize-then-multiply path for
// busier experts (same page, section 5); a grouped GEMM over the active experts only, with the
// 4-bit weights unpacked on chip and never written back dequantised ("Optimizing Models to Be
// Fast at Codegen", section 2).
//
// Work list: ffn_plan (a one-wavefront kernel launched before the GEMMs) walks the
// active experts in order and lists every tile of MT rows of every expert with at least
// min_rows rows, each with its expert's descriptor (expert, first tile, rows, first row).  grid.y runs over a host-side bound of that list; blocks
// past its end return.  Nothing is read back by the host.
//
// Arithmetic: activations (x, converted from bf16 on its way into LDS, or h) and decoded weights
// enter v_mfma_f32_32x32x16_f16 as f16;
// e2m1 * e4m3 is exact in f16 (at most 6 significant bits, magnitude in [2^-10, 2688]); the
// fp32 tensor scales multiply the fp32 accumulators in the epilogue.
#include "common.h"

namespace moe {

constexpr int gK = 64;       // K per pipeline stage
constexpr int gLD = gK + 8;  // padded LDS row, in halves
constexpr int kXcds = 8;     // MI355X: 8 accelerator dies (XCDs), workgroups dealt round-robin
constexpr int kGemmSets = 4;  // register sets of the load pipeline

__device__ inline f16x8 gdecode8(uint32_t q, f16x2 s) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * s;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// x [T][H] bf16 -> f16 (8 values per thread, for 128-row tiles); block 0's first wavefront also
// builds the tile list of the busy experts.
__global__ __launch_bounds__(256) void x_to_f16_plan_kernel(
    const uint16_t* __restrict__ x, _Float16* __restrict__ x16, size_t n8,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int MT,
    int min_rows, int4* __restrict__ tiles, int max_tiles, int32_t* __restrict__ n_tiles) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n8) {
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
  if (blockIdx.x == 0 && threadIdx.x < 64)
    ffn_plan(count, offset, active, n_active, MT, min_rows, tiles, max_tiles, n_tiles);
}

// The tile list of the busy experts alone (one wavefront; smaller tiles, whose GEMM converts x).
__global__ __launch_bounds__(64) void ffn_plan_kernel(
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int MT,
    int min_rows, int4* __restrict__ tiles, int max_tiles, int32_t* __restrict__ n_tiles) {
  ffn_plan(count, offset, active, n_active, MT, min_rows, tiles, max_tiles, n_tiles);
}

// Block: NW wavefronts side by side in N; MT rows x 64 NW weight rows; K in stages of
// 64.  Every wavefront computes all MT rows (MI = MT / 32 tiles of 32) against its own 2 weight
// tiles of 32 rows:
//   gate/up: wavefront wn takes features f0 + 32 wn .. + 31 of the block's 32 NW: its gate tile
//            and the up tile of the same features; h = silu(g) * u in the epilogue;
//   down:    rows n0 + 64 wn + {0, 32} -> 64 NW output features per block.
// Wider blocks read each activation tile fewer times (once per block of weight rows).
// Each weight byte is loaded and decoded by one wavefront only, and each decoded fragment feeds
// MI MFMAs.  Activations go through LDS (double buffered, rows padded to 144 bytes) and every
// wavefront reads all of them.  Weights do not: each lane loads, per stage and per weight
// tile, the 16 packed bytes (32 codes) of weight row l % 32 and K-group 2 (st % 2) + l / 32 of
// the stage's 128-column chunk, plus its two scale bytes, and decodes one code dword right
// before each of the stage's four 16-K MFMA steps.  The MFMA sums over its 16 k positions, so
// K may be permuted: step i takes codes 8i..8i+7 of the lane's group, and the activation
// operand is read from LDS columns 32 (l / 32) + 8i of the stage (same permutation).  Global
// loads of activations and packed weights run ahead in S register sets.
// The launch bound's second argument is the minimum number of wavefronts per SIMD: two (up to
// 256 VGPRs) below 8 wavefronts per block, one with 8 (whose 512 threads give two per SIMD).
template <bool GATEUP, int MTT, bool Y_F16, int S, int NW, bool XBF>
__global__ __launch_bounds__(64 * NW, NW >= 8 ? 1 : 2) void ffn_gemm_kernel(
    const uint16_t* __restrict__ xa, const uint8_t* __restrict__ qm0,
    const uint8_t* __restrict__ sm0, const uint8_t* __restrict__ qm1,
    const uint8_t* __restrict__ sm1, const float* __restrict__ ts,
    const int32_t* __restrict__ sorted_slot, const int4* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int k, int H, int I, void* __restrict__ out) {
  constexpr int NTH = 64 * NW;      // threads per block
  constexpr int MT = MTT;
  constexpr int MI = MT / 32;        // 32-row tiles per wavefront
  constexpr int NA = MT * 8 / NTH;   // 16-byte activation pieces per thread per stage
  static_assert(NA >= 1, "block tile too small for its threads");
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // native vector: stays in VGPRs
  __shared__ __attribute__((aligned(16))) _Float16 As[2][MT][gLD];
  // Block order.  Workgroups go round-robin to the 8 XCDs, each with its own L2; renumber so
  // that every XCD gets one contiguous range of the logical order.  The logical order takes
  // the experts one after another (their tiles are consecutive in the list) and, inside an
  // expert, the weight blocks one after another and for each the expert's row tiles: the
  // blocks that run together on an XCD are the row tiles of one expert against the same
  // weight slice, which is then read from HBM about once.
  const int NB = gridDim.x;  // weight blocks
  const int ntl = *n_tiles;
  const int total = NB * ntl;
  const int bid = blockIdx.x + NB * blockIdx.y;
  if (bid >= total) return;
  int L;
  {
    const int q = bid % kXcds, loc = bid / kXcds;
    const int per = total / kXcds, rem = total % kXcds;
    L = q * per + min(q, rem) + loc;
  }
  // expert e owns items [NB j0, NB (j0 + ne)), so tile L / NB is one of its tiles
  const int4 td = tiles[L / NB];
  const int e = td.x, rows = td.z, base = td.w;
  const int ne = (rows + MT - 1) / MT;
  const int o = L - NB * td.y;
  const int fb = o / ne;
  const int m0 = (o - fb * ne) * MT;
  const int K = GATEUP ? H : I;  // reduction length
  const int N = GATEUP ? I : H;  // rows of one weight matrix
  const int nchunk = K / 128;
  const int nstage = K / gK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  // activation rows of this thread's pieces (rows past the expert's end repeat its last row, or
  // are zero on 32-row tiles: their outputs are never stored).  Offsets are 32-bit element offsets from a uniform base
  // (x and h are far below 2^32 elements), which keeps the per-lane state small.
  uint32_t aoff[NA];
  bool alive[NA];  // the piece's row is one of the expert's rows
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int sidx = tid + NTH * i;
    alive[i] = m0 + (sidx >> 3) < rows;
    const int r = min(m0 + (sidx >> 3), rows - 1);
    const uint32_t src = GATEUP ? (uint32_t)(sorted_slot[base + r] / k) * (uint32_t)H
                                : (uint32_t)(base + r) * (uint32_t)I;
    aoff[i] = src + (uint32_t)(sidx & 7) * 8;
  }

  // weight rows of this lane in its 2 weight tiles; rows past N (only possible in the last
  // block of down when H % 256 != 0) re-read row N - 1 and are never stored.  Byte offsets
  // within the expert's matrix (< 2^32) from uniform bases.
  const int r32 = lane & 31, hgrp = lane >> 5;
  const uint8_t* qb0 = qm0 + (size_t)e * ((size_t)N * K / 2);
  const uint8_t* sb0 = sm0 + (size_t)e * ((size_t)N * K / 16);
  const uint8_t* qb1 = GATEUP ? qm1 + (size_t)e * ((size_t)N * K / 2) : qb0;
  const uint8_t* sb1 = GATEUP ? sm1 + (size_t)e * ((size_t)N * K / 16) : sb0;
  // The lane loads weight row pr of its 32-row tile rather than row r32, chosen so that, with
  // the weights as the first MFMA operand, accumulator element v of lane l is feature
  // 16 (l / 32) + v of the tile: each lane then holds 16 consecutive features of one token row
  // (pr has the parity of r32, so the scale byte sits in the same half of its dword).
  const int pr = ((r32 >> 2) & 1) * 16 + (r32 >> 3) * 4 + (r32 & 3);
  uint32_t qoff[2], soff[2];
  int feat[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row0 = GATEUP ? fb * (32 * NW) + wn * 32 : fb * (64 * NW) + wn * 64 + t * 32;
    const int row = row0 + pr;
    feat[t] = row0;  // first feature of the tile
    const int rc = min(row, N - 1);
    const uint32_t tile0 = (uint32_t)(rc >> 4) * (uint32_t)nchunk;
    qoff[t] = tile0 * 1024u + (uint32_t)(rc & 15) * 16u + (uint32_t)hgrp * 256u;
    soff[t] = tile0 * 128u + (uint32_t)(rc & 15) * 2u + (uint32_t)hgrp * 32u;
  }
  const uint8_t* qbt1 = GATEUP ? qb1 : qb0;  // tile 1: the up matrix (gate/up) or down again
  const uint8_t* sbt1 = GATEUP ? sb1 : sb0;

  struct Stage {
    u32x4 a[NA];
    u32x4 q0, q1;
    uint32_t s0, s1;
  };
  auto load = [&](Stage& r, int st) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)st * gK;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      // 32-row tiles (small batches, where most experts have a few rows): rows past the
      // expert's end are not loaded but zero, which spares the load path the repeated last row
      // (measured at T = 64: layer 951 -> 906 us; at T = 128 with I = 256 no change).  Larger
      // tiles load the repeated row (with the skip, the prefill expert FFN measured 10.31 ->
      // 10.74 ms: few of its rows are past an expert's end)
      if (MT == 32)
        r.a[i] = alive[i] ? *reinterpret_cast<const u32x4*>(xa + (aoff[i] + k0)) : u32x4{0, 0, 0, 0};
      else
        r.a[i] = *reinterpret_cast<const u32x4*>(xa + (aoff[i] + k0));
    }
    // tile-lane of this lane's K-group in the stage's chunk: 16 * g + row % 16, where
    // g = 2 (st % 2) + lane / 32 (the lane / 32 part is already in qoff / soff)
    const uint32_t cq = (uint32_t)(st >> 1) * 1024u + (uint32_t)(st & 1) * 512u;
    const uint32_t cs = (uint32_t)(st >> 1) * 128u + (uint32_t)(st & 1) * 64u;
    // 32-row tiles (small batches): an expert has one or two tiles, so its weights are read
    // about once: non-temporal loads.  Larger tiles share weight slices through L2.
    if (MT == 32) {
      r.q0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qb0 + (qoff[0] + cq)));
      r.q1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qbt1 + (qoff[1] + cq)));
    } else {
      r.q0 = *reinterpret_cast<const u32x4*>(qb0 + (qoff[0] + cq));
      r.q1 = *reinterpret_cast<const u32x4*>(qbt1 + (qoff[1] + cq));
    }
    // the lane's two scale bytes sit in the low (even row) or high (odd row) half of an aligned
    // dword; loading the whole dword keeps the value free of any zero-extension, which the
    // compiler would otherwise place right after the load (in the previous step) and so wait
    // for every load in flight
    r.s0 = *reinterpret_cast<const uint32_t*>(sb0 + ((soff[0] + cs) & ~3u));
    r.s1 = *reinterpret_cast<const uint32_t*>(sbt1 + ((soff[1] + cs) & ~3u));
  };
  auto store_a = [&](const Stage& r, int buf) __attribute__((always_inline)) {
    // piece i of this thread: s = tid + NTH * i -> row s >> 3, 16-byte column s & 7.  With XBF
    // (gate/up on 32- and 64-row tiles) the activations are bf16 x, converted here (round to
    // nearest even, as a bf16 -> f16 cast does); 128-row tiles read x converted once by
    // x_to_f16_plan_kernel, since every weight block of a tile would otherwise convert it again
    const int c8 = (tid & 7) * 8;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      u32x4 v = r.a[i];
      if (XBF) {
        f16x8 hv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hv[2 * j] = (_Float16)__uint_as_float(v[j] << 16);
          hv[2 * j + 1] = (_Float16)__uint_as_float(v[j] & 0xffff0000u);
        }
        v = __builtin_bit_cast(u32x4, hv);
      }
      *reinterpret_cast<u32x4*>(&As[buf][(tid >> 3) + (NTH / 8) * i][c8]) = v;
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][t][v] = 0.f;
  const bool odd_row = (r32 & 1) != 0;  // which half of the scale dword is this lane's
  auto bfrag = [&](u32x4 q, uint32_t sdword, int step) __attribute__((always_inline)) {
    const f16x2 sc = odd_row ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sdword, 1.0f, true)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sdword, 1.0f, false);
    const f16x2 sv = step < 2 ? f16x2{sc[0], sc[0]} : f16x2{sc[1], sc[1]};
    return gdecode8(q[step], sv);
  };
  auto compute = [&](const Stage& r, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const f16x8 b0 = bfrag(r.q0, r.s0, step);
      const f16x8 b1 = bfrag(r.q1, r.s1, step);
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(&As[buf][i * 32 + r32][hgrp * 32 + step * 8]);
        // weights first: the accumulator holds the transposed tile (see the epilogue)
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, a, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, a, acc[i][1], 0, 0, 0);
      }
    }
  };

  // pipeline over S register sets.  Set j holds stage s = st + j: its weights feed compute,
  // and right after it the set is refilled with stage s + S; the activations of stage s + 1
  // (loaded S - 1 steps earlier) go to the other LDS buffer, so loads run S - 1 stages ahead.
  // The main loop covers the largest multiple of S stages with no conditions in its body.  Its
  // last round skips the refills past the last stage (uniform conditions): a load left in
  // flight would be waited for before the epilogue reuses its registers, a memory latency per
  // block.  The host picks S so that the stage count is a multiple of it where it can: with
  // stages left after that round, the conditional refills make the compiler wait for every load
  // before each remaining stage.  64-row tiles re-read the last stage instead (the second copy
  // of the round would make their gate/up spill).  The remaining stages (fewer than S) follow,
  // each guarded by a uniform condition.
  Stage r[S];
  const int last = nstage - 1;
  const int nmain = nstage - nstage % S;
#pragma unroll
  for (int jj = 0; jj < S; ++jj) load(r[jj], min(jj, last));
  store_a(r[0], 0);
  lds_barrier();
  if constexpr (MT != 64) {
    int st = 0;
    for (; st + S < nmain; st += S) {
#pragma unroll
      for (int jj = 0; jj < S; ++jj) {
        compute(r[jj], (st + jj) & 1);
        store_a(r[(jj + 1) % S], (st + jj + 1) & 1);
        load(r[jj], st + jj + S);
        lds_barrier();
      }
    }
    if (st < nmain) {
#pragma unroll
      for (int jj = 0; jj < S; ++jj) {
        compute(r[jj], (st + jj) & 1);
        store_a(r[(jj + 1) % S], (st + jj + 1) & 1);
        if (st + jj + S < nstage) load(r[jj], st + jj + S);
        lds_barrier();
      }
    }
  } else {
    for (int st = 0; st < nmain; st += S) {
#pragma unroll
      for (int jj = 0; jj < S; ++jj) {
        compute(r[jj], (st + jj) & 1);
        store_a(r[(jj + 1) % S], (st + jj + 1) & 1);
        load(r[jj], min(st + jj + S, last));
        lds_barrier();
      }
    }
  }
#pragma unroll
  for (int jj = 0; jj < S - 1; ++jj) {
    if (nmain + jj < nstage) {
      compute(r[jj], (nmain + jj) & 1);
      store_a(r[(jj + 1) % S], (nmain + jj + 1) & 1);
      lds_barrier();
    }
  }

  // epilogue.  With the weights as the first operand and the row order above, lane l holds
  // features 16 (l / 32) .. + 15 of its weight tile for token row l % 32 of each 32-row
  // sub-tile: two 16-byte (f16) or four 16-byte (fp32) stores per row and tile.
  if (GATEUP) {
    const float tsg = ts[e * 3 + 0], tsu = ts[e * 3 + 1];
    _Float16* h16 = reinterpret_cast<_Float16*>(out);
    const int f0 = feat[0];  // first feature of the gate tile (= of the up tile)
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + i * 32 + r32;
      if (m < rows && f0 < I) {
        f16x8 o[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float gv = acc[i][0][v] * tsg, uv = acc[i][1][v] * tsu;
          o[v >> 3][v & 7] = (_Float16)(gv / (1.0f + expf(-gv)) * uv);
        }
        f16x8* dst = reinterpret_cast<f16x8*>(h16 + (size_t)(base + m) * I + f0 + hgrp * 16);
        dst[0] = o[0];
        dst[1] = o[1];
      }
    }
  } else {
    const float tsd = ts[e * 3 + 2];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = m0 + i * 32 + r32;
      if (m >= rows) continue;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int f0 = feat[t];
        if (f0 >= N) continue;  // N is a multiple of 32: a tile is wholly in or out
        const size_t o = (size_t)(base + m) * H + f0 + hgrp * 16;
        if (Y_F16) {
          f16x8 v8[2];
#pragma unroll
          for (int v = 0; v < 16; ++v) v8[v >> 3][v & 7] = (_Float16)(acc[i][t][v] * tsd);
          f16x8* dst = reinterpret_cast<f16x8*>(reinterpret_cast<_Float16*>(out) + o);
          dst[0] = v8[0];
          dst[1] = v8[1];
        } else {
          f32x4* dst = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + o);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dst[q] = f32x4{acc[i][t][4 * q] * tsd, acc[i][t][4 * q + 1] * tsd,
                           acc[i][t][4 * q + 2] * tsd, acc[i][t][4 * q + 3] * tsd};
        }
      }
    }
  }
}

// rows of a grouped-GEMM tile (the f16 path)
int gemm_rows_per_tile(int T) { return T >= 2048 ? 128 : T >= 512 ? 64 : 32; }

size_t gemm_max_tiles(int T, int k, int E) {
  const int MT = gemm_rows_per_tile(T);
  const size_t n = (size_t)T * k;
  const size_t ne = (size_t)(E < (int)n ? E : (int)n);
  return n / MT + 1 + ne;
}

hipError_t launch_ffn_gemm(const FfnArgs& a, int min_rows, int4* tiles, int32_t* n_tiles,
                           hipStream_t s) {
  const int MT = gemm_rows_per_tile(a.T);
  const int max_tiles = (int)gemm_max_tiles(a.T, a.k, a.E);
  if (MT == 128) {
    const size_t n8 = (size_t)a.T * a.H / 8;
    x_to_f16_plan_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(
        a.x, a.x16, n8, a.count, a.offset, a.active, a.n_active, MT, min_rows, tiles, max_tiles,
        n_tiles);
  } else if (!a.planned) {
    ffn_plan_kernel<<<1, 64, 0, s>>>(a.count, a.offset, a.active, a.n_active, MT, min_rows, tiles,
                                     max_tiles, n_tiles);
  }
  // 128-row tiles from 2048 tokens: 8 wavefronts (512 weight rows per block); 64-row tiles from
  // 512 tokens and 32-row tiles below, on 4 wavefronts: most experts of a small batch have a
  // few rows, and a smaller tile wastes fewer matrix-core cycles on rows past the expert's end
  // (measured at T = 128: 130 against 153 us; at T = 64: 954 against 965 us).  The gate/up of
  // narrow experts (I <= 512, six register sets) takes 2-wavefront blocks: twice the blocks, so
  // that more CUs hold two of them (measured at T = 128, I = 256: expert FFN 117.5 against
  // 119.3 us)
#define MOE_GEMM(GU_, MT_, S_, F16_, XBF_, XA_, Q0_, S0_, Q1_, S1_, OUT_)                       \
  do {                                                                                        \
    constexpr int NW_ = MT_ == 128 ? 8 : (GU_ && MT_ == 32 && S_ >= 6) ? 2 : 4;              \
    const dim3 g_(GU_ ? (a.I + 32 * NW_ - 1) / (32 * NW_) : (a.H + 64 * NW_ - 1) / (64 * NW_), \
                  max_tiles);                                                                 \
    ffn_gemm_kernel<GU_, MT_, F16_, S_, NW_, XBF_><<<g_, 64 * NW_, 0, s>>>(                   \
        (const uint16_t*)(XA_), Q0_, S0_, Q1_, S1_, a.ts, a.sorted_slot, tiles, n_tiles, a.k,  \
        a.H, a.I, OUT_);                                                                      \
  } while (0)
#define MOE_GEMM_MT(MT_, S_, XBF_)                                                             \
  do {                                                                                        \
    MOE_GEMM(true, MT_, S_, false, XBF_, XBF_ ? (const void*)a.x : (const void*)a.x16, a.gq,   \
             a.gs, a.uq, a.us, a.h16);                                                        \
    if (a.y_f16)                                                                              \
      MOE_GEMM(false, MT_, S_, true, false, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);              \
    else                                                                                      \
      MOE_GEMM(false, MT_, S_, false, false, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);             \
  } while (0)
  // register sets of the load pipeline: 4, or more for the gate/up of a small batch of narrow
  // experts (I <= 512), whose few blocks are each bound by the bytes they keep in flight
  // (measured at T = 128, I = 256: 122 against 132 us with 6 sets; at T = 64, I = 2048, where
  // the blocks fill the chip, 6 sets cost occupancy: 943 against 921 us).  With 32-row tiles the
  // stage count should be a multiple of the set count (see the kernel's pipeline): the narrow
  // gate/up takes 8 sets when H / 64 is a multiple of 8 (else 6), its down 4 (K = I: 4 or 8
  // stages, all requested at once).
  if (MT == 128) {
    MOE_GEMM_MT(128, kGemmSets, false);
  } else if (MT == 64) {
    MOE_GEMM_MT(64, kGemmSets, true);
  } else if (a.I <= 512) {
    if ((a.H / gK) % 8 == 0)
      MOE_GEMM(true, 32, 8, false, true, (const void*)a.x, a.gq, a.gs, a.uq, a.us, a.h16);
    else
      MOE_GEMM(true, 32, 6, false, true, (const void*)a.x, a.gq, a.gs, a.uq, a.us, a.h16);
    if (a.y_f16)
      MOE_GEMM(false, 32, kGemmSets, true, false, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
    else
      MOE_GEMM(false, 32, kGemmSets, false, false, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
  } else {
    MOE_GEMM_MT(32, kGemmSets, true);
  }
#undef MOE_GEMM_MT
#undef MOE_GEMM
  return hipGetLastError();
}

}  // namespace moe
