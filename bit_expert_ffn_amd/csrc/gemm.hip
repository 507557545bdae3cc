// Grouped GEMM over the busy experts: gate/up (+ SwiGLU) and down on the matrix cores.
//
// Sources: per expert gate/up, SwiGLU, then down; one expert's weights are streamed while the
// rows routed to it are multiplied ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU",
// section 8, "The fused MoE kernel and the pair exchange"); a dequantize-then-multiply path for
// busier experts (same page, section 5); a grouped GEMM over the active experts only, with the
// 4-bit weights unpacked on chip and never written back dequantised ("Optimizing Models to Be
// Fast at Codegen", section 2).
//
// Work list: ffn_plan (run by the first block of the activation-conversion kernel) walks the
// active experts in order and lists every tile of MT rows of every expert with at least
// min_rows rows: (expert, first row).  grid.y runs over a host-side bound of that list; blocks
// past its end return.  Nothing is read back by the host.
//
// Block: 256 threads = 2 x 2 wavefronts, MT rows x 128 weight rows, K in stages of 64.
//   gate/up: the 128 weight rows are 64 gate rows and the same 64 up rows, so each wavefront
//            holds gate and up accumulators of the same 32 features and forms h = silu(g) * u
//            in registers (h stored as f16);
//   down:    the 128 weight rows are 128 output features.
// Per stage every thread loads its share of the activation tile (16-byte pieces of gathered
// rows) and 16 bytes of packed codes + 2 scale bytes of one weight tile row, decodes the 32
// weights (v_cvt_scalef32_pk_f16_fp4, then the e4m3 block scale with v_pk_mul_f16, exact in
// f16) and writes both tiles to LDS (rows padded to 144 bytes).  LDS is double buffered and the
// global loads run two stages ahead in registers.  Each wavefront then issues WM x 2 MFMAs
// (v_mfma_f32_32x32x16_f16, fp32 accumulate) per 16 columns of K.
#include "common.h"

namespace moe {

constexpr int gK = 64;       // K per pipeline stage
constexpr int gLD = gK + 8;  // padded LDS row, in halves
constexpr int gBR = 128;     // weight rows per block
constexpr int kXcds = 8;     // MI355X: 8 accelerator dies (XCDs), workgroups dealt round-robin
constexpr int kGroup = 4;    // consecutive row tiles whose blocks are ordered together

__device__ inline f16x8 gdecode8(uint32_t q, f16x2 s) {
  const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * s;
  const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * s;
  const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * s;
  const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * s;
  return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// List the MT-row tiles of every expert with >= min_rows rows (one wavefront).
__device__ void ffn_plan(const int32_t* __restrict__ count, const int32_t* __restrict__ active,
                         const int32_t* __restrict__ n_active, int MT, int min_rows,
                         int2* __restrict__ tiles, int max_tiles, int32_t* __restrict__ n_tiles) {
  const int lane = threadIdx.x & 63;
  const int na = *n_active;
  int ex[4], nt[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = lane * 4 + i;
    ex[i] = idx < na ? active[idx] : -1;
    const int c = ex[i] >= 0 ? count[ex[i]] : 0;
    nt[i] = c >= min_rows ? (c + MT - 1) / MT : 0;
    sum += nt[i];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  int start = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    for (int t = 0; t < nt[i] && start + t < max_tiles; ++t) tiles[start + t] = make_int2(ex[i], t * MT);
    start += nt[i];
  }
  if (lane == 63) *n_tiles = incl < max_tiles ? incl : max_tiles;
}

// x [T][H] bf16 -> f16 (8 values per thread); block 0's first wavefront also builds the tile
// list of the busy experts.
__global__ __launch_bounds__(256) void x_to_f16_plan_kernel(
    const uint16_t* __restrict__ x, _Float16* __restrict__ x16, size_t n8,
    const int32_t* __restrict__ count, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, int MT, int min_rows, int2* __restrict__ tiles,
    int max_tiles, int32_t* __restrict__ n_tiles) {
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
    ffn_plan(count, active, n_active, MT, min_rows, tiles, max_tiles, n_tiles);
}

template <bool GATEUP, int WM, bool Y_F16>
__global__ __launch_bounds__(256) void ffn_gemm_kernel(
    const _Float16* __restrict__ xa, const uint8_t* __restrict__ qm0,
    const uint8_t* __restrict__ sm0, const uint8_t* __restrict__ qm1,
    const uint8_t* __restrict__ sm1, const float* __restrict__ ts,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ sorted_slot, const int2* __restrict__ tiles,
    const int32_t* __restrict__ n_tiles, int k, int H, int I, void* __restrict__ out) {
  constexpr int MT = 64 * WM;
  constexpr int NA = 2 * WM;  // 16-byte activation pieces per thread per stage
  __shared__ __attribute__((aligned(16))) _Float16 As[2][MT][gLD];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][gBR][gLD];
  // Block order.  Workgroups go round-robin to the 8 XCDs, each with its own L2; renumber so
  // that every XCD gets one contiguous range of the logical order, and in that order take
  // groups of kGroup consecutive row tiles (about one expert), then the weight blocks, then the
  // tiles of the group.  The blocks resident on one XCD then share a few activation tiles and
  // a few weight slices.
  const int NB = gridDim.x;  // weight blocks (feature blocks)
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
  int j, fb;
  {
    const int grp = L / (kGroup * NB);
    const int gsz = min(kGroup, ntl - grp * kGroup);
    const int within = L - grp * kGroup * NB;
    fb = within / gsz;
    j = grp * kGroup + within % gsz;
  }
  const int2 te = tiles[j];
  const int e = te.x, m0 = te.y;
  const int rows = count[e];
  const int base = offset[e];
  const int K = GATEUP ? H : I;  // reduction length
  const int N = GATEUP ? I : H;  // rows of one weight matrix
  const int nchunk = K / 128;
  const int nstage = K / gK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // activation rows of this thread's pieces (rows past the expert's end repeat its last row:
  // their outputs are never stored).  Named variables, not arrays, so that they stay in
  // registers.
  auto arow_of = [&](int i) __attribute__((always_inline)) {
    const int s = tid + 256 * i;
    const int r = min(m0 + (s >> 3), rows - 1);
    const size_t src = GATEUP ? (size_t)(sorted_slot[base + r] / k) * H : (size_t)(base + r) * I;
    return xa + src + (s & 7) * 8;
  };
  const _Float16* arow0 = arow_of(0);
  const _Float16* arow1 = arow_of(1);
  const _Float16* arow2 = NA > 2 ? arow_of(2) : arow0;
  const _Float16* arow3 = NA > 2 ? arow_of(3) : arow0;
  // weight tile row of this thread: 8 tiles of 16 rows, 32 threads per tile
  const int bt = tid >> 5, sub = tid & 31;
  const int rt = GATEUP ? fb * 4 + (bt & 3) : fb * 8 + bt;
  const uint8_t* qsel = (GATEUP && bt >= 4) ? qm1 : qm0;
  const uint8_t* ssel = (GATEUP && bt >= 4) ? sm1 : sm0;
  const uint8_t* qb = qsel + (size_t)e * ((size_t)N * K / 2) + (size_t)rt * nchunk * 1024;
  const uint8_t* sb = ssel + (size_t)e * ((size_t)N * K / 16) + (size_t)rt * nchunk * 128;

  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;  // native vector: stays in VGPRs
  struct Stage {
    u32x4 a0, a1, a2, a3;
    u32x4 b;
    uint32_t s;
  };
  auto load = [&](Stage& r, int st) __attribute__((always_inline)) {
    const int k0 = st * gK;
    r.a0 = *reinterpret_cast<const u32x4*>(arow0 + k0);
    r.a1 = *reinterpret_cast<const u32x4*>(arow1 + k0);
    if (NA > 2) {
      r.a2 = *reinterpret_cast<const u32x4*>(arow2 + k0);
      r.a3 = *reinterpret_cast<const u32x4*>(arow3 + k0);
    }
    const int l = (st & 1) * 32 + sub;  // tile lane of this stage's 64-column half
    r.b = *reinterpret_cast<const u32x4*>(qb + ((size_t)(st >> 1) * 64 + l) * 16);
    r.s = *reinterpret_cast<const uint16_t*>(sb + ((size_t)(st >> 1) * 64 + l) * 2);
  };
  auto store = [&](const Stage& r, int buf) __attribute__((always_inline)) {
    // piece i of this thread: s = tid + 256 * i -> row s >> 3, 16-byte column s & 7
    const int c8 = (tid & 7) * 8;
    *reinterpret_cast<u32x4*>(&As[buf][(tid >> 3)][c8]) = r.a0;
    *reinterpret_cast<u32x4*>(&As[buf][(tid >> 3) + 32][c8]) = r.a1;
    if (NA > 2) {
      *reinterpret_cast<u32x4*>(&As[buf][(tid >> 3) + 64][c8]) = r.a2;
      *reinterpret_cast<u32x4*>(&As[buf][(tid >> 3) + 96][c8]) = r.a3;
    }
    const f16x2 sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(r.s, 1.0f, false);
    const f16x2 s0 = {sc[0], sc[0]};
    const f16x2 s1 = {sc[1], sc[1]};
    _Float16* dst = &Bs[buf][bt * 16 + (sub & 15)][(sub >> 4) * 32];
    *reinterpret_cast<f16x8*>(dst + 0) = gdecode8(r.b.x, s0);
    *reinterpret_cast<f16x8*>(dst + 8) = gdecode8(r.b.y, s0);
    *reinterpret_cast<f16x8*>(dst + 16) = gdecode8(r.b.z, s1);
    *reinterpret_cast<f16x8*>(dst + 24) = gdecode8(r.b.w, s1);
  };

  const int wm = w & 1, wn = w >> 1;
  f32x16 acc[WM][2];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int jn = 0; jn < 2; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.f;
  auto compute = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < gK; kk += 16) {
      f16x8 a[WM], b[2];
#pragma unroll
      for (int i = 0; i < WM; ++i)
        a[i] = *reinterpret_cast<const f16x8*>(
            &As[buf][wm * 32 * WM + i * 32 + (lane & 31)][kk + (lane >> 5) * 8]);
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int brow = GATEUP ? jn * 64 + wn * 32 : wn * 64 + jn * 32;
        b[jn] = *reinterpret_cast<const f16x8*>(&Bs[buf][brow + (lane & 31)][kk + (lane >> 5) * 8]);
      }
#pragma unroll
      for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn)
          acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[jn], acc[i][jn], 0, 0, 0);
    }
  };

  // pipeline: LDS double buffer; global loads two stages ahead (register sets r0 / r1 hold
  // the even / odd stages).  nstage = K / 64 is even (K is a multiple of 128), so the loop body
  // has no conditions; the two loads past the last stage re-read it (clamped) and are unused.
  Stage r0, r1;
  load(r0, 0);
  load(r1, 1);
  store(r0, 0);
  load(r0, min(2, nstage - 1));
  __syncthreads();
  for (int st = 0; st < nstage; st += 2) {
    compute(0);
    store(r1, 1);
    load(r1, min(st + 3, nstage - 1));
    __syncthreads();
    compute(1);
    store(r0, 0);
    load(r0, min(st + 4, nstage - 1));
    __syncthreads();
  }

  // epilogue; accumulator element v of a 32x32 tile: row (v/4)*8 + (lane/32)*4 + v%4, col lane%32
  const int rm = lane >> 5, cn = lane & 31;
  if (GATEUP) {
    const int f = fb * 64 + wn * 32 + cn;
    const float tsg = ts[e * 3 + 0], tsu = ts[e * 3 + 1];
    _Float16* h16 = reinterpret_cast<_Float16*>(out);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * 32 * WM + i * 32 + (v >> 2) * 8 + rm * 4 + (v & 3);
        if (m < rows) {
          const float gv = acc[i][0][v] * tsg, uv = acc[i][1][v] * tsu;
          h16[(size_t)(base + m) * I + f] = (_Float16)(gv / (1.0f + expf(-gv)) * uv);
        }
      }
  } else {
    const float tsd = ts[e * 3 + 2];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int jn = 0; jn < 2; ++jn) {
        const int f = fb * 128 + wn * 64 + jn * 32 + cn;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * 32 * WM + i * 32 + (v >> 2) * 8 + rm * 4 + (v & 3);
          if (m < rows) {
            const float yv = acc[i][jn][v] * tsd;
            const size_t o = (size_t)(base + m) * H + f;
            if (Y_F16)
              reinterpret_cast<_Float16*>(out)[o] = (_Float16)yv;
            else
              reinterpret_cast<float*>(out)[o] = yv;
          }
        }
      }
  }
}

int gemm_rows_per_tile(int T) { return T >= 2048 ? 128 : 64; }

size_t gemm_max_tiles(int T, int k, int E) {
  const int MT = gemm_rows_per_tile(T);
  const size_t n = (size_t)T * k;
  const size_t ne = (size_t)(E < (int)n ? E : (int)n);
  return n / MT + 1 + ne;
}

hipError_t launch_ffn_gemm(const FfnArgs& a, int min_rows, int2* tiles, int32_t* n_tiles,
                           hipStream_t s) {
  const int MT = gemm_rows_per_tile(a.T);
  const int max_tiles = (int)gemm_max_tiles(a.T, a.k, a.E);
  const size_t n8 = (size_t)a.T * a.H / 8;
  x_to_f16_plan_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(
      a.x, a.x16, n8, a.count, a.active, a.n_active, MT, min_rows, tiles, max_tiles, n_tiles);
  const dim3 gg(a.I / 64, max_tiles), gd(a.H / 128, max_tiles);
#define MOE_GEMM(GU_, WM_, F16_, GRID_, XA_, Q0_, S0_, Q1_, S1_, OUT_)                         \
  ffn_gemm_kernel<GU_, WM_, F16_><<<GRID_, 256, 0, s>>>(XA_, Q0_, S0_, Q1_, S1_, a.ts,          \
                                                        a.count, a.offset, a.sorted_slot,       \
                                                        tiles, n_tiles, a.k, a.H, a.I, OUT_)
  if (MT == 128) {
    MOE_GEMM(true, 2, false, gg, a.x16, a.gq, a.gs, a.uq, a.us, a.h16);
    if (a.y_f16) MOE_GEMM(false, 2, true, gd, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
    else MOE_GEMM(false, 2, false, gd, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
  } else {
    MOE_GEMM(true, 1, false, gg, a.x16, a.gq, a.gs, a.uq, a.us, a.h16);
    if (a.y_f16) MOE_GEMM(false, 1, true, gd, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
    else MOE_GEMM(false, 1, false, gd, a.h16, a.dq, a.ds, a.dq, a.ds, a.y);
  }
#undef MOE_GEMM
  return hipGetLastError();
}

}  // namespace moe
