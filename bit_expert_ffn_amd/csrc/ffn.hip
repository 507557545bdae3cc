// Expert FFN over NVFP4 weights, few-row experts, and the dispatch of the whole FFN call.
//
// Sources: per expert gate/up, SwiGLU, then down ("Optimizing Muse Spark Open on TPU v7 with
// SGLang-TorchTPU", section 8, "The fused MoE kernel and the pair exchange"); packed 4-bit
// weights are streamed and unpacked with their per-16 block scale in registers, never
// dequantised to HBM ("Optimizing Models to Be Fast at Codegen", section 2 "Kernels optimized
// for latency or throughput"); experts are split by row count into a few-row path and a busy
// path (Muse Spark page, section 5).
//
// Dispatch: every expert has at most T rows (a token's k experts are distinct).  The host picks
// R in {0, 1, 2, 4} from T; experts with <= R rows run the VALU kernels below, the others the
// matrix-core grouped GEMM (gemm.hip); from 32 tokens up R = 0 and the GEMM takes every expert.  Both read the tile-major weight layout (pack.hip): for a
// 16-feature row tile and a 128-column chunk, lane l = 16*g + n of a wavefront loads feature
// n's 32 values K = [c*128 + g*32, +32) (16 bytes) and their two e4m3 scale bytes; the
// wavefront's 64 loads are one contiguous 1 KB block.
// Decode: v_cvt_scalef32_pk_{bf16,f16}_fp4 turns one byte (two e2m1 codes) into two exact
// 16-bit values (the hardware uses only the exponent of its fp32 scale operand, so it is given
// 1.0); the e4m3 block scale multiplies each 16-value block sum in fp32; the fp32 tensor scale
// multiplies the final sum once.
// Activations: x is dotted as bf16 (exact); h is stored as f16 (the down projection's input).
#include <mutex>

#include "common.h"
#include "dot.h"

namespace moe {

// ---------------------------------------------------------------------------------------
// Few-row experts (at most R rows): VALU dot products.  A step's experts are sorted by row
// count and the few-row ones run in their own loop, apart from the busy experts' path
// ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", section 5 "Keeping register
// pressure off the common path"); most experts of a decode step serve one or two rows.
// Block: 4 wavefronts, one 16-feature tile each, over the whole K.  The first weights are
// requested as soon as the expert is known; the expert's activation rows are then staged once
// in LDS; each lane keeps up to 2 * kSet chunks of packed weights in flight: two register sets
// alternate, one loading while the other is used.  Lane l = 16*g + n
// decodes its 32 values of feature n per chunk and dots them with the matching 32 activation
// values of each row (two 16-value blocks, each block's sum times its e4m3 scale); the four
// K-groups of a feature are added by two cross-lane shuffles in a fixed order.
constexpr int kSet = 4;  // chunks per load set; two sets alternate

template <int R, int KS>
__global__ __launch_bounds__(256) void ffn_gateup_few_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ gq,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ us, const float* __restrict__ ts,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ sorted_slot, const int32_t* __restrict__ active,
    const int32_t* __restrict__ n_active, int k, int H, int I, _Float16* __restrict__ h16,
    int early) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [R][H] bf16
  __shared__ float red[4][R][2][16];
  const int slot = blockIdx.y;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ks = wv % KS;  // this wavefront's K slice of its tile
  const int rt = blockIdx.x * (4 / KS) + wv / KS;  // 16-feature row tile
  const int nchunk_all = H / kChunk;
  // balanced split: the host keeps KS <= nchunk_all, so every slice has at least one chunk
  const int cbeg = ks * nchunk_all / KS;
  const int nchunk = (ks + 1) * nchunk_all / KS - cbeg;  // chunks of this slice
  const size_t tile0 = (size_t)rt * nchunk_all + cbeg;
  const uint8_t* gqp = gq + (size_t)e * ((size_t)I * H / 2) + (tile0 * 64 + lane) * 16;
  const uint8_t* uqp = uq + (size_t)e * ((size_t)I * H / 2) + (tile0 * 64 + lane) * 16;
  const uint8_t* gsp = gs + (size_t)e * ((size_t)I * H / 16) + (tile0 * 64 + (lane & ~1)) * 2;
  const uint8_t* usp = us + (size_t)e * ((size_t)I * H / 16) + (tile0 * 64 + (lane & ~1)) * 2;
  // two sets of kSet chunks alternate: one set's loads are in flight while the other is used
  uint4 qgA[kSet], quA[kSet], qgB[kSet], quB[kSet];
  uint32_t sgA[kSet], suA[kSet], sgB[kSet], suB[kSet];
  auto load_set = [&](uint4* qg, uint4* qu, uint32_t* sg, uint32_t* su, int c0) {
#pragma unroll
    for (int u = 0; u < kSet; ++u) {
      const int c = min(c0 + u, nchunk - 1);  // clamped: past the end re-reads the last chunk
      qg[u] = load_stream16(gqp + c * 1024);
      qu[u] = load_stream16(uqp + c * 1024);
      sg[u] = load_scale_dword(gsp + c * 128);
      su[u] = load_scale_dword(usp + c * 128);
    }
  };
  // the first weights depend only on the expert: with few tokens (early != 0) request them
  // before the chain of dependent loads (row count, offsets, token ids, activations) that
  // staging the rows needs; with many tokens most experts are busy, so check the count first
  if (early) load_set(qgA, quA, sgA, suA, 0);
  const int rows = count[e];
  if (rows > R) return;  // a busy expert: the matrix-core path takes it
  if (!early) load_set(qgA, quA, sgA, suA, 0);
  const int base = offset[e];
  // stage the expert's activation rows
  for (int r = 0; r < rows; ++r) {
    const int tok = sorted_slot[base + r] / k;
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)tok * H);
    uint4* dst = reinterpret_cast<uint4*>(xs + (size_t)r * H);
    for (int i = threadIdx.x; i < H / 8; i += 256) dst[i] = src[i];
  }
  lds_barrier();
  float ag[R], au[R];
#pragma unroll
  for (int r = 0; r < R; ++r) ag[r] = au[r] = 0.f;
  auto use_set = [&](const uint4* qg, const uint4* qu, const uint32_t* sg, const uint32_t* su,
                     int c0) {
#pragma unroll
    for (int u = 0; u < kSet; ++u) {
      const int c = c0 + u;
      if (c < nchunk) {
        Dec32bf dg, du;  // decoded once, dotted with every row
        decode32(qg[u], scale_pair(sg[u], lane), dg);
        decode32(qu[u], scale_pair(su[u], lane), du);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (r < rows) {
            const uint4* xv = reinterpret_cast<const uint4*>(xs + (size_t)r * H + (cbeg + c) * kChunk + g * 32);
            ag[r] += dot32(dg, xv);
            au[r] += dot32(du, xv);
          }
        }
      }
    }
  };
  // sets of kSet chunks: the loop runs while two more sets exist and the tail takes the last one
  // or two, so no set past the end is requested (its loads would be waited for at the block's
  // reduction, a memory latency)
  const int nsets = (nchunk + kSet - 1) / kSet;
  int s = 0;
  for (; s + 2 < nsets; s += 2) {
    load_set(qgB, quB, sgB, suB, (s + 1) * kSet);
    use_set(qgA, quA, sgA, suA, s * kSet);
    load_set(qgA, quA, sgA, suA, (s + 2) * kSet);
    use_set(qgB, quB, sgB, suB, (s + 1) * kSet);
  }
  if (s + 1 < nsets) {
    load_set(qgB, quB, sgB, suB, (s + 1) * kSet);
    use_set(qgA, quA, sgA, suA, s * kSet);
    use_set(qgB, quB, sgB, suB, (s + 1) * kSet);
  } else {
    use_set(qgA, quA, sgA, suA, s * kSet);
  }
  // K-groups of a feature (cross-lane), then the block's K slices in order (LDS)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      ag[r] = sum_groups(ag[r]);
      au[r] = sum_groups(au[r]);
      if (KS > 1 && g == 0) {
        red[wv][r][0][n] = ag[r];
        red[wv][r][1][n] = au[r];
      }
    }
  }
  if (KS > 1) {
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows) {
        float sg2 = red[wv][r][0][n], su2 = red[wv][r][1][n];
#pragma unroll
        for (int j = 1; j < KS; ++j) {
          sg2 += red[wv + j][r][0][n];
          su2 += red[wv + j][r][1][n];
        }
        ag[r] = sg2;
        au[r] = su2;
      }
    }
  }
  const float tsg = ts[e * 3 + 0], tsu = ts[e * 3 + 1];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows && g == 0) {
      const float gv = ag[r] * tsg, uv = au[r] * tsu;
      const float hv = gv / (1.0f + expf(-gv)) * uv;
      h16[(size_t)(base + r) * I + rt * 16 + n] = (_Float16)hv;
    }
  }
}

template <int R, int KS, bool Y_F16>
__global__ __launch_bounds__(256) void ffn_down_few_kernel(
    const _Float16* __restrict__ h16, const uint8_t* __restrict__ dq,
    const uint8_t* __restrict__ dsc, const float* __restrict__ ts,
    const int32_t* __restrict__ count, const int32_t* __restrict__ offset,
    const int32_t* __restrict__ active, const int32_t* __restrict__ n_active, int H, int I,
    void* __restrict__ y, int early) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hs[];  // [R][I] f16
  __shared__ float red[4][R][16];
  const int slot = blockIdx.y;
  if (slot >= *n_active) return;
  const int e = active[slot];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ks = wv % KS;
  const int rt = blockIdx.x * (4 / KS) + wv / KS;
  const int nchunk_all = I / kChunk;
  const int cbeg = ks * nchunk_all / KS;
  const int nchunk = (ks + 1) * nchunk_all / KS - cbeg;
  const size_t tile0 = (size_t)rt * nchunk_all + cbeg;
  const uint8_t* qp = dq + (size_t)e * ((size_t)H * I / 2) + (tile0 * 64 + lane) * 16;
  const uint8_t* sp = dsc + (size_t)e * ((size_t)H * I / 16) + (tile0 * 64 + (lane & ~1)) * 2;
  uint4 qA[kSet], qB[kSet];
  uint32_t sA[kSet], sB[kSet];
  auto load_set = [&](uint4* q, uint32_t* sc, int c0) {
#pragma unroll
    for (int u = 0; u < kSet; ++u) {
      const int c = min(c0 + u, nchunk - 1);
      q[u] = load_stream16(qp + c * 1024);
      sc[u] = load_scale_dword(sp + c * 128);
    }
  };
  // first weights before the dependent loads that staging h needs (few tokens only)
  if (early) load_set(qA, sA, 0);
  const int rows = count[e];
  if (rows > R) return;
  if (!early) load_set(qA, sA, 0);
  const int base = offset[e];
  {
    const uint4* src = reinterpret_cast<const uint4*>(h16 + (size_t)base * I);
    uint4* dst = reinterpret_cast<uint4*>(hs);
    for (int i = threadIdx.x; i < rows * I / 8; i += 256) dst[i] = src[i];
  }
  lds_barrier();
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.f;
  auto use_set = [&](const uint4* q, const uint32_t* sc, int c0) {
#pragma unroll
    for (int u = 0; u < kSet; ++u) {
      const int c = c0 + u;
      if (c < nchunk) {
        Dec32h d;  // decoded once, dotted with every row
        decode32(q[u], scale_pair(sc[u], lane), d);
#pragma unroll
        for (int r = 0; r < R; ++r)
          if (r < rows)
            acc[r] += dot32(d, reinterpret_cast<const uint4*>(hs + (size_t)r * I + (cbeg + c) * kChunk + g * 32));
      }
    }
  };
  // the loop runs while two more sets exist; the tail requests nothing past the end
  const int nsets = (nchunk + kSet - 1) / kSet;
  int s = 0;
  for (; s + 2 < nsets; s += 2) {
    load_set(qB, sB, (s + 1) * kSet);
    use_set(qA, sA, s * kSet);
    load_set(qA, sA, (s + 2) * kSet);
    use_set(qB, sB, (s + 1) * kSet);
  }
  if (s + 1 < nsets) {
    load_set(qB, sB, (s + 1) * kSet);
    use_set(qA, sA, s * kSet);
    use_set(qB, sB, (s + 1) * kSet);
  } else {
    use_set(qA, sA, s * kSet);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows) {
      acc[r] = sum_groups(acc[r]);
      if (KS > 1 && g == 0) red[wv][r][n] = acc[r];
    }
  }
  if (KS > 1) {
    __syncthreads();
    if (ks != 0) return;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (r < rows) {
        float v = red[wv][r][n];
#pragma unroll
        for (int j = 1; j < KS; ++j) v += red[wv + j][r][n];
        acc[r] = v;
      }
    }
  }
  const float tsd = ts[e * 3 + 2];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (r < rows && g == 0) {
      const float v = acc[r] * tsd;
      const size_t o = (size_t)(base + r) * H + rt * 16 + n;
      if (Y_F16)
        reinterpret_cast<_Float16*>(y)[o] = (_Float16)v;
      else
        reinterpret_cast<float*>(y)[o] = v;
    }
  }
}

// K slices per 16-feature tile in the few-row kernels: enough wavefronts (and bytes in flight)
// to cover the HBM latency when there are few tiles.
static int few_ksplit(int tiles, int nchunk) {
  int ks = tiles <= 2048 ? 4 : tiles <= 4096 ? 2 : 1;
  while (ks > nchunk) ks >>= 1;  // every K slice keeps at least one chunk
  return ks;
}

// Largest row count of a "few-row" expert; 0 sends every expert to the grouped GEMM.  From 32
// tokens up the grouped GEMM (32-row tiles, streamed weight loads) is faster than the VALU
// kernels (measured at T = 64, I = 2048: expert FFN 915 against 978 us; at T = 128, I = 256:
// 130 against 190 us).
static int few_rows(int T, int H, int I) {
  int R = T <= 1 ? 1 : T <= 2 ? 2 : T < 32 ? 4 : 0;
  const int kmax = H > I ? H : I;
  while (R > 0 && (size_t)R * kmax * 2 > 65536) R >>= 1;
  return R;
}

bool ffn_separate_plan(int T, int H, int I, int* MT, int* min_rows) {
  const int R = few_rows(T, H, I);
  const int mt = gemm_rows_per_tile(T);
  if (T <= R || mt == 128) return false;
  *MT = mt;
  *min_rows = R + 1;
  return true;
}

// A second stream per device for the busy experts' chain (tile plan, grouped GEMMs), with the
// two events that fork it from the caller's stream and join it back.  The chain shares no data
// with the few-row chain (disjoint experts, so disjoint rows of h and y, and its own workspace
// regions), so the two run side by side and the caller's stream waits for both.  Created once
// per device, on first use, with the default priority, and kept until the process ends; the
// mutex is held while a call enqueues its fork, launches and join, so calls from several host
// threads take turns on the events and queue on the stream in order.
struct SideChain {
  hipStream_t stream;
  hipEvent_t fork, join;
};
static std::mutex side_mu;

static hipError_t side_chain(SideChain** out) {
  static SideChain chains[64];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideChain& c = chains[dev];
  if (!c.stream) {
    hipStream_t st = nullptr;
    hipEvent_t f = nullptr, j = nullptr;
    err = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&f, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&j, hipEventDisableTiming);
    if (err != hipSuccess) {
      if (j) (void)hipEventDestroy(j);
      if (f) (void)hipEventDestroy(f);
      if (st) (void)hipStreamDestroy(st);
      return err;
    }
    c.fork = f;
    c.join = j;
    c.stream = st;
  }
  *out = &c;
  return hipSuccess;
}

hipError_t launch_ffn(const FfnArgs& a, int4* tiles, int32_t* n_tiles, hipStream_t s) {
  const int maxe = a.E < a.T * a.k ? a.E : a.T * a.k;
  const int R = few_rows(a.T, a.H, a.I);
  const bool heavy = a.T > R;  // some expert may have more than R rows
  // both paths present: fork the busy chain onto the side stream, launched first so that its
  // blocks start alongside the few-row kernels
  SideChain* side = nullptr;
  std::unique_lock<std::mutex> side_lock(side_mu, std::defer_lock);
  if (R > 0 && heavy && !a.serial) {
    side_lock.lock();
    hipError_t err = side_chain(&side);
    if (err == hipSuccess) err = hipEventRecord(side->fork, s);
    if (err == hipSuccess) err = hipStreamWaitEvent(side->stream, side->fork, 0);
    if (err == hipSuccess) err = launch_ffn_gemm(a, R + 1, tiles, n_tiles, side->stream);
    if (err == hipSuccess) err = hipEventRecord(side->join, side->stream);
    if (err != hipSuccess) return err;
  }
  // with few tokens nearly every expert is few-row: request weights before checking the count
  const int early = (size_t)a.T * a.k <= (size_t)4 * a.E ? 1 : 0;
  // gate/up + SwiGLU
  if (R > 0) {
    const int ks = few_ksplit(maxe * (a.I / 16), a.H / kChunk);
    const dim3 grid(a.I / 16 / (4 / ks), maxe);
    const size_t lds = (size_t)R * a.H * 2;
#define MOE_FEW_GU(R_, KS_)                                                                  \
  ffn_gateup_few_kernel<R_, KS_><<<grid, 256, lds, s>>>(a.x, a.gq, a.uq, a.gs, a.us, a.ts,   \
                                                        a.count, a.offset, a.sorted_slot,    \
                                                        a.active, a.n_active, a.k, a.H, a.I, \
                                                        a.h16, early)
#define MOE_FEW_GU_R(R_)                 \
  do {                                   \
    if (ks == 4) MOE_FEW_GU(R_, 4);      \
    else if (ks == 2) MOE_FEW_GU(R_, 2); \
    else MOE_FEW_GU(R_, 1);              \
  } while (0)
    if (R == 1) MOE_FEW_GU_R(1);
    else if (R == 2) MOE_FEW_GU_R(2);
    else MOE_FEW_GU_R(4);
#undef MOE_FEW_GU_R
#undef MOE_FEW_GU
  }
  // down
  if (R > 0) {
    const int ks = few_ksplit(maxe * (a.H / 16), a.I / kChunk);
    const dim3 grid(a.H / 16 / (4 / ks), maxe);
    const size_t lds = (size_t)R * a.I * 2;
#define MOE_FEW_D(R_, KS_, F16_)                                                                 \
  ffn_down_few_kernel<R_, KS_, F16_><<<grid, 256, lds, s>>>(a.h16, a.dq, a.ds, a.ts, a.count,    \
                                                            a.offset, a.active, a.n_active, a.H, \
                                                            a.I, a.y, early)
#define MOE_FEW_D_R(R_, F16_)                   \
  do {                                          \
    if (ks == 4) MOE_FEW_D(R_, 4, F16_);        \
    else if (ks == 2) MOE_FEW_D(R_, 2, F16_);   \
    else MOE_FEW_D(R_, 1, F16_);                \
  } while (0)
    if (a.y_f16) {
      if (R == 1) MOE_FEW_D_R(1, true);
      else if (R == 2) MOE_FEW_D_R(2, true);
      else MOE_FEW_D_R(4, true);
    } else {
      if (R == 1) MOE_FEW_D_R(1, false);
      else if (R == 2) MOE_FEW_D_R(2, false);
      else MOE_FEW_D_R(4, false);
    }
#undef MOE_FEW_D_R
#undef MOE_FEW_D
  }
  hipError_t err = hipGetLastError();
  if (side) {
    // join: the caller's stream continues once the busy chain is done as well
    const hipError_t werr = hipStreamWaitEvent(s, side->join, 0);
    return err != hipSuccess ? err : werr;
  }
  if (err != hipSuccess) return err;
  if (heavy) return launch_ffn_gemm(a, R + 1, tiles, n_tiles, s);
  return hipGetLastError();
}

}  // namespace moe
