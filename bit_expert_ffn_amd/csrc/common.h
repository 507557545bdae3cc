// Internal declarations shared by the HIP sources of libmoe_nvfp4 (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

namespace moe {

constexpr int kMaxExperts = 256;
// rows handled by the one-block grouping kernel; above this the three-pass grouping runs
constexpr int kGroupSmallMax = 16384;
// slots per block of the three-pass grouping (16 waves x 256 slots: at 131,072 slots, 32 blocks
// for the histogram and scatter passes)
constexpr int kGroupChunk = 4096;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Router launch plan: TT tokens per block (RG wavefronts), the hidden dimension split into KS
// slices of kc rows, `tiles` token tiles.  mfma: the matrix-core router (many tokens), which
// needs the router weights split into three bf16 planes in the workspace.
struct RoutePlan {
  int TT, RG, KS, kc, tiles;
  bool mfma;
};
// fewest tokens for which the router runs on the matrix cores
constexpr int kRouteMfmaMinT = 512;

RoutePlan route_plan(int T, int H, int E);

// Byte offsets of every call's scratch inside the caller's workspace.  The first kSyncBytes
// hold the single-launch layer's counters and are used by nothing else.
constexpr size_t kSyncBytes = 65536;
// 32-bit words of the sync region that the host reads or writes: the error word (non-zero after
// a wait of the single-launch kernel gave up) and the spin-limit word (polls before a wait gives
// up; 0 = the default)
constexpr int kSyncErrWord = 48;
constexpr int kSyncSpinWord = 49;
struct WsLayout {
  size_t route_partial;  // [KS][T][E] fp32
  size_t route_wsplit;   // 3 x ceil(E / 32) x 32 x H bf16, operand order (matrix-core router only)
  size_t route_end;
  size_t group_whist;    // [nblk*16][E] int32 (three-pass grouping only)
  size_t group_end;
  size_t ffn_x16;        // [T][H] f16
  size_t ffn_h16;        // [T*k][I] f16
  size_t ffn_tiles;      // busy-expert tile list: [gemm_max_tiles] int4, then the count (int32)
  size_t ffn_end;
  size_t mx8_x8;         // fp8 variant: [T][H] e4m3 codes
  size_t mx8_xs;         // [T][H/32] e8m0 scales
  size_t mx8_h8;         // [T*k][I] e4m3 codes
  size_t mx8_hs;         // [T*k][I/32] e8m0 scales
  size_t mx8_tiles;      // tile list as ffn_tiles
  size_t mx8_end;
  size_t ls_partial;     // single-launch layer: [32][T][E] fp32 router partials
  size_t ls_h;           // single-launch layer: [T*k][I] f16
  size_t rg_masks;       // fused routing: [E][4] token masks
  size_t ls_xpart;       // single-launch layer, one token: [k][H] fp32 weighted expert rows
  size_t ls_end;
  size_t total;
};
WsLayout ws_layout(int T, int H, int I, int E, int k);

hipError_t launch_route(const uint16_t* x, const float* wr, const float* bias, int T, int H,
                        int E, int k, float* logits, int32_t* topk_id, float* topk_w,
                        float* partial, uint16_t* wsplit, hipStream_t s);
// plan_MT > 0 (one-block grouping only, T * k <= kGroupSmallMax): the grouping kernel also
// writes the busy experts' tile list, as ffn_plan would.
struct GroupPlan {
  int MT, min_rows, max_tiles;
  int4* tiles;
  int32_t* n_tiles;
};
hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* count,
                        int32_t* offset, int32_t* sorted_slot, int32_t* slot_row,
                        int32_t* active, int32_t* n_active, int32_t* whist, hipStream_t s,
                        const GroupPlan* plan = nullptr);

struct FfnArgs {
  const uint16_t* x;  // [T][H] bf16
  const uint8_t *gq, *uq, *dq, *gs, *us, *ds;
  const float* ts;
  const int32_t *count, *offset, *sorted_slot, *active, *n_active;
  int T, k, E, H, I;
  void* y;
  int y_f16;
  _Float16* x16;  // workspace
  _Float16* h16;  // workspace
  int planned;    // the tile list of the busy experts is already written (by the grouping)
  int serial;     // run every kernel on the caller's stream (no side stream, no events)
};
hipError_t launch_ffn(const FfnArgs& a, int4* tiles, int32_t* n_tiles, hipStream_t s);
hipError_t launch_ffn_gemm(const FfnArgs& a, int min_rows, int4* tiles, int32_t* n_tiles,
                           hipStream_t s);
int gemm_rows_per_tile(int T);
// Tile list that the expert-FFN call writes in a one-wavefront kernel of its own: false if it
// writes none there (no expert can be busy, or 128-row tiles, whose list comes with the x
// conversion); else its rows per tile and the fewest rows of a listed expert.
bool ffn_separate_plan(int T, int H, int I, int* MT, int* min_rows);
size_t gemm_max_tiles(int T, int k, int E);

// fp8 variant of the expert FFN (mx8.hip): MXFP8 weights in the tile layout of the scaled
// matrix cores, x and h quantised to MXFP8 on the fly, y in f16.
struct Mx8Args {
  const uint16_t* x;                           // [T][H] bf16
  const uint8_t *gq, *gs, *uq, *us, *dq, *ds;  // MXFP8 tile layout
  const int32_t *count, *offset, *sorted_slot, *active, *n_active;
  int T, k, E, H, I;
  _Float16* y;         // [T*k][H] grouped row order
  uint8_t *x8, *xs;    // workspace
  uint8_t *h8, *hs;    // workspace
  int4* tiles;         // workspace: tile descriptors
  int32_t* n_tiles;    // workspace
};
hipError_t launch_ffn_mx8(const Mx8Args& a, hipStream_t s);
hipError_t launch_nvfp4_to_mx8(const uint8_t* q, const uint8_t* s, const float* ts, int tsi,
                               int E, int N, int K, uint8_t* q8, uint8_t* s8, hipStream_t st);

// Single-launch layer for one or two tokens (layer_small.hip).
constexpr int kLsMaxSlots = 32;  // most (token, slot) rows of the single-launch layer
struct LayerSmallArgs {
  const uint16_t* x;  // [T][H] bf16
  const float* wr;    // [H][E]
  const float* bias;  // [E] or null
  const uint8_t *gq, *uq, *dq, *gs, *us, *ds;  // tile-major NVFP4
  const float* ts;                             // [E][3]
  int T, H, I, E, k;
  float* logits;  // [T][E] or null
  int32_t *topk_id, *count, *offset, *sorted_slot, *slot_row, *active, *n_active;
  float* topk_w;
  float* out;        // [T][H]
  uint32_t* sync;    // kSyncBytes: counters, flags and an error word, zero between calls
  float* partial;    // [32][T][E]
  uint32_t* h;       // [T*k][I/2] f16 pairs
  float* xpart;      // [k][H] fp32: one token's weighted expert rows (per-XCD mode)
};
size_t layer_small_lds(int T, int H, int I, int k);
bool layer_small_fits(int T, int H, int I, int E, int k);
hipError_t launch_layer_small(const LayerSmallArgs& a, hipStream_t s);

// Fused routing for a small batch (route_group.hip): router, top-k + softmax, grouping and the
// grouped GEMM's tile plan in one persistent kernel, for T <= kRgMaxT and T * k <= kRgMaxSlots.
constexpr int kRgMaxT = 128;
constexpr int kRgMaxSlots = 4096;
struct RouteGroupArgs {
  const uint16_t* x;  // [T][H] bf16
  const float* wr;    // [H][E]
  const float* bias;  // [E] or null
  int T, H, E, k;
  float* logits;  // [T][E] or null
  int32_t* topk_id;
  float* topk_w;
  int32_t *count, *offset, *sorted_slot, *slot_row, *active, *n_active;
  uint32_t* sync;   // kSyncBytes: counters and flags (shared with the single-launch layer)
  float* partial;   // [32][T][E]
  uint32_t* masks;  // [E][kRgMaxT / 32] token masks
  int plan_MT, plan_min_rows, max_tiles;  // plan_MT == 0: no tile list
  int4* tiles;
  int32_t* n_tiles;
};
bool route_group_fits(int T, int k);
hipError_t launch_route_group(const RouteGroupArgs& a, hipStream_t s);

hipError_t launch_pack(const uint8_t* q_in, const uint8_t* s_in, int E, int N, int K,
                       uint8_t* q_out, uint8_t* s_out, hipStream_t s);

hipError_t launch_combine(const void* y, int y_f16, const int32_t* slot_row, const float* w,
                          int T, int k, int H, float* out, hipStream_t s);

// Combine variants (per-expert RMS norm before the weighted sum; post-norm + scaled residual +
// next pre-norm epilogue).  resid and out may be the same array.
struct CombineNormArgs {
  const void* y;          // [rows][H] f16 or fp32, grouped row order
  const int32_t* slot_row;
  const float* w;         // [T][k]
  int T, k, H;
  int expert_norm, epilogue;
  float eps, alpha, beta;
  const float* resid;     // [T][H] (epilogue)
  const float* gain;      // [H] (epilogue)
  float* out;             // [T][H]
  uint16_t* x_next;       // [T][H] bf16 (epilogue)
};
hipError_t launch_combine_norm(const CombineNormArgs& a, int y_f16, hipStream_t s);

// List the MT-row tiles of every expert with >= min_rows rows (one wavefront).  Every tile
// of expert e gets the same descriptor {e, index of e's first tile, rows of e, first grouped
// row of e}: a tile's own first row is (its index - the first index) * MT, and the expert's
// tiles are consecutive in the list.  count, offset and active may be in global memory or in
// LDS (generic pointers); na is the number of active experts.
__device__ inline void ffn_plan_n(const int32_t* count, const int32_t* offset,
                                  const int32_t* active, int na, int MT, int min_rows,
                                  int4* __restrict__ tiles, int max_tiles,
                                  int32_t* __restrict__ n_tiles) {
  const int lane = threadIdx.x & 63;
  int ex[4], nt[4], cnt[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = lane * 4 + i;
    ex[i] = idx < na ? active[idx] : -1;
    cnt[i] = ex[i] >= 0 ? count[ex[i]] : 0;
    nt[i] = cnt[i] >= min_rows ? (cnt[i] + MT - 1) / MT : 0;
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
    if (nt[i] > 0) {
      const int4 d = make_int4(ex[i], start, cnt[i], offset[ex[i]]);
      for (int t = 0; t < nt[i] && start + t < max_tiles; ++t) tiles[start + t] = d;
    }
    start += nt[i];
  }
  if (lane == 63) *n_tiles = incl < max_tiles ? incl : max_tiles;
}
__device__ inline void ffn_plan(const int32_t* __restrict__ count,
                                const int32_t* __restrict__ offset,
                                const int32_t* __restrict__ active,
                                const int32_t* __restrict__ n_active, int MT, int min_rows,
                                int4* __restrict__ tiles, int max_tiles,
                                int32_t* __restrict__ n_tiles) {
  ffn_plan_n(count, offset, active, *n_active, MT, min_rows, tiles, max_tiles, n_tiles);
}

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Workgroup barrier that orders LDS only.  __syncthreads() also releases global memory, which
// makes every wavefront wait for all of its outstanding global loads (vmcnt(0)) before the
// barrier; a kernel whose global loads only feed registers (prefetch for later stages) keeps
// them in flight across this barrier instead.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace moe
