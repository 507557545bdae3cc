// C ABI of libmoe_nvfp4.so (declarations and contracts in include/moe_nvfp4.h).
// Every entry point validates its arguments on the host before enqueueing anything; a failing
// check returns an error code and launches nothing.
#include "moe_nvfp4.h"

#include <mutex>

#include "common.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {

WsLayout ws_layout(int T, int H, int I, int E, int k) {
  WsLayout L;
  // bytes [0, kSyncBytes): the single-launch layer's counters; no other call touches them
  const size_t base = kSyncBytes;
  const RoutePlan p = route_plan(T, H, E);
  L.route_partial = base;
  L.route_wsplit = base + align_up((size_t)p.KS * T * E * sizeof(float), 256);
  L.route_end = L.route_wsplit;
  if (p.mfma) L.route_end += align_up((size_t)3 * ((E + 31) / 32 * 32) * H * sizeof(uint16_t), 256);
  const size_t n = (size_t)T * k;
  L.group_whist = base;
  L.group_end = 0;
  if (n > (size_t)kGroupSmallMax) {
    const size_t nblk = (n + kGroupChunk - 1) / kGroupChunk;
    L.group_end = base + align_up(nblk * 16 * E * sizeof(int32_t), 256);
  }
  L.ffn_x16 = base;
  L.ffn_h16 = base + align_up((size_t)T * H * sizeof(_Float16), 256);
  L.ffn_tiles = L.ffn_h16 + align_up(n * I * sizeof(_Float16), 256);
  L.ffn_end = L.ffn_tiles + align_up(gemm_max_tiles(T, k, E) * sizeof(int4) + sizeof(int32_t), 256);
  L.mx8_x8 = base;
  L.mx8_xs = L.mx8_x8 + align_up((size_t)T * H, 256);
  L.mx8_h8 = L.mx8_xs + align_up((size_t)T * H / 32, 256);
  L.mx8_hs = L.mx8_h8 + align_up(n * I, 256);
  L.mx8_tiles = L.mx8_hs + align_up(n * I / 32, 256);
  L.mx8_end = L.mx8_tiles + align_up(gemm_max_tiles(T, k, E) * sizeof(int4) + sizeof(int32_t), 256);
  L.ls_partial = base;
  L.ls_h = base + align_up((size_t)32 * T * E * sizeof(float), 256);
  L.rg_masks = L.ls_h + align_up(n * I * sizeof(_Float16), 256);
  L.ls_xpart = L.rg_masks + align_up((size_t)E * (kRgMaxT / 32) * sizeof(uint32_t), 256);
  L.ls_end = L.ls_xpart + align_up((size_t)k * H * sizeof(float), 256);
  size_t tot = L.route_end;
  if (L.group_end > tot) tot = L.group_end;
  if (L.ffn_end > tot) tot = L.ffn_end;
  if (L.ls_end > tot) tot = L.ls_end;
  if (L.mx8_end > tot) tot = L.mx8_end;
  L.total = tot;
  return L;
}

}  // namespace moe

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_shape(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k) {
  if (T < 1 || k < 1 || E < 1 || k > E || H < 1 || I < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (H % 128 != 0 || I % 128 != 0 || H > 65536 || I > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T * k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

// Calls that read x through 32-bit element offsets (T*H) and h through 32-bit element offsets
// (T*k*I): the grouped GEMMs keep per-lane offsets from a uniform base in 32 bits.
moe_status check_rows(int64_t T, int64_t H, int64_t I, int64_t k) {
  if (T * H >= (int64_t)1 << 32 || T * k * I >= (int64_t)1 << 32) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

MOE_API int32_t moe_abi_version(void) { return MOE_NVFP4_ABI_VERSION; }

MOE_API const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument (NULL or misaligned pointer, bad size or dtype)";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "unsupported shape (E > 256, H or I not a multiple of 128 or above 65536, T*k >= 2^31, T*H >= 2^32 or T*k*I >= 2^32)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_INTERNAL: return "internal error";
    case MOE_ERR_SCRATCH_TOO_SMALL: return "the layer needs more scratch than moe_layer_nvfp4_noalloc holds (moe_workspace_size above 16 MiB)";
    case MOE_ERR_TIMEOUT: return "a wait inside the single-launch layer gave up (outputs undefined; sync region cleared)";
    default: return "unknown status";
  }
}

MOE_API size_t moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k) {
  if (check_shape(T, H, I, E, k) != MOE_OK || check_rows(T, H, I, k) != MOE_OK) return 0;
  return moe::ws_layout(T, H, I, E, k).total;
}

MOE_API moe_status moe_route(const void* x_dev, const float* w_router_dev, const float* bias_dev,
                             int32_t T, int32_t H, int32_t E, int32_t k, float* logits_dev,
                             int32_t* topk_id_dev, float* topk_w_dev, void* ws_dev,
                             size_t ws_bytes, void* stream) {
  if (!x_dev || !w_router_dev || !topk_id_dev || !topk_w_dev || !ws_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x_dev) || !aligned16(w_router_dev) || !aligned16(topk_id_dev) ||
      !aligned16(topk_w_dev) || !aligned16(ws_dev) || (bias_dev && !aligned16(bias_dev)) ||
      (logits_dev && !aligned16(logits_dev)))
    return MOE_ERR_INVALID_ARGUMENT;
  // the router does not depend on I: validate with the smallest legal I
  moe_status st = check_shape(T, H, 128, E, k);
  if (st != MOE_OK) return st;
  const moe::WsLayout L = moe::ws_layout(T, H, 128, E, k);
  if (ws_bytes < L.route_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  float* partial = reinterpret_cast<float*>((char*)ws_dev + L.route_partial);
  uint16_t* wsplit = reinterpret_cast<uint16_t*>((char*)ws_dev + L.route_wsplit);
  return from_hip(moe::launch_route((const uint16_t*)x_dev, w_router_dev, bias_dev, T, H, E, k,
                                    logits_dev, topk_id_dev, topk_w_dev, partial, wsplit,
                                    (hipStream_t)stream));
}

// moe_group; with plan, the grouping kernel also writes the busy experts' tile list
static moe_status group_run(const int32_t* topk_id_dev, int32_t T, int32_t k, int32_t E,
                            int32_t* count_dev, int32_t* offset_dev, int32_t* sorted_slot_dev,
                            int32_t* slot_row_dev, int32_t* active_dev, int32_t* n_active_dev,
                            void* ws_dev, size_t ws_bytes, void* stream,
                            const moe::GroupPlan* plan) {
  if (!topk_id_dev || !count_dev || !offset_dev || !sorted_slot_dev || !slot_row_dev ||
      !active_dev || !n_active_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(topk_id_dev) || !aligned16(count_dev) || !aligned16(offset_dev) ||
      !aligned16(sorted_slot_dev) || !aligned16(slot_row_dev) || !aligned16(active_dev) ||
      !aligned16(n_active_dev))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, 128, 128, E, k);
  if (st != MOE_OK) return st;
  const moe::WsLayout L = moe::ws_layout(T, 128, 128, E, k);
  if (L.group_end > 0) {
    if (!ws_dev || !aligned16(ws_dev)) return MOE_ERR_INVALID_ARGUMENT;
    if (ws_bytes < L.group_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  int32_t* whist = reinterpret_cast<int32_t*>((char*)ws_dev + L.group_whist);
  return from_hip(moe::launch_group(topk_id_dev, T, k, E, count_dev, offset_dev,
                                    sorted_slot_dev, slot_row_dev, active_dev, n_active_dev,
                                    whist, (hipStream_t)stream, plan));
}

MOE_API moe_status moe_group(const int32_t* topk_id_dev, int32_t T, int32_t k, int32_t E,
                             int32_t* count_dev, int32_t* offset_dev, int32_t* sorted_slot_dev,
                             int32_t* slot_row_dev, int32_t* active_dev, int32_t* n_active_dev,
                             void* ws_dev, size_t ws_bytes, void* stream) {
  return group_run(topk_id_dev, T, k, E, count_dev, offset_dev, sorted_slot_dev, slot_row_dev,
                   active_dev, n_active_dev, ws_dev, ws_bytes, stream, nullptr);
}

// moe_expert_ffn_nvfp4; planned: the tile list in the workspace is already written
static moe_status expert_ffn_run(const void* x_dev, const moe_nvfp4_experts* w,
                                 const int32_t* count_dev, const int32_t* offset_dev,
                                 const int32_t* sorted_slot_dev, const int32_t* active_dev,
                                 const int32_t* n_active_dev, int32_t T, int32_t k, void* y_dev,
                                 int32_t y_dtype, void* ws_dev, size_t ws_bytes, void* stream,
                                 int planned, int serial) {
  if (!x_dev || !w || !count_dev || !offset_dev || !sorted_slot_dev || !active_dev ||
      !n_active_dev || !y_dev || !ws_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!w->gate_q || !w->up_q || !w->down_q || !w->gate_s || !w->up_s || !w->down_s ||
      !w->tensor_scale)
    return MOE_ERR_INVALID_ARGUMENT;
  if (y_dtype != MOE_F32 && y_dtype != MOE_F16) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x_dev, count_dev, offset_dev, sorted_slot_dev, active_dev, n_active_dev,
                        y_dev, ws_dev, w->gate_q, w->up_q, w->down_q, w->gate_s, w->up_s,
                        w->down_s, w->tensor_scale};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, w->H, w->I, w->E, k);
  if (st == MOE_OK) st = check_rows(T, w->H, w->I, k);
  if (st != MOE_OK) return st;
  const moe::WsLayout L = moe::ws_layout(T, w->H, w->I, w->E, k);
  if (ws_bytes < L.ffn_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  moe::FfnArgs a;
  a.x = (const uint16_t*)x_dev;
  a.gq = w->gate_q; a.uq = w->up_q; a.dq = w->down_q;
  a.gs = w->gate_s; a.us = w->up_s; a.ds = w->down_s;
  a.ts = w->tensor_scale;
  a.count = count_dev; a.offset = offset_dev; a.sorted_slot = sorted_slot_dev;
  a.active = active_dev; a.n_active = n_active_dev;
  a.T = T; a.k = k; a.E = w->E; a.H = w->H; a.I = w->I;
  a.y = y_dev;
  a.y_f16 = y_dtype == MOE_F16;
  a.x16 = reinterpret_cast<_Float16*>((char*)ws_dev + L.ffn_x16);
  a.h16 = reinterpret_cast<_Float16*>((char*)ws_dev + L.ffn_h16);
  a.planned = planned;
  a.serial = serial;
  int4* tiles = reinterpret_cast<int4*>((char*)ws_dev + L.ffn_tiles);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(tiles + moe::gemm_max_tiles(T, k, w->E));
  return from_hip(moe::launch_ffn(a, tiles, n_tiles, (hipStream_t)stream));
}

MOE_API moe_status moe_expert_ffn_nvfp4(const void* x_dev, const moe_nvfp4_experts* w,
                                        const int32_t* count_dev, const int32_t* offset_dev,
                                        const int32_t* sorted_slot_dev, const int32_t* active_dev,
                                        const int32_t* n_active_dev, int32_t T, int32_t k,
                                        void* y_dev, int32_t y_dtype, void* ws_dev,
                                        size_t ws_bytes, void* stream) {
  return expert_ffn_run(x_dev, w, count_dev, offset_dev, sorted_slot_dev, active_dev,
                        n_active_dev, T, k, y_dev, y_dtype, ws_dev, ws_bytes, stream, 0, 0);
}

MOE_API moe_status moe_combine(const void* y_dev, int32_t y_dtype, const int32_t* slot_row_dev,
                               const float* topk_w_dev, int32_t T, int32_t k, int32_t H,
                               float* out_dev, void* stream) {
  if (!y_dev || !slot_row_dev || !topk_w_dev || !out_dev) return MOE_ERR_INVALID_ARGUMENT;
  if (y_dtype != MOE_F32 && y_dtype != MOE_F16) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_dev) || !aligned16(slot_row_dev) || !aligned16(topk_w_dev) ||
      !aligned16(out_dev))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, H, 128, k, k);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_combine(y_dev, y_dtype == MOE_F16, slot_row_dev, topk_w_dev, T, k,
                                      H, out_dev, (hipStream_t)stream));
}

MOE_API moe_status moe_combine_norm(const void* y_dev, int32_t y_dtype,
                                    const int32_t* slot_row_dev, const float* topk_w_dev,
                                    int32_t T, int32_t k, int32_t H, uint32_t flags, float eps,
                                    const float* resid_dev, float alpha, float beta,
                                    const float* gain_dev, float* out_dev, uint16_t* x_next_dev,
                                    void* stream) {
  if (!y_dev || !slot_row_dev || !topk_w_dev || !out_dev) return MOE_ERR_INVALID_ARGUMENT;
  if (y_dtype != MOE_F32 && y_dtype != MOE_F16) return MOE_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)(MOE_COMBINE_EXPERT_NORM | MOE_COMBINE_RESIDUAL_NORM))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!(eps >= 0.0f) || eps == __builtin_inff()) return MOE_ERR_INVALID_ARGUMENT;
  const bool epi = (flags & MOE_COMBINE_RESIDUAL_NORM) != 0;
  if (epi && (!resid_dev || !gain_dev || !x_next_dev)) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(y_dev) || !aligned16(slot_row_dev) || !aligned16(topk_w_dev) ||
      !aligned16(out_dev))
    return MOE_ERR_INVALID_ARGUMENT;
  if (epi && (!aligned16(resid_dev) || !aligned16(gain_dev) || !aligned16(x_next_dev)))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, H, 128, k, k);
  if (st != MOE_OK) return st;
  moe::CombineNormArgs a;
  a.y = y_dev; a.slot_row = slot_row_dev; a.w = topk_w_dev;
  a.T = T; a.k = k; a.H = H;
  a.expert_norm = (flags & MOE_COMBINE_EXPERT_NORM) != 0;
  a.epilogue = epi;
  a.eps = eps; a.alpha = alpha; a.beta = beta;
  a.resid = resid_dev; a.gain = gain_dev; a.out = out_dev; a.x_next = x_next_dev;
  return from_hip(moe::launch_combine_norm(a, y_dtype == MOE_F16, (hipStream_t)stream));
}

// moe_layer_nvfp4 on a given scratch buffer; serial: no side stream or events (every kernel on
// `stream`), for the allocation-free entry point
static moe_status layer_run(const void* x_dev, const float* w_router_dev, const float* bias_dev,
                            const moe_nvfp4_experts* w, int32_t T, int32_t k, float* logits_dev,
                            int32_t* topk_id_dev, float* topk_w_dev, int32_t* count_dev,
                            int32_t* offset_dev, int32_t* sorted_slot_dev, int32_t* slot_row_dev,
                            int32_t* active_dev, int32_t* n_active_dev, void* y_dev,
                            int32_t y_dtype, float* out_dev, void* ws_dev, size_t ws_bytes,
                            void* stream, int serial, moe_status too_small) {
  if (!x_dev || !w_router_dev || !w || !topk_id_dev || !topk_w_dev || !count_dev ||
      !offset_dev || !sorted_slot_dev || !slot_row_dev || !active_dev || !n_active_dev ||
      !y_dev || !out_dev || !ws_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!w->gate_q || !w->up_q || !w->down_q || !w->gate_s || !w->up_s || !w->down_s ||
      !w->tensor_scale)
    return MOE_ERR_INVALID_ARGUMENT;
  if (y_dtype != MOE_F32 && y_dtype != MOE_F16) return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x_dev, w_router_dev, topk_id_dev, topk_w_dev, count_dev, offset_dev,
                        sorted_slot_dev, slot_row_dev, active_dev, n_active_dev, y_dev, out_dev,
                        ws_dev, w->gate_q, w->up_q, w->down_q, w->gate_s, w->up_s, w->down_s,
                        w->tensor_scale};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if ((bias_dev && !aligned16(bias_dev)) || (logits_dev && !aligned16(logits_dev)))
    return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, w->H, w->I, w->E, k);
  if (st == MOE_OK) st = check_rows(T, w->H, w->I, k);
  if (st != MOE_OK) return st;
  const moe::WsLayout L = moe::ws_layout(T, w->H, w->I, w->E, k);
  if (ws_bytes < L.total) return too_small;
  const int H = w->H, I = w->I, E = w->E;
  if (moe::layer_small_fits(T, H, I, E, k)) {
    moe::LayerSmallArgs a;
    a.x = (const uint16_t*)x_dev;
    a.wr = w_router_dev;
    a.bias = bias_dev;
    a.gq = w->gate_q; a.uq = w->up_q; a.dq = w->down_q;
    a.gs = w->gate_s; a.us = w->up_s; a.ds = w->down_s;
    a.ts = w->tensor_scale;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.logits = logits_dev;
    a.topk_id = topk_id_dev; a.topk_w = topk_w_dev;
    a.count = count_dev; a.offset = offset_dev; a.sorted_slot = sorted_slot_dev;
    a.slot_row = slot_row_dev; a.active = active_dev; a.n_active = n_active_dev;
    a.out = out_dev;
    a.sync = reinterpret_cast<uint32_t*>(ws_dev);
    a.partial = reinterpret_cast<float*>((char*)ws_dev + L.ls_partial);
    a.h = reinterpret_cast<uint32_t*>((char*)ws_dev + L.ls_h);
    a.xpart = reinterpret_cast<float*>((char*)ws_dev + L.ls_xpart);
    const hipError_t e = moe::launch_layer_small(a, (hipStream_t)stream);
    if (e != hipErrorInvalidConfiguration) return from_hip(e);
    // the device cannot keep one block per CU resident: run the four calls instead
  }
  // the grouping (fused or not) also writes the busy experts' tile list, which saves the FFN
  // call's one-wavefront planning launch
  moe::GroupPlan gp{0, 0, 0, nullptr, nullptr};
  const bool fuse = (size_t)T * k <= (size_t)moe::kGroupSmallMax &&
                    moe::ffn_separate_plan(T, H, I, &gp.MT, &gp.min_rows);
  if (fuse) {
    gp.max_tiles = (int)moe::gemm_max_tiles(T, k, E);
    gp.tiles = reinterpret_cast<int4*>((char*)ws_dev + L.ffn_tiles);
    gp.n_tiles = reinterpret_cast<int32_t*>(gp.tiles + gp.max_tiles);
  }
  bool routed = false;
  if (moe::route_group_fits(T, k)) {
    // router, top-k, grouping and tile list in one persistent kernel
    moe::RouteGroupArgs r;
    r.x = (const uint16_t*)x_dev;
    r.wr = w_router_dev;
    r.bias = bias_dev;
    r.T = T; r.H = H; r.E = E; r.k = k;
    r.logits = logits_dev;
    r.topk_id = topk_id_dev; r.topk_w = topk_w_dev;
    r.count = count_dev; r.offset = offset_dev; r.sorted_slot = sorted_slot_dev;
    r.slot_row = slot_row_dev; r.active = active_dev; r.n_active = n_active_dev;
    r.sync = reinterpret_cast<uint32_t*>(ws_dev);
    r.partial = reinterpret_cast<float*>((char*)ws_dev + L.ls_partial);
    r.masks = reinterpret_cast<uint32_t*>((char*)ws_dev + L.rg_masks);
    r.plan_MT = fuse ? gp.MT : 0;
    r.plan_min_rows = gp.min_rows;
    r.max_tiles = gp.max_tiles;
    r.tiles = gp.tiles;
    r.n_tiles = gp.n_tiles;
    const hipError_t e = moe::launch_route_group(r, (hipStream_t)stream);
    if (e != hipSuccess && e != hipErrorInvalidConfiguration) return MOE_ERR_HIP;
    routed = e == hipSuccess;
    // else the device cannot keep one block per CU resident: separate kernels below
  }
  if (!routed) {
    st = moe_route(x_dev, w_router_dev, bias_dev, T, H, E, k, logits_dev, topk_id_dev,
                   topk_w_dev, ws_dev, ws_bytes, stream);
    if (st != MOE_OK) return st;
    st = group_run(topk_id_dev, T, k, E, count_dev, offset_dev, sorted_slot_dev, slot_row_dev,
                   active_dev, n_active_dev, ws_dev, ws_bytes, stream, fuse ? &gp : nullptr);
    if (st != MOE_OK) return st;
  }
  st = expert_ffn_run(x_dev, w, count_dev, offset_dev, sorted_slot_dev, active_dev,
                      n_active_dev, T, k, y_dev, y_dtype, ws_dev, ws_bytes, stream,
                      fuse ? 1 : 0, serial);
  if (st != MOE_OK) return st;
  return moe_combine(y_dev, y_dtype, slot_row_dev, topk_w_dev, T, k, H, out_dev, stream);
}

MOE_API moe_status moe_layer_nvfp4(const void* x_dev, const float* w_router_dev,
                                   const float* bias_dev, const moe_nvfp4_experts* w, int32_t T,
                                   int32_t k, float* logits_dev, int32_t* topk_id_dev,
                                   float* topk_w_dev, int32_t* count_dev, int32_t* offset_dev,
                                   int32_t* sorted_slot_dev, int32_t* slot_row_dev,
                                   int32_t* active_dev, int32_t* n_active_dev, void* y_dev,
                                   int32_t y_dtype, float* out_dev, void* ws_dev,
                                   size_t ws_bytes, void* stream) {
  return layer_run(x_dev, w_router_dev, bias_dev, w, T, k, logits_dev, topk_id_dev, topk_w_dev,
                   count_dev, offset_dev, sorted_slot_dev, slot_row_dev, active_dev,
                   n_active_dev, y_dev, y_dtype, out_dev, ws_dev, ws_bytes, stream, 0,
                   MOE_ERR_WORKSPACE_TOO_SMALL);
}

// ---- allocation-free variant of moe_layer_nvfp4 ----
// Its scratch is this file-scope device array (one copy per GPU, held until the process ends).
// In host code the array's name is only a host-side stand-in: its device address on the current
// device comes from hipGetSymbolAddress, taken once per device on the first call there and
// kept; every kernel argument uses that address.  The first kSyncBytes (the single-launch
// kernel's counters and flags) start zero at load, and every call leaves them zero (a call
// whose waits give up included), so nothing needs clearing per call.
namespace {
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[64];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

MOE_API moe_status moe_layer_nvfp4_noalloc(const void* x_dev, const float* w_router_dev,
                                           const float* bias_dev, const moe_nvfp4_experts* w,
                                           int32_t T, int32_t k, float* logits_dev,
                                           int32_t* topk_id_dev, float* topk_w_dev,
                                           int32_t* count_dev, int32_t* offset_dev,
                                           int32_t* sorted_slot_dev, int32_t* slot_row_dev,
                                           int32_t* active_dev, int32_t* n_active_dev,
                                           void* y_dev, int32_t y_dtype, float* out_dev,
                                           void* stream) {
  // shapes that need more scratch than the array holds are refused before any HIP call
  if (w && check_shape(T, w->H, w->I, w->E, k) == MOE_OK &&
      check_rows(T, w->H, w->I, k) == MOE_OK &&
      moe::ws_layout(T, w->H, w->I, w->E, k).total > kNoAllocScratchBytes)
    return MOE_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MOE_ERR_HIP;
  return layer_run(x_dev, w_router_dev, bias_dev, w, T, k, logits_dev, topk_id_dev, topk_w_dev,
                   count_dev, offset_dev, sorted_slot_dev, slot_row_dev, active_dev,
                   n_active_dev, y_dev, y_dtype, out_dev, ws, kNoAllocScratchBytes, stream, 1,
                   MOE_ERR_SCRATCH_TOO_SMALL);
}

MOE_API moe_status moe_nvfp4_pack(const uint8_t* q_rowmajor_dev, const uint8_t* s_rowmajor_dev,
                                  int32_t E, int32_t N, int32_t K, uint8_t* q_tiled_dev,
                                  uint8_t* s_tiled_dev, void* stream) {
  if (!q_rowmajor_dev || !s_rowmajor_dev || !q_tiled_dev || !s_tiled_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(q_rowmajor_dev) || !aligned16(s_rowmajor_dev) || !aligned16(q_tiled_dev) ||
      !aligned16(s_tiled_dev))
    return MOE_ERR_INVALID_ARGUMENT;
  if (E < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N % 16 != 0 || K % 128 != 0 || N > 65536 || K > 65536) return MOE_ERR_UNSUPPORTED_SHAPE;
  const size_t qbytes = (size_t)E * N * K / 2, sbytes = (size_t)E * N * K / 16;
  const uintptr_t qi = (uintptr_t)q_rowmajor_dev, qo = (uintptr_t)q_tiled_dev;
  const uintptr_t si = (uintptr_t)s_rowmajor_dev, so = (uintptr_t)s_tiled_dev;
  if (qi < qo + qbytes && qo < qi + qbytes) return MOE_ERR_INVALID_ARGUMENT;  // no overlap
  if (si < so + sbytes && so < si + sbytes) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(moe::launch_pack(q_rowmajor_dev, s_rowmajor_dev, E, N, K, q_tiled_dev,
                                   s_tiled_dev, (hipStream_t)stream));
}

MOE_API moe_status moe_nvfp4_to_mxfp8(const uint8_t* q_rowmajor_dev, const uint8_t* s_rowmajor_dev,
                                      const float* tensor_scale_dev, int32_t matrix, int32_t E,
                                      int32_t N, int32_t K, uint8_t* q8_dev, uint8_t* s8_dev,
                                      void* stream) {
  if (!q_rowmajor_dev || !s_rowmajor_dev || !tensor_scale_dev || !q8_dev || !s8_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {q_rowmajor_dev, s_rowmajor_dev, tensor_scale_dev, q8_dev, s8_dev};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  if (matrix < 0 || matrix > 2 || E < 1 || N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (E > moe::kMaxExperts || N % 32 != 0 || K % 256 != 0 || N > 65536 || K > 65536)
    return MOE_ERR_UNSUPPORTED_SHAPE;
  const size_t qin = (size_t)E * N * K / 2, sin = (size_t)E * N * K / 16;
  const size_t qout = (size_t)E * N * K, sout = (size_t)E * N * K / 32;
  auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
  };
  if (overlap(q8_dev, qout, q_rowmajor_dev, qin) || overlap(q8_dev, qout, s_rowmajor_dev, sin) ||
      overlap(s8_dev, sout, q_rowmajor_dev, qin) || overlap(s8_dev, sout, s_rowmajor_dev, sin) ||
      overlap(q8_dev, qout, s8_dev, sout))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(moe::launch_nvfp4_to_mx8(q_rowmajor_dev, s_rowmajor_dev, tensor_scale_dev,
                                           matrix, E, N, K, q8_dev, s8_dev,
                                           (hipStream_t)stream));
}

MOE_API moe_status moe_expert_ffn_mx8(const void* x_dev, const moe_mx8_experts* w,
                                      const int32_t* count_dev, const int32_t* offset_dev,
                                      const int32_t* sorted_slot_dev, const int32_t* active_dev,
                                      const int32_t* n_active_dev, int32_t T, int32_t k,
                                      void* y_dev, void* ws_dev, size_t ws_bytes, void* stream) {
  if (!x_dev || !w || !count_dev || !offset_dev || !sorted_slot_dev || !active_dev ||
      !n_active_dev || !y_dev || !ws_dev)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!w->gate_q || !w->up_q || !w->down_q || !w->gate_s || !w->up_s || !w->down_s)
    return MOE_ERR_INVALID_ARGUMENT;
  const void* ptrs[] = {x_dev, count_dev, offset_dev, sorted_slot_dev, active_dev, n_active_dev,
                        y_dev, ws_dev, w->gate_q, w->up_q, w->down_q, w->gate_s, w->up_s,
                        w->down_s};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape(T, w->H, w->I, w->E, k);
  if (st == MOE_OK) st = check_rows(T, w->H, w->I, k);
  if (st != MOE_OK) return st;
  if (w->H % 256 != 0 || w->I % 256 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
  const moe::WsLayout L = moe::ws_layout(T, w->H, w->I, w->E, k);
  if (ws_bytes < L.mx8_end) return MOE_ERR_WORKSPACE_TOO_SMALL;
  moe::Mx8Args a;
  a.x = (const uint16_t*)x_dev;
  a.gq = w->gate_q; a.gs = w->gate_s; a.uq = w->up_q; a.us = w->up_s;
  a.dq = w->down_q; a.ds = w->down_s;
  a.count = count_dev; a.offset = offset_dev; a.sorted_slot = sorted_slot_dev;
  a.active = active_dev; a.n_active = n_active_dev;
  a.T = T; a.k = k; a.E = w->E; a.H = w->H; a.I = w->I;
  a.y = (_Float16*)y_dev;
  char* ws = (char*)ws_dev;
  a.x8 = (uint8_t*)(ws + L.mx8_x8);
  a.xs = (uint8_t*)(ws + L.mx8_xs);
  a.h8 = (uint8_t*)(ws + L.mx8_h8);
  a.hs = (uint8_t*)(ws + L.mx8_hs);
  a.tiles = (int4*)(ws + L.mx8_tiles);
  a.n_tiles = (int32_t*)(a.tiles + moe::gemm_max_tiles(T, k, w->E));
  return from_hip(moe::launch_ffn_mx8(a, (hipStream_t)stream));
}

MOE_API moe_status moe_layer_check(void* ws_dev, size_t ws_bytes, void* stream) {
  if (!ws_dev || !aligned16(ws_dev)) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < moe::kSyncBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(s);
  uint32_t err = 0;
  if (e == hipSuccess)
    e = hipMemcpy(&err, (char*)ws_dev + moe::kSyncErrWord * 4, sizeof(err), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (err == 0) return MOE_OK;
  // clear the sync region for the next call, except the caller's spin-limit word
  const size_t spin = (size_t)moe::kSyncSpinWord * 4;
  e = hipMemsetAsync(ws_dev, 0, spin, s);
  if (e == hipSuccess) e = hipMemsetAsync((char*)ws_dev + spin + 4, 0, moe::kSyncBytes - spin - 4, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? MOE_ERR_TIMEOUT : MOE_ERR_HIP;
}
