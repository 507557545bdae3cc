/*
 * moe_nvfp4.h -- C ABI of libmoe_nvfp4.so: one sparse mixture-of-experts FFN layer with NVFP4
 * (4-bit) expert weights on an AMD Instinct MI355X (gfx950).
 *
 * The layer, as the source pages state it:
 *   - a router sends every token to k of E experts (8 of 256 in the pages' model):
 *     "Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", Background / "The model";
 *   - expert weights are 4-bit with one scale per 16 values, a microscaling format: same page,
 *     "NVFP4 experts"; weights stay 4-bit until they are unpacked in registers, never
 *     dequantised to HBM: "Optimizing Models to Be Fast at Codegen", section 2 "Kernels
 *     optimized for latency or throughput";
 *   - each chosen expert runs gate/up, SwiGLU and down, and the token's owner adds the expert
 *     outputs in a weighted sum: "Optimizing Muse Spark Open ...", section 8 "Prefill: a fused
 *     MoE kernel and fair batching" ("The fused MoE kernel and the pair exchange", "A one-pass
 *     combine");
 *   - busy and few-row experts take different paths after a step's experts are sorted by row
 *     count: same page, section 5 "Keeping register pressure off the common path";
 *   - index building stays on the device, with no host synchronisation: "Day-0 Inference
 *     Adaptation for Ultra-Large Sparse Models", "Operator Layer", Index Pipeline.
 * Readings taken where the pages are silent: the block scale is OCP E4M3FN, every expert matrix
 * also has one fp32 tensor scale, and the routing weights are the softmax over the k selected
 * logits (equal to the full softmax renormalised over them).
 *
 * Four calls make one layer, in this order on one stream:
 *     moe_route -> moe_group -> moe_expert_ffn_nvfp4 -> moe_combine
 *
 * Conventions for every call
 *   - Pointers named *_dev are device pointers (hipMalloc'd or torch CUDA tensors); everything
 *     else is host memory read during the call.  Device pointers must be 16-byte aligned.
 *     Arrays are dense, row-major, with the last index contiguous.
 *   - Ownership: the caller allocates and frees every buffer.  The library never allocates
 *     device memory for a call, frees nothing of the caller's and keeps no pointer after a call
 *     returns; kernels still queued on `stream` read and write the buffers until they finish.
 *     Calls may come from any thread; calls that share a workspace must be ordered on one
 *     stream.  The library keeps no per-call state.  Per device, on first use, it creates and
 *     keeps until the process ends: one side stream and two events (moe_expert_ffn_nvfp4 forks
 *     its busy-expert chain onto them for 3..31 tokens), and the single-launch kernel's
 *     occupancy.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is asynchronous: it
 *     validates its arguments on the host, enqueues kernels on `stream` and returns.  There is
 *     no host-device synchronisation inside any call.
 *   - Errors: arguments are checked before anything is enqueued; a failing check returns a
 *     negative moe_status and launches nothing.  A launch failure returns MOE_ERR_HIP.  Faults
 *     inside kernels surface at the caller's next synchronisation.  Expert ids are trusted
 *     (they come from moe_route); ids outside [0, E) are undefined behaviour.  NaN/Inf inputs
 *     propagate; there are no device-side checks.
 *   - Shape limits: 1 <= k <= E <= 256; H and I multiples of 128 with 128 <= H, I <= 65536;
 *     T >= 1 and T*k < 2^31; for the calls that take I, also T*H < 2^32 and T*k*I < 2^32.
 *   - Activation range: on the matrix-core path (32 tokens and more) x enters the matrix cores
 *     as f16, so |x| must not exceed 65504 (larger values become Inf there, while the few-row
 *     and single-launch paths, which dot x as bf16, stay finite); magnitudes below 2^-14 lose
 *     precision as f16 subnormals.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_NVFP4_ABI_VERSION 5

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1,   /* NULL pointer, misaligned pointer, T < 1, k > E, bad dtype */
  MOE_ERR_UNSUPPORTED_SHAPE = -2,  /* H or I not a multiple of 128, E > 256, sizes too large   */
  MOE_ERR_WORKSPACE_TOO_SMALL = -3,
  MOE_ERR_HIP = -4,                /* a HIP launch or runtime call failed                      */
  MOE_ERR_INTERNAL = -5,
  MOE_ERR_TIMEOUT = -6,            /* moe_layer_check: a wait of the single-launch layer gave up */
  MOE_ERR_SCRATCH_TOO_SMALL = -7   /* moe_layer_nvfp4_noalloc: the shape needs more than 16 MiB */
};

/* element type tag of the expert-output buffer y */
enum { MOE_F32 = 0, MOE_F16 = 1 };

/* NVFP4 expert weights, as moe_expert_ffn_nvfp4 reads them.  All pointers are device
 * pointers.  Per expert e there are three matrices W[n][k] with N rows (outputs) and K columns
 * (the reduction):  gate and up (N = I, K = H) and down (N = H, K = I).  Weight value:
 *     W[n][k] = e2m1(code[n][k]) * e4m3(scale[n][k / 16]) * tensor_scale[e][matrix]
 * with e2m1 codes (4 bits) and OCP E4M3FN scale codes, one scale per 16 consecutive k.
 * Byte layout: TILE-MAJOR (moe_nvfp4_pack converts the usual row-major layout, codes [N][K/2]
 * with the low nibble holding the even k, and scales [N][K/16]).  The matrix is cut into
 * 16-row x 128-column tiles (r = n / 16, c = k / 128), ordered r-major; inside a tile, slot
 * l = 16 * ((k % 128) / 32) + n % 16 holds the 32 codes of row n, columns 128c + 32g .. +32
 * (16 bytes, low nibble = even k) and their two scale bytes:
 *     code byte  of (n, k): ((r * (K/128) + c) * 64 + l) * 16 + (k % 32) / 2
 *     scale byte of (n, k): ((r * (K/128) + c) * 64 + l) * 2  + (k % 32) / 16
 * Expert e's matrix starts at byte e * N*K/2 (codes) and e * N*K/16 (scales), i.e.
 *   gate_q, up_q [E] x I*H/2 bytes,  gate_s, up_s [E] x I*H/16 bytes,
 *   down_q       [E] x H*I/2 bytes,  down_s       [E] x H*I/16 bytes,
 *   tensor_scale [E][3] fp32 (gate, up, down).
 * One wavefront load then reads one tile: 1 KB of codes or 128 B of scales, contiguous.
 * The struct itself is host memory, read during the call only. */
typedef struct moe_nvfp4_experts {
  const uint8_t *gate_q, *up_q, *down_q;
  const uint8_t *gate_s, *up_s, *down_s;
  const float *tensor_scale;
  int32_t E, H, I;
} moe_nvfp4_experts;

/* Version of this ABI (MOE_NVFP4_ABI_VERSION of the built library). */
int32_t moe_abi_version(void);

/* Static English text for a status code; never NULL. */
const char *moe_status_string(moe_status status);

/* Bytes of device workspace that every call of a layer with these sizes needs (one buffer
 * serves all calls, which must then be ordered on one stream).  Returns 0 if the sizes are
 * outside the shape limits.  Apart from its first 64 KiB the contents are scratch: calls keep
 * nothing there from one call to the next.  The first 64 KiB hold the counters and flags of
 * moe_layer_nvfp4's single-launch path: they must be zero before the first moe_layer_nvfp4 call
 * on the buffer (for example, allocate it zero-filled), every call leaves the counters and
 * flags zero, and no other call reads or writes them.  Two 32-bit words there are the
 * caller's: word 48 (bytes 192..195), the error word, becomes non-zero if a wait inside the
 * single-launch kernel gave up (that call's outputs are then undefined; moe_layer_check reads
 * and clears it); word 49 (bytes 196..199), if non-zero, is the number of polls after which
 * such a wait gives up (0: the default, about 2 s). */
size_t moe_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t k);

/* Router and top-k ("The model": every token is routed to k of E experts).
 *   x_dev        [T][H] bf16 activations
 *   w_router_dev [H][E] fp32 router weights
 *   bias_dev     [E] fp32 added to every token's logits, or NULL
 *   logits_dev   [T][E] fp32 output, or NULL: logits[t][e] = sum_h x[t][h] * Wr[h][e] + bias[e],
 *                accumulated in fp32
 *   topk_id_dev  [T][k] int32 output: the k largest logits of each token in descending order,
 *                equal logits by ascending expert id
 *   topk_w_dev   [T][k] fp32 output: exp(l_j - l_max) / sum over the selected of exp(l - l_max)
 *   ws_dev       workspace of ws_bytes >= moe_workspace_size(...) bytes (contents scratch) */
moe_status moe_route(const void *x_dev, const float *w_router_dev, const float *bias_dev,
                     int32_t T, int32_t H, int32_t E, int32_t k, float *logits_dev,
                     int32_t *topk_id_dev, float *topk_w_dev, void *ws_dev, size_t ws_bytes,
                     void *stream);

/* Token-to-expert grouping: a stable counting sort of the T*k (token, slot) pairs by expert,
 * built on the device (Day-0 page, Index Pipeline), plus the experts sorted by row count for
 * the few-row / busy split (Muse Spark page, section 5).  Outputs (device, int32):
 *   count_dev       [E]    rows routed to each expert
 *   offset_dev      [E+1]  exclusive prefix sum of count; offset[E] = T*k
 *   sorted_slot_dev [T*k]  slot t*k+j of each row, rows ordered by (expert, t, j)
 *   slot_row_dev    [T*k]  inverse: the row that slot t*k+j landed on
 *   active_dev      [E]    experts with count > 0 by count descending then id ascending; the
 *                          remaining entries are -1
 *   n_active_dev    [1]    number of experts with count > 0
 * Every output is bit-exact and deterministic. */
moe_status moe_group(const int32_t *topk_id_dev, int32_t T, int32_t k, int32_t E,
                     int32_t *count_dev, int32_t *offset_dev, int32_t *sorted_slot_dev,
                     int32_t *slot_row_dev, int32_t *active_dev, int32_t *n_active_dev,
                     void *ws_dev, size_t ws_bytes, void *stream);

/* Expert FFN for every routed row (Muse Spark page, section 8: gate/up, SwiGLU, down):
 *   g = Wg.x, u = Wu.x, h = g / (1 + exp(-g)) * u, y = Wd.h
 * x_dev is [T][H] bf16; the grouping arrays are moe_group's outputs for the same T, k and E.
 * y_dev is [T*k][H] in grouped row order (row r belongs to sorted_slot[r]), of element type
 * y_dtype (MOE_F32 or MOE_F16).  Packed weights are decoded in registers and never written
 * out.  Arithmetic: x and h enter the matrix cores as f16, the decoded weights
 * e2m1 * e4m3 are exact in f16, products accumulate in fp32, h is stored as f16. */
moe_status moe_expert_ffn_nvfp4(const void *x_dev, const moe_nvfp4_experts *w, const int32_t *count_dev,
                                const int32_t *offset_dev, const int32_t *sorted_slot_dev,
                                const int32_t *active_dev, const int32_t *n_active_dev, int32_t T,
                                int32_t k, void *y_dev, int32_t y_dtype, void *ws_dev,
                                size_t ws_bytes, void *stream);

/* Layout conversion for NVFP4 weights: E matrices [N][K] from row-major (codes [E][N][K/2],
 * low nibble = even k; scales [E][N][K/16]) to the tile-major layout moe_expert_ffn_nvfp4
 * reads (see moe_nvfp4_experts).  Run once per matrix kind when weights are loaded: gate and
 * up with (N, K) = (I, H), down with (N, K) = (H, I).  Input and output must not overlap.
 * Requires N % 16 == 0, K % 128 == 0, N, K <= 65536.  Asynchronous on `stream`. */
moe_status moe_nvfp4_pack(const uint8_t *q_rowmajor_dev, const uint8_t *s_rowmajor_dev,
                          int32_t E, int32_t N, int32_t K, uint8_t *q_tiled_dev,
                          uint8_t *s_tiled_dev, void *stream);

/* Routing-weighted combine (Muse Spark page, section 8, "A one-pass combine"; "No zero fill"):
 *   out[t][n] = sum over j = 0..k-1 of topk_w[t][j] * y[slot_row[t*k+j]][n], in fp32.
 * Reads y once and writes every out row exactly once.  out_dev is [T][H] fp32. */
moe_status moe_combine(const void *y_dev, int32_t y_dtype, const int32_t *slot_row_dev,
                       const float *topk_w_dev, int32_t T, int32_t k, int32_t H, float *out_dev,
                       void *stream);

/* Combine variants: the weighted sum of moe_combine with one or both of
 *   MOE_COMBINE_EXPERT_NORM: every expert output row is RMS-normalised (no gain) before it is
 *     weighted ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", section 8, "The
 *     fused MoE kernel and the pair exchange": each expert's output is normalised before the
 *     weighted sum; "A one-pass combine": norm and weighted sum in one pass over the rows):
 *         f[t] = sum over j of topk_w[t][j] * y_j / sqrt(mean(y_j^2) + eps),
 *         y_j = y[slot_row[t*k+j]]; without the flag f[t] is moe_combine's sum;
 *   MOE_COMBINE_RESIDUAL_NORM: the epilogue that follows the MoE output in the residual stream
 *     (same page, section 3, "What makes this possible is where Muse Spark normalizes": the next
 *     layer's input is an RMS norm of alpha * x + beta * s * f, s being f's own RMS factor;
 *     "A 501B sparse model gets day-one serving support": post-norm, scaled residual and next
 *     pre-norm fused in one kernel):
 *         s = 1 / sqrt(mean(f[t]^2) + eps)
 *         out[t] = alpha * resid[t] + beta * s * f[t]                  (fp32, new residual)
 *         x_next[t] = bf16(gain * out[t] / sqrt(mean(out[t]^2) + eps))  (round to nearest even)
 *     Without the flag out[t] = f[t]; resid, gain and x_next are not read or written and may be
 *     NULL.
 * RMS norm as defined by Zhang and Sennrich, "Root Mean Square Layer Normalization" (the norm
 * the Muse Spark page cites).  The readings taken where the pages are silent: the per-expert
 * norm and the post-norm have no gain, the one eps serves all three norms, alpha and beta are
 * scalars.
 * Shapes: y_dev [T*k][H] of y_dtype (grouped rows, as written by moe_expert_ffn_nvfp4),
 * slot_row_dev [T*k], topk_w_dev [T][k] fp32, resid_dev and out_dev [T][H] fp32, gain_dev [H]
 * fp32, x_next_dev [T][H] bf16 (the input format of the next layer's moe_route).  resid_dev may
 * equal out_dev (update in place); no other overlap between inputs and outputs is allowed.
 * Every out and x_next row is written once.  Requires flags within the two bits, finite
 * eps >= 0 and every pointer the flags use non-NULL and 16-byte aligned, else
 * MOE_ERR_INVALID_ARGUMENT.  With eps = 0 an all-zero row gives Inf/NaN (not checked).
 * flags = 0 gives results bit-identical to moe_combine. */
#define MOE_COMBINE_EXPERT_NORM 1u
#define MOE_COMBINE_RESIDUAL_NORM 2u
moe_status moe_combine_norm(const void *y_dev, int32_t y_dtype, const int32_t *slot_row_dev,
                            const float *topk_w_dev, int32_t T, int32_t k, int32_t H,
                            uint32_t flags, float eps, const float *resid_dev, float alpha,
                            float beta, const float *gain_dev, float *out_dev,
                            uint16_t *x_next_dev, void *stream);

/* The whole layer in one call: route, group, expert FFN and combine, with the same arguments,
 * outputs and meaning as the four calls above (one token: out[t] = sum over the token's k
 * experts of topk_w * FFN_e(x[t])).
 * One or two tokens (T*k <= 32 and small enough LDS staging) run as ONE persistent kernel:
 * every token's expert weights are requested as soon as its routing is known and no launch
 * gap separates the steps ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU",
 * section 1 "A megakernel", section 2 "Pipelining everything inside the megakernel").  The
 * kernel launches one block per CU and its blocks wait for each other through the counters at
 * the start of ws_dev (see moe_workspace_size).  Precondition: every block must become
 * resident while the others wait, so no other work may hold the device's CUs for the length
 * of a wait (about 2 s by default) -- for example a long kernel on another stream.  If a wait
 * gives up, its block writes NaN over its features of out and skips the rest of its work (any
 * give-up keeps a barrier from completing for every block that has out features, so out shows
 * NaN; the other outputs are undefined), the error word is set (moe_layer_check reports it) and
 * the counters are still reset for the next call.
 * That path writes logits (if not NULL), topk_id, topk_w, the grouping arrays and out, but not
 * y; the combine there adds each token's experts in the order of the active list rather than
 * by slot, except for one token with k = 8, where each block group (one per XCD) runs one
 * slot's expert and the 8 weighted expert rows, each rounded to fp32, are added in slot order.
 * From 3 to 128 tokens (T*k <= 4096) the router, top-k + softmax, grouping and the grouped
 * GEMM's tile list run as ONE persistent kernel (same pages and sections), then the expert FFN
 * and the combine: y_dev ([T*k][H] of y_dtype, grouped row order) holds the expert outputs.
 * Its logits are summed on the matrix cores from exact three-piece bf16 splits of the fp32
 * router weights, so they differ from moe_route's only in the order of fp32 additions; ids,
 * weights and grouping follow from the logits exactly as in moe_route and moe_group.  It
 * waits at grid barriers like the single-launch kernel (same precondition and error word; if a
 * wait gives up, the grouping arrays describe no active expert and topk_w is NaN, so the
 * later kernels do nothing and out shows NaN).
 * Above 128 tokens, or on a device that cannot keep one block per CU resident, the four calls
 * run in order, and the one-block grouping also writes the grouped GEMM's tile list into
 * ws_dev, which saves the expert-FFN call one launch; every output is then bit-identical to
 * that of the four calls.  Calls that share ws_dev must not overlap in time. */
moe_status moe_layer_nvfp4(const void *x_dev, const float *w_router_dev, const float *bias_dev,
                           const moe_nvfp4_experts *w, int32_t T, int32_t k, float *logits_dev,
                           int32_t *topk_id_dev, float *topk_w_dev, int32_t *count_dev,
                           int32_t *offset_dev, int32_t *sorted_slot_dev, int32_t *slot_row_dev,
                           int32_t *active_dev, int32_t *n_active_dev, void *y_dev,
                           int32_t y_dtype, float *out_dev, void *ws_dev, size_t ws_bytes,
                           void *stream);

/* moe_layer_nvfp4 without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, outputs and meaning as moe_layer_nvfp4 minus ws_dev / ws_bytes; the caller still
 * passes every input and output buffer.  The scratch is a 16 MiB array of device memory that
 * the library holds per GPU from its first use there until the process ends; a call whose
 * moe_workspace_size(T, H, I, E, k) exceeds 16 MiB returns MOE_ERR_SCRATCH_TOO_SMALL and
 * launches nothing (at H = 7168, I = 2048, E = 256, k = 8 that is above about 340 tokens).
 * The call makes no device allocation or free, no library call that allocates, creates no
 * stream or event (every kernel, also the busy-expert chain of 3..31 tokens, runs on `stream`),
 * and the first call on a device only looks up the array's address there.  The array keeps
 * the last call's contents; the only part that must start zero -- the single-launch kernel's
 * counters and flags -- is zero at load and left zero by every call.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two streams, two threads
 * without ordering) race and give undefined results.  A single-launch wait that gives up shows
 * as NaN in out (see moe_layer_nvfp4); its error word is not readable by the caller. */
moe_status moe_layer_nvfp4_noalloc(const void *x_dev, const float *w_router_dev,
                                   const float *bias_dev, const moe_nvfp4_experts *w, int32_t T,
                                   int32_t k, float *logits_dev, int32_t *topk_id_dev,
                                   float *topk_w_dev, int32_t *count_dev, int32_t *offset_dev,
                                   int32_t *sorted_slot_dev, int32_t *slot_row_dev,
                                   int32_t *active_dev, int32_t *n_active_dev, void *y_dev,
                                   int32_t y_dtype, float *out_dev, void *stream);

/* Status of the single-launch layer on this workspace: waits until `stream` is idle, reads the
 * error word (word 48 of ws_dev) and returns MOE_OK if it is zero.  Otherwise a wait inside an
 * earlier moe_layer_nvfp4 call on this workspace gave up (the outputs of that call are
 * undefined): the call clears the first 64 KiB of ws_dev except word 49 (the spin limit) and
 * returns MOE_ERR_TIMEOUT.  Synchronising; pass the stream the layer calls were made on.
 * ws_dev must be 16-byte aligned and ws_bytes >= 65536. */
moe_status moe_layer_check(void *ws_dev, size_t ws_bytes, void *stream);

/* ---- fp8-compute variant ------------------------------------------------------------------
 * The pages' serving stack computes in fp8 with NVFP4 expert weights ("Optimizing Muse Spark
 * Open on TPU v7 with SGLang-TorchTPU", Figure 1).  On gfx950 that runs on the scaled matrix
 * cores in OCP MX form: MXFP8 = e4m3 (OCP E4M3FN) values with one e8m0 (power-of-two) scale
 * per 32 consecutive values along the reduction.  Quantiser, per block of 32: E =
 * floor(log2(max |v|)) - 8 clamped to [-127, 127] (an all-zero block gets E = -127 and zero
 * codes); element code = e4m3 of v / 2^E, rounded to nearest with ties to even and saturated
 * at 448; scale byte = E + 127.  This is an approximation of the layer, NOT the NVFP4 result:
 * the weights are requantised (an NVFP4 weight has 1..4 significant bits times an e4m3 scale,
 * which e4m3 under a shared power of two cannot always hold), and x and h are quantised.  On
 * the pages' layer shapes with Gaussian inputs the expert outputs differ from the exact layer
 * by about 7 % (relative L2); the variant is for callers that accept fp8 accuracy.
 *
 * MXFP8 expert weights.  Per expert e and matrix [N][K] (gate/up: N = I, K = H; down: N = H,
 * K = I), with r = n / 32, st = kk / 64, b = kk / 32 (the 32-block), and within the block
 * i = kk % 32:
 *     code  byte of (n, kk): e*N*K + ((r*(K/64) + st)*64 + n%32 + 32*(i/16))*32 + 16*(b%2) + i%16
 *     scale byte of (n, b):  e*N*K/32 + ((r*(K/256) + st/4)*64 + n%32 + 32*(b%2))*4 + st%4
 * i.e. 32-row x 64-column tiles of 2 KB in which each of the 64 lanes of a wavefront finds the
 * 32 bytes one matrix-core operand takes, and per 32-row tile and four 64-column steps 256
 * bytes of scales, four per lane.  Sizes: codes E*N*K bytes, scales E*N*K/32 bytes. */
typedef struct moe_mx8_experts {
  const uint8_t *gate_q, *up_q, *down_q;
  const uint8_t *gate_s, *up_s, *down_s;
  int32_t E, H, I;
} moe_mx8_experts;

/* Load-time requantisation of one NVFP4 matrix kind (row-major input, as moe_nvfp4_pack takes:
 * codes [E][N][K/2] with the low nibble holding the even k, scales [E][N][K/16]) to MXFP8 in
 * the layout above.  tensor_scale_dev is [E][3] fp32 and `matrix` (0 gate, 1 up, 2 down)
 * selects the column applied.  Every NVFP4 weight is dequantised exactly (in double) before
 * the quantiser runs, so the result is deterministic.  Requires N % 32 == 0, K % 256 == 0,
 * N, K <= 65536; outputs must not overlap the inputs.  Asynchronous on `stream`. */
moe_status moe_nvfp4_to_mxfp8(const uint8_t *q_rowmajor_dev, const uint8_t *s_rowmajor_dev,
                              const float *tensor_scale_dev, int32_t matrix, int32_t E,
                              int32_t N, int32_t K, uint8_t *q8_dev, uint8_t *s8_dev,
                              void *stream);

/* Expert FFN in fp8 (same rows, grouping arrays and output order as moe_expert_ffn_nvfp4):
 *   x8 = MXFP8(x) per token row; g = W8g.x8, u = W8u.x8 (products on the scaled matrix cores,
 *   fp32 accumulation); h = g / (1 + exp(-g)) * u in fp32, h8 = MXFP8(h) per 32 features;
 *   y = W8d.h8, written as f16 (y_dev [T*k][H] f16, grouped row order).
 * Requires H % 256 == 0 and I % 256 == 0 besides the common limits.  ws_dev as for the other
 * calls (moe_workspace_size). */
moe_status moe_expert_ffn_mx8(const void *x_dev, const moe_mx8_experts *w,
                              const int32_t *count_dev, const int32_t *offset_dev,
                              const int32_t *sorted_slot_dev, const int32_t *active_dev,
                              const int32_t *n_active_dev, int32_t T, int32_t k, void *y_dev,
                              void *ws_dev, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
