/*
 * CPU oracle for one sparse mixture-of-experts FFN layer with NVFP4 expert weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link, load or call this
 * code: only the test suite, the smoke check and the benchmark's CPU-baseline leg use it.  It
 * shares no source, header, table or helper with the HIP library; it decodes the input bytes
 * with its own tables.
 *
 * What it computes (the plain definition of the layer, in fp64 unless stated):
 *   router logits  ->  top-k of E experts  ->  softmax over the selected k  ->  grouping of
 *   (token, slot) rows by expert  ->  per row: gate/up projections, SwiGLU, down projection
 *   ->  routing-weighted sum of the k expert outputs of each token.
 * Combine variants (oracle_combine_norm): each expert output RMS-normalised before the weighted
 * sum, and the epilogue after it (the MoE output's own RMS factor, the scaled residual
 * alpha * x + beta * s * f, an RMS norm with a gain for the next layer's input).
 * Sources (the web pages this layer comes from):
 *   - "Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", Background / "The model":
 *     every token is routed to 8 of 256 experts; "NVFP4 experts": 4-bit expert weights with one
 *     scale per 16 values (a microscaling format).
 *   - same page, section 8 "Prefill: a fused MoE kernel and fair batching", "The fused MoE
 *     kernel and the pair exchange": per expert gate/up, SwiGLU, then down; the token's owner
 *     adds the expert outputs in a weighted sum.
 *   - "Mixture of Experts" topic page, Transformer Engine summary: grouped expert GEMMs with
 *     SwiGLU and routing-weight scaling.
 *   - Muse Spark page, section 8: each expert's output is normalised before the weighted sum;
 *     section 3, "What makes this possible is where Muse Spark normalizes": the residual stream
 *     and the RMS norm (Zhang and Sennrich) that feeds the next layer; "A 501B sparse model gets
 *     day-one serving support": post-norm, scaled residual and next pre-norm in one kernel.
 *
 * Precision.  Sums, SwiGLU and the combine run in double.  Router logits are summed in double
 * and rounded once to float: the top-k decision is taken on those float logits, in the same
 * precision the GPU path decides in.  Softmax weights are computed in double from the float
 * logits.
 *
 * Input byte formats (shared definition of the inputs, not of any arithmetic):
 *   x          [T][H]        bf16 bit patterns (uint16)
 *   w_router   [H][E]        float
 *   bias       [E] or NULL   float, added to the logits
 *   *_q        [E][N][K/2]   two e2m1 codes per byte, low nibble = even k
 *   *_s        [E][N][K/16]  e4m3 (OCP E4M3FN) scale codes, one per 16 consecutive k of a row
 *   ts         [E][3]        float tensor scales: gate, up, down
 *   gate/up: N = I, K = H.   down: N = H, K = I.
 */
#ifndef BIT_EXPERT_FFN_ORACLE_H
#define BIT_EXPERT_FFN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  const uint8_t *gate_q, *up_q, *down_q;
  const uint8_t *gate_s, *up_s, *down_s;
  const float *ts;
  int32_t E, H, I;
} oracle_experts;

double oracle_e2m1(int code);            /* 4-bit code -> value */
double oracle_e4m3(int code);            /* 8-bit OCP E4M3FN code -> value (NaN for 0x7F/0xFF) */
double oracle_bf16(uint16_t bits);       /* bf16 bit pattern -> value */

/* One dequantised weight W'[n][kk] of matrix m (0 gate, 1 up, 2 down) of expert e. */
double oracle_weight(const oracle_experts *w, int e, int m, int n, int kk);

void oracle_router(const uint16_t *x, const float *w_router, const float *bias,
                   int T, int H, int E, float *logits);
void oracle_topk(const float *logits, int T, int E, int k, int32_t *topk_id, double *topk_w);
void oracle_group(const int32_t *topk_id, int T, int k, int E, int32_t *count, int32_t *offset,
                  int32_t *sorted_slot, int32_t *slot_row, int32_t *active, int32_t *n_active);
/* FFN of expert e applied to token rows x[tok[r]] for r < nrows; y is [nrows][H]. */
void oracle_expert_rows(const uint16_t *x, int H, const oracle_experts *w, int e,
                        const int32_t *tok, int nrows, double *y);
/* h (SwiGLU output, [nrows][I]) of expert e for the same rows; diagnostic. */
void oracle_expert_hidden(const uint16_t *x, int H, const oracle_experts *w, int e,
                          const int32_t *tok, int nrows, double *h);
void oracle_combine(const double *y, const int32_t *slot_row, const double *topk_w,
                    int T, int k, int H, double *out);
/* Combine variants: per-expert RMS norm before the weighted sum (expert_norm) and the
 * post-norm + scaled residual + next pre-norm epilogue (epilogue); definitions in oracle.c. */
void oracle_combine_norm(const double *y, const int32_t *slot_row, const double *topk_w, int T,
                         int k, int H, int expert_norm, int epilogue, double eps,
                         const double *resid, double alpha, double beta, const double *gain,
                         double *f, double *s, double *out, double *r, double *xn);
/* The whole layer for the listed tokens only (routing is per token, so any subset is exact).
 * ids/w/logits/out are [ntok][k], [ntok][k], [ntok][E], [ntok][H]. */
void oracle_layer_tokens(const uint16_t *x, const float *w_router, const float *bias,
                         const oracle_experts *w, int H, int E, int k, const int32_t *tokens,
                         int ntok, float *logits, int32_t *topk_id, double *topk_w, double *out);
/* Low-precision variant (fp8 compute, OCP MX): MXFP8 weights requantised from NVFP4, MXFP8
 * activations and h.  Definitions and readings in oracle.c. */
int oracle_mx_exp(double amax, int emax);          /* shared exponent E (scale byte E + 127) */
int oracle_e4m3_code(double v);                    /* nearest e4m3 code, ties to even, saturated */
double oracle_mx_scale(int byte);                  /* e8m0 byte -> 2^(byte - 127) */
void oracle_mx8_quant(const double *v, int n, uint8_t *codes, uint8_t *scales);
void oracle_nvfp4_to_mxfp8(const oracle_experts *w, int m, uint8_t *q8, uint8_t *s8);
void oracle_expert_rows_mx(const uint16_t *x, int H, int I, int e, const uint8_t *gq,
                           const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                           const uint8_t *dq, const uint8_t *ds, const int32_t *tok, int nrows,
                           double *y);
/* Threads the oracle's parallel loops use (1 without OpenMP). */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
