/*
 * CPU oracle for the NVFP4 sparse-MoE FFN layer.  TEST INFRASTRUCTURE ONLY: used by the test
 * suite, the smoke check and the benchmark's CPU-baseline leg, never by the product path.
 * Plain loops, no blocking or fusion; each function names the passage it follows.  The layer
 * and the byte formats are described in oracle.h.
 *
 * Parity pins for every function live in tests/test_oracle.py (hand-worked decode tables,
 * brute force on tiny inputs, closed forms, invariants and a dense-equivalent case).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent 0 is subnormal:
 * value = m * 0.5.  Otherwise value = 2^(e-1) * (1 + m/2).  Written from the bit fields, not a
 * table, so the hand-worked table in the tests is an independent check.
 * ("Optimizing Models to Be Fast at Codegen", section 2: weights stored as FP4 e2m1.) */
double oracle_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no infinities; the
 * all-ones exponent+mantissa pattern is NaN; largest finite 448.  This is the reading taken for
 * the per-16 block scale of the microscaling format ("NVFP4 experts"). */
double oracle_e4m3(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

double oracle_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Dequantisation of one weight: W'[n][kk] = e2m1(code) * e4m3(scale of the 16-block holding kk)
 * * tensor scale.  ("NVFP4 experts": one scale per 16 values.)  Exact in double. */
double oracle_weight(const oracle_experts *w, int e, int m, int n, int kk) {
  int N = (m == 2) ? w->H : w->I;
  int K = (m == 2) ? w->I : w->H;
  const uint8_t *q = (m == 0) ? w->gate_q : (m == 1) ? w->up_q : w->down_q;
  const uint8_t *s = (m == 0) ? w->gate_s : (m == 1) ? w->up_s : w->down_s;
  size_t row = (size_t)e * N + n;
  uint8_t byte = q[row * (K / 2) + kk / 2];
  int code = (kk & 1) ? (byte >> 4) : (byte & 15);
  double scale = oracle_e4m3(s[row * (K / 16) + kk / 16]);
  return oracle_e2m1(code) * scale * (double)w->ts[e * 3 + m];
}

/* Router: logits[t][e] = sum_h x[t][h] * Wr[h][e] (+ bias[e]).  The router picks experts per
 * token ("The model": each layer routes every token to 8 of 256 experts). */
void oracle_router(const uint16_t *x, const float *w_router, const float *bias,
                   int T, int H, int E, float *logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += oracle_bf16(x[(size_t)t * H + h]) * (double)w_router[(size_t)h * E + e];
      if (bias) acc += (double)bias[e];
      logits[(size_t)t * E + e] = (float)acc;
    }
  }
}

/* Top-k then softmax over the selected k.  Order: descending logit, equal logits by ascending
 * expert id.  w_j = exp(l_j - l_max) / sum over the selected of exp(l - l_max), which equals the
 * full softmax renormalised over the selected experts. */
void oracle_topk(const float *logits, int T, int E, int k, int32_t *topk_id, double *topk_w) {
  for (int t = 0; t < T; ++t) {
    const float *l = logits + (size_t)t * E;
    int32_t *id = topk_id + (size_t)t * k;
    char *taken = (char *)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower id on ties */
      }
      taken[best] = 1;
      id[j] = best;
    }
    free(taken);
    double mx = (double)l[id[0]], den = 0.0;
    for (int j = 0; j < k; ++j) den += exp((double)l[id[j]] - mx);
    for (int j = 0; j < k; ++j) topk_w[(size_t)t * k + j] = exp((double)l[id[j]] - mx) / den;
  }
}

/* Grouping of the T*k (token, slot) rows by expert: a stable counting sort.
 *   count[e]        rows routed to e
 *   offset[e]       exclusive prefix sum of count (offset[E] = T*k)
 *   sorted_slot[r]  slot index t*k+j of the r-th row, rows ordered by (e, t, j)
 *   slot_row[s]     inverse permutation: the row that slot s landed on
 *   active[i]       experts with count > 0, by count descending then id ascending
 * The pages sort a step's experts by row count to dispatch few-row and busy experts separately
 * ("Optimizing Muse Spark Open on TPU v7", section 5 "Keeping register pressure off the common
 * path"); the index building stays on the device (Day-0 adaptation page, "Operator Layer",
 * Index Pipeline). */
void oracle_group(const int32_t *topk_id, int T, int k, int E, int32_t *count, int32_t *offset,
                  int32_t *sorted_slot, int32_t *slot_row, int32_t *active, int32_t *n_active) {
  int n = T * k;
  for (int e = 0; e < E; ++e) count[e] = 0;
  for (int s = 0; s < n; ++s) count[topk_id[s]]++;
  offset[0] = 0;
  for (int e = 0; e < E; ++e) offset[e + 1] = offset[e] + count[e];
  int32_t *fill = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  for (int s = 0; s < n; ++s) {
    int e = topk_id[s];
    int r = offset[e] + fill[e]++;
    sorted_slot[r] = s;
    slot_row[s] = r;
  }
  free(fill);
  int na = 0;
  for (int e = 0; e < E; ++e)
    if (count[e] > 0) active[na++] = e;
  /* insertion sort by (count desc, id asc) */
  for (int i = 1; i < na; ++i) {
    int v = active[i], j = i - 1;
    while (j >= 0 && (count[active[j]] < count[v] ||
                      (count[active[j]] == count[v] && active[j] > v))) {
      active[j + 1] = active[j];
      --j;
    }
    active[j + 1] = v;
  }
  for (int i = na; i < E; ++i) active[i] = -1;
  *n_active = na;
}

/* Per-expert FFN: g = Wg'.x, u = Wu'.x, h = silu(g) * u with silu(g) = g / (1 + exp(-g)),
 * y = Wd'.h ("Prefill: a fused MoE kernel ...": gate/up, SwiGLU, then down). */
void oracle_expert_hidden(const uint16_t *x, int H, const oracle_experts *w, int e,
                          const int32_t *tok, int nrows, double *h) {
  int I = w->I;
  for (int r = 0; r < nrows; ++r) {
    const uint16_t *xr = x + (size_t)tok[r] * H;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < I; ++n) {
      double g = 0.0, u = 0.0;
      for (int kk = 0; kk < H; ++kk) {
        double xv = oracle_bf16(xr[kk]);
        g += oracle_weight(w, e, 0, n, kk) * xv;
        u += oracle_weight(w, e, 1, n, kk) * xv;
      }
      h[(size_t)r * I + n] = g / (1.0 + exp(-g)) * u;
    }
  }
}

void oracle_expert_rows(const uint16_t *x, int H, const oracle_experts *w, int e,
                        const int32_t *tok, int nrows, double *y) {
  int I = w->I;
  double *h = (double *)malloc(sizeof(double) * (size_t)nrows * I);
  oracle_expert_hidden(x, H, w, e, tok, nrows, h);
  for (int r = 0; r < nrows; ++r) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int i = 0; i < I; ++i) acc += oracle_weight(w, e, 2, n, i) * h[(size_t)r * I + i];
      y[(size_t)r * H + n] = acc;
    }
  }
  free(h);
}

/* Combine: out[t] = sum over j ascending of w[t][j] * y[slot_row[t*k+j]] ("A one-pass combine":
 * the weighted sum of a token's expert outputs; every output row written once). */
void oracle_combine(const double *y, const int32_t *slot_row, const double *topk_w,
                    int T, int k, int H, double *out) {
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j)
        acc += topk_w[(size_t)t * k + j] * y[(size_t)slot_row[t * k + j] * H + n];
      out[(size_t)t * H + n] = acc;
    }
}

/* Root-mean-square norm factor of one row: 1 / sqrt(mean(v^2) + eps) (Zhang and Sennrich,
 * "Root Mean Square Layer Normalization", the RMS norm the Muse Spark page cites). */
static double rms_factor(const double *v, int H, double eps) {
  double ss = 0.0;
  for (int n = 0; n < H; ++n) ss += v[n] * v[n];
  return 1.0 / sqrt(ss / H + eps);
}

/* Combine variants ("Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU", section 8 "A
 * one-pass combine" and "The fused MoE kernel and the pair exchange"; section 3, the residual
 * stream of "What makes this possible is where Muse Spark normalizes"; "A 501B sparse model
 * gets day-one serving support": post-norm, scaled residual and next pre-norm in one kernel).
 *   expert_norm: each expert row is RMS-normalised (no gain) before the weighted sum:
 *       f[t] = sum over j ascending of w[t][j] * rms_factor(y_j) * y_j,   y_j = y[slot_row[t*k+j]]
 *     otherwise f[t] is the plain weighted sum.
 *   epilogue: s = rms_factor(f[t]) (the MoE output's own norm factor),
 *       out[t]  = alpha * resid[t] + beta * s * f[t]          (the new residual stream)
 *       r       = rms_factor(out[t])
 *       xn[t]   = gain * out[t] * r                            (the next layer's input)
 *     otherwise out[t] = f[t] and s, r, xn are not written.
 * f, out, xn are [T][H]; s and r are [T] (may be NULL). */
void oracle_combine_norm(const double *y, const int32_t *slot_row, const double *topk_w, int T,
                         int k, int H, int expert_norm, int epilogue, double eps,
                         const double *resid, double alpha, double beta, const double *gain,
                         double *f, double *s, double *out, double *r, double *xn) {
  for (int t = 0; t < T; ++t) {
    double *ft = f + (size_t)t * H;
    for (int n = 0; n < H; ++n) ft[n] = 0.0;
    for (int j = 0; j < k; ++j) {
      const double *yj = y + (size_t)slot_row[t * k + j] * H;
      const double c = topk_w[(size_t)t * k + j] * (expert_norm ? rms_factor(yj, H, eps) : 1.0);
      for (int n = 0; n < H; ++n) ft[n] += c * yj[n];
    }
    double *ot = out + (size_t)t * H;
    if (!epilogue) {
      for (int n = 0; n < H; ++n) ot[n] = ft[n];
      continue;
    }
    const double st = rms_factor(ft, H, eps);
    for (int n = 0; n < H; ++n) ot[n] = alpha * resid[(size_t)t * H + n] + beta * st * ft[n];
    const double rt = rms_factor(ot, H, eps);
    for (int n = 0; n < H; ++n) xn[(size_t)t * H + n] = gain[n] * ot[n] * rt;
    if (s) s[t] = st;
    if (r) r[t] = rt;
  }
}

void oracle_layer_tokens(const uint16_t *x, const float *w_router, const float *bias,
                         const oracle_experts *w, int H, int E, int k, const int32_t *tokens,
                         int ntok, float *logits, int32_t *topk_id, double *topk_w, double *out) {
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  for (int i = 0; i < ntok; ++i) {
    int t = tokens[i];
    oracle_router(x + (size_t)t * H, w_router, bias, 1, H, E, logits + (size_t)i * E);
    oracle_topk(logits + (size_t)i * E, 1, E, k, topk_id + (size_t)i * k, topk_w + (size_t)i * k);
    for (int n = 0; n < H; ++n) out[(size_t)i * H + n] = 0.0;
    for (int j = 0; j < k; ++j) {
      int32_t one = t;
      oracle_expert_rows(x, H, w, topk_id[(size_t)i * k + j], &one, 1, y);
      for (int n = 0; n < H; ++n) out[(size_t)i * H + n] += topk_w[(size_t)i * k + j] * y[n];
    }
  }
  free(y);
}

/* ---------------------------------------------------------------------------------------------
 * Low-precision variant: fp8 compute, MXFP8 weights and activations (OCP Microscaling Formats
 * v1.0).  "Optimizing Muse Spark Open on TPU v7 with SGLang-TorchTPU" runs fp8 compute with NVFP4
 * expert weights (Figure 1).  The MX format shares one power-of-two scale X = 2^E (an e8m0 byte
 * E + 127) between 32 consecutive values: E = floor(log2(amax)) - 8 (8 = the largest exponent of
 * e4m3); each element is rounded to e4m3 to nearest, ties to even, and saturates at 448.  The
 * NVFP4 weights (e2m1 * e4m3 * fp32 tensor scale, exact in double) are requantised to MXFP8 once;
 * x and h are quantised to MXFP8 where they enter a product.  Readings: amax == 0 gives E = -127
 * and zero codes; E is clamped to [-127, 127]; a negative value keeps its sign bit even when its
 * magnitude rounds to zero. */

int oracle_mx_exp(double amax, int emax) {
  if (!(amax > 0.0)) return -127;
  int ex;
  frexp(amax, &ex);       /* amax = f * 2^ex, f in [0.5, 1): floor(log2(amax)) = ex - 1 */
  int E = ex - 1 - emax;
  return E < -127 ? -127 : (E > 127 ? 127 : E);
}

/* nearest integer, ties to even (the default rounding mode) */
static double rne(double v) { return nearbyint(v); }

int oracle_e4m3_code(double v) {
  const int sign = v < 0 ? 0x80 : 0;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) return sign | (int)rne(ldexp(a, 9)); /* subnormals, step 2^-9 */
  int ex;
  frexp(a, &ex);
  int e = ex - 1;                             /* 2^e <= a < 2^(e+1), e in [-6, 8] */
  int m = (int)rne((ldexp(a, -e) - 1.0) * 8.0);
  if (m == 8) { m = 0; ++e; }
  return sign | ((e + 7) << 3) | m;
}

double oracle_mx_scale(int byte) { return ldexp(1.0, byte - 127); }

/* MXFP8 quantisation of n values (n a multiple of 32): codes[n], scales[n / 32]. */
void oracle_mx8_quant(const double *v, int n, uint8_t *codes, uint8_t *scales) {
  for (int b = 0; b < n / 32; ++b) {
    double amax = 0.0;
    for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(v[32 * b + i]));
    const int E = oracle_mx_exp(amax, 8);
    scales[b] = (uint8_t)(E + 127);
    for (int i = 0; i < 32; ++i)
      codes[32 * b + i] = amax > 0.0 ? (uint8_t)oracle_e4m3_code(ldexp(v[32 * b + i], -E)) : 0;
  }
}

/* NVFP4 matrix m (0 gate, 1 up, 2 down) of every expert -> MXFP8 in the logical row-major
 * layout: q8 [E][N][K] e4m3 codes, s8 [E][N][K/32] e8m0 scale bytes. */
void oracle_nvfp4_to_mxfp8(const oracle_experts *w, int m, uint8_t *q8, uint8_t *s8) {
  const int N = (m == 2) ? w->H : w->I;
  const int K = (m == 2) ? w->I : w->H;
#pragma omp parallel for schedule(static)
  for (int row = 0; row < w->E * N; ++row) {
    const int e = row / N, n = row % N;
    double *v = (double *)malloc(sizeof(double) * (size_t)K);
    for (int kk = 0; kk < K; ++kk) v[kk] = oracle_weight(w, e, m, n, kk);
    oracle_mx8_quant(v, K, q8 + (size_t)row * K, s8 + (size_t)row * (K / 32));
    free(v);
  }
}

static double mx8_value(const uint8_t *q, const uint8_t *s, int K, size_t row, int kk) {
  return oracle_e4m3(q[row * K + kk]) * oracle_mx_scale(s[row * (K / 32) + kk / 32]);
}

/* Expert e's FFN on token rows tok[0..nrows) in the fp8 variant: x rows -> MXFP8; gate/up with
 * the MXFP8 weights (exact products, sums in double); h = silu(g) * u -> MXFP8; down -> y. */
void oracle_expert_rows_mx(const uint16_t *x, int H, int I, int e, const uint8_t *gq,
                           const uint8_t *gs, const uint8_t *uq, const uint8_t *us,
                           const uint8_t *dq, const uint8_t *ds, const int32_t *tok, int nrows,
                           double *y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < nrows; ++r) {
    const int L = H > I ? H : I;
    double *xv = (double *)malloc(sizeof(double) * (size_t)H);
    double *hv = (double *)malloc(sizeof(double) * (size_t)I);
    uint8_t *c8 = (uint8_t *)malloc((size_t)L);
    uint8_t *s8 = (uint8_t *)malloc((size_t)L / 32);
    for (int k = 0; k < H; ++k) xv[k] = oracle_bf16(x[(size_t)tok[r] * H + k]);
    oracle_mx8_quant(xv, H, c8, s8);
    for (int k = 0; k < H; ++k) xv[k] = oracle_e4m3(c8[k]) * oracle_mx_scale(s8[k / 32]);
    for (int f = 0; f < I; ++f) {
      double g = 0.0, u = 0.0;
      const size_t row = (size_t)e * I + f;
      for (int k = 0; k < H; ++k) {
        g += xv[k] * mx8_value(gq, gs, H, row, k);
        u += xv[k] * mx8_value(uq, us, H, row, k);
      }
      hv[f] = g / (1.0 + exp(-g)) * u;
    }
    oracle_mx8_quant(hv, I, c8, s8);
    for (int f = 0; f < I; ++f) hv[f] = oracle_e4m3(c8[f]) * oracle_mx_scale(s8[f / 32]);
    for (int n = 0; n < H; ++n) {
      double acc = 0.0;
      const size_t row = (size_t)e * H + n;
      for (int f = 0; f < I; ++f) acc += hv[f] * mx8_value(dq, ds, I, row, f);
      y[(size_t)r * H + n] = acc;
    }
    free(xv);
    free(hv);
    free(c8);
    free(s8);
  }
}
