/*
 * moe_oracle.c -- plain, slow CPU oracle of the local-expert MoE block.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library never
 * links, calls or reads it, and it shares no code, header, table or constant
 * generator with the GPU kernels.
 *
 * What it computes (one rank's local experts, S token rows):
 *   1. router logits in fp64, sigmoid scores, top-k, renormalised weights
 *      (Muse Spark K3 page, stages "A" and "route"; K5 page, the HA routing
 *      tail: fp32 router, top-8 per token);
 *   2. bucketing of the picks that land on the local experts
 *      (K3 page, stage "route" and function "dn_loads": active-expert table);
 *   3. per pick: MXFP4 gate_up GEMM, SwiGLU, MXFP4 down GEMM
 *      (K3 page, stages "C, D": MXFP4 weights decoded, bf16 MFMA);
 *   4. per-pick RMSNorm of the expert output
 *      (K3 page, stage "E"; the RMSNorm form of the KDA page, "kda_norm");
 *   5. the routing-weighted sum into an fp32 partial (K3 page, stage "E");
 *   6. around the block: the dense latent projection before it and its norm,
 *      and the projection of the summed partial after it (K5 page, HA and
 *      HB; K3 page, stages "A" and "F").
 *
 * Precision: every sum is an fp64 sum in index order; the products of bf16 or
 * fp32 inputs with decoded MXFP4 weights are exact in fp64. The KDA page's
 * module docstring states the rounding rule of these kernels: elementwise
 * rounding matches the unfused path wherever one stage hands bf16 data to the
 * next, and only split-K sums may change order. So values are rounded to bf16
 * (nearest, ties to even) at exactly those points here: the gate_up output, the
 * SwiGLU output and the down output. Routing weights and the final partial are
 * rounded to fp32; the normalised expert output is not rounded.
 *
 * Readings where the pages are silent (each one is a choice, listed with its
 * reason in the design notes):
 *   - the router bias is added to the logit before ranking and sigmoid
 *     (bias_mode 0); the K3 page's one-line summary of "route_token" breaks
 *     off after "sigmoid +", so the other reading, a bias that steers the selection only
 *     while the weights come from the sigmoid of the unbiased logit, is kept
 *     as bias_mode 1 (orc_topk_sel);
 *   - equal logits: the lower expert id ranks first;
 *   - renormalisation is over all k picks, local or not;
 *   - rows [0, I) of gate_up are the gate, rows [I, 2I) the up projection;
 *     SwiGLU is silu(gate) * up with silu(g) = g / (1 + exp(-g));
 *   - RMSNorm: z = y / sqrt(mean(y^2) + eps) * gamma, one gamma for all experts;
 *   - the always-on shared expert (bf16 weights) is added with weight 1, after
 *     the routed picks, without the per-pick norm.
 *
 * MXFP4 element decoding follows the OCP Microscaling (MX) v1.0 formats (an
 * outside definition: the pages only name MXFP4 and e8m0): e2m1 = [sign | 2-bit
 * exponent | 1-bit mantissa], bias 1; e8m0 = 2^(X - 127), 0xFF = NaN.
 *
 * Parity of every function here is pinned by tests against closed forms,
 * library routines and brute force; see the tests for which pin covers what.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* Threads: the batch functions (router logits, top-k, the expert FFN over
 * bucket rows, the combine over tokens, the projections) and the rows of one
 * GEMV run their independent outputs on OpenMP threads; every output value
 * is still computed by one thread in the order written below, so results do
 * not depend on the thread count. */
void orc_set_threads(int n) {
  if (n > 0) omp_set_num_threads(n);
}
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp64                                                             */
/* ------------------------------------------------------------------------ */

double orc_bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round v to the nearest bf16 (8 significant bits, fp32's exponent range,
 * subnormals down to 2^-133), ties to the even significand. */
uint16_t orc_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  int neg = signbit(v) != 0;
  uint16_t sign = neg ? 0x8000 : 0;
  if (isinf(v)) return sign | 0x7F80;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e = ilogb(a); /* a in [2^e, 2^(e+1)) */
  if (e < -126) e = -126; /* subnormal: fixed spacing 2^-133 */
  double q = ldexp(1.0, e - 7); /* spacing of bf16 values at this exponent */
  double r = nearbyint(a / q) * q; /* default rounding mode: ties to even */
  if (r >= 0x1p128) return sign | 0x7F80;
  float f = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* MXFP4 decode [ext: OCP MX v1.0]                                           */
/* ------------------------------------------------------------------------ */

/* e2m1: bit 3 sign, bits 2..1 exponent E, bit 0 mantissa M.
 * E = 0: subnormal, M * 0.5; E > 0: 2^(E-1) * (1 + M / 2). */
double orc_e2m1(unsigned nib) {
  unsigned s = (nib >> 3) & 1u, E = (nib >> 1) & 3u, M = nib & 1u;
  double mag = (E == 0) ? 0.5 * (double)M : ldexp(1.0 + 0.5 * (double)M, (int)E - 1);
  return s ? -mag : mag;
}

/* e8m0: 2^(X - 127); X = 0xFF is NaN. */
double orc_e8m0(unsigned x) {
  x &= 0xFFu;
  if (x == 0xFFu) return NAN;
  return ldexp(1.0, (int)x - 127);
}

/* Element k of one MXFP4 row: nibble k (low nibble of byte k/2 for even k),
 * scaled by scale byte k/32, as the number the expert GEMMs multiply. The K3
 * page (stages "C, D") decodes MXFP4 in registers into the bf16 operands of
 * the MFMA; bf16 and fp32 share one exponent range, and an e2m1 value times
 * 2^(X-127) has at most two significant bits and lies at or above 2^-128, so
 * the decoded value is exact in either format unless its magnitude reaches
 * 2^128 (scale bytes 253 and 254), where it overflows to infinity. Rounding
 * the exact product to fp32 states exactly that. */
double orc_mx_elem(const uint8_t* q_row, const uint8_t* s_row, long k) {
  uint8_t byte = q_row[k >> 1];
  unsigned nib = (k & 1) ? (byte >> 4) : (byte & 0xFu);
  return (double)(float)(orc_e2m1(nib) * orc_e8m0(s_row[k >> 5]));
}

/* ------------------------------------------------------------------------ */
/* 1. routing                                                                */
/* ------------------------------------------------------------------------ */

/* logits[t][e] = sum_j x[t][j] * wr[e][j] (+ bias[e]) */
int orc_router_logits(int S, int d, int E, const uint16_t* x, const float* wr,
                      const float* bias, double* logits) {
  if (S < 0 || d <= 0 || E <= 0 || !x || !wr || !logits) return ORC_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < S; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j)
        acc += orc_bf16_to_f64(x[(long)t * d + j]) * (double)wr[(long)e * d + j];
      if (bias) acc += (double)bias[e];
      logits[(long)t * E + e] = acc;
    }
  return ORC_OK;
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* Routing weights of the given picks: sigmoid of their logits, divided by the
 * sum over the token's k picks when renorm is set. */
int orc_route_weights(int S, int E, int topk, int renorm, const double* logits,
                      const int32_t* ids, float* w) {
  if (S < 0 || E <= 0 || topk <= 0 || topk > E || !logits || !ids || !w) return ORC_EINVAL;
  for (int t = 0; t < S; ++t) {
    double s[256], sum = 0.0;
    if (topk > 256) return ORC_EINVAL;
    for (int i = 0; i < topk; ++i) {
      int e = ids[t * topk + i];
      if (e < 0 || e >= E) return ORC_EINVAL;
      s[i] = sigmoid(logits[(long)t * E + e]);
      sum += s[i];
    }
    for (int i = 0; i < topk; ++i) w[t * topk + i] = (float)(renorm ? s[i] / sum : s[i]);
  }
  return ORC_OK;
}

/* Top-k by repeated selection: slot i holds the largest logit not yet taken,
 * equal logits to the lower id. Then the routing weights. */
int orc_topk(int S, int E, int topk, int renorm, const double* logits, int32_t* ids,
             float* w) {
  if (S < 0 || E <= 0 || E > 4096 || topk <= 0 || topk > E || !logits || !ids) return ORC_EINVAL;
  for (int t = 0; t < S; ++t) {
    unsigned char taken[4096];
    memset(taken, 0, (size_t)E);
    const double* l = logits + (long)t * E;
    for (int i = 0; i < topk; ++i) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict: ties keep the lower id */
      }
      taken[best] = 1;
      ids[t * topk + i] = best;
    }
  }
  return w ? orc_route_weights(S, E, topk, renorm, logits, ids, w) : ORC_OK;
}

/* Selection-only bias (bias_mode 1): the picks are the top-k of the scores
 * logits + bias (fp64, equal scores to the lower id), the weights are the
 * sigmoids of the unbiased logits of those picks. */
int orc_topk_sel(int S, int E, int topk, int renorm, const double* logits, const float* bias,
                 int32_t* ids, float* w) {
  if (S < 0 || E <= 0 || E > 4096 || topk <= 0 || topk > E || !logits || !bias || !ids)
    return ORC_EINVAL;
  double* score = (double*)malloc(sizeof(double) * ((size_t)S * E + 1));
  if (!score) return ORC_EINVAL;
  for (int t = 0; t < S; ++t)
    for (int e = 0; e < E; ++e) score[(long)t * E + e] = logits[(long)t * E + e] + (double)bias[e];
  int rc = orc_topk(S, E, topk, renorm, score, ids, NULL);
  free(score);
  if (rc || !w) return rc;
  return orc_route_weights(S, E, topk, renorm, logits, ids, w);
}

/* ------------------------------------------------------------------------ */
/* 2. bucketing                                                              */
/* ------------------------------------------------------------------------ */

/* For each local expert el (id local_base + el) in ascending order, the
 * tokens that picked it, ascending. Outputs:
 *   counts[n_loc], offsets[n_loc + 1] (exclusive prefix sums),
 *   rows[S * min(topk, n_loc)]: token of each bucket row, -1 past the end,
 *   pick_pos[S][topk]: bucket row of each pick, -1 if not local,
 *   active[1 + n_loc]: number of experts with a pick, then their local
 *   indices ascending, -1 after.
 * A token's ids must be distinct (as top-k produces them). */
int orc_bucket(int S, int topk, int n_loc, int local_base, const int32_t* ids,
               int32_t* counts, int32_t* offsets, int32_t* rows, int32_t* pick_pos,
               int32_t* active) {
  if (S < 0 || topk <= 0 || n_loc <= 0 || !ids || !counts || !offsets || !rows || !pick_pos ||
      !active)
    return ORC_EINVAL;
  for (int t = 0; t < S; ++t)
    for (int i = 0; i < topk; ++i)
      for (int j = 0; j < i; ++j)
        if (ids[t * topk + i] == ids[t * topk + j]) return ORC_EINVAL;
  int kk = topk < n_loc ? topk : n_loc;
  for (long r = 0; r < (long)S * kk; ++r) rows[r] = -1;
  for (long p = 0; p < (long)S * topk; ++p) pick_pos[p] = -1;
  for (int i = 0; i <= n_loc; ++i) active[i] = -1;
  int pos = 0, nv = 0;
  for (int el = 0; el < n_loc; ++el) {
    offsets[el] = pos;
    for (int t = 0; t < S; ++t)
      for (int i = 0; i < topk; ++i)
        if (ids[t * topk + i] == local_base + el) {
          rows[pos] = t;
          pick_pos[t * topk + i] = pos;
          ++pos;
        }
    counts[el] = pos - offsets[el];
    if (counts[el] > 0) active[1 + nv++] = el;
  }
  offsets[n_loc] = pos;
  active[0] = nv;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 3. the expert FFN of one pick                                              */
/* ------------------------------------------------------------------------ */

static double silu(double g) { return g / (1.0 + exp(-g)); }

/* gate_up and SwiGLU of one token row through one MXFP4 expert:
 *   gu[n] = bf16( sum_j x[j] * W13[n][j] ),             n < 2I
 *   h[i]  = bf16( silu(gu[i]) * gu[I + i] ),           i < I
 * w13q [2I][d/2], w13s [2I][d/32] are this expert's slices; gu may be NULL. */
int orc_mx_gate_up(int d, int I, const uint16_t* x, const uint8_t* w13q, const uint8_t* w13s,
                   uint16_t* gu_out, uint16_t* h) {
  if (d <= 0 || I <= 0 || (d % 32) || !x || !w13q || !w13s || !h) return ORC_EINVAL;
  uint16_t* gu = (uint16_t*)malloc(sizeof(uint16_t) * 2 * (size_t)I);
  if (!gu) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < 2 * I; ++n) {
    const uint8_t* qr = w13q + (long)n * (d / 2);
    const uint8_t* sr = w13s + (long)n * (d / 32);
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += orc_bf16_to_f64(x[j]) * orc_mx_elem(qr, sr, j);
    gu[n] = orc_f64_to_bf16(acc);
  }
  for (int i = 0; i < I; ++i) {
    double g = orc_bf16_to_f64(gu[i]), u = orc_bf16_to_f64(gu[I + i]);
    h[i] = orc_f64_to_bf16(silu(g) * u);
  }
  if (gu_out) memcpy(gu_out, gu, sizeof(uint16_t) * 2 * (size_t)I);
  free(gu);
  return ORC_OK;
}

/* down of one SwiGLU row through one MXFP4 expert:
 *   y[c] = bf16( sum_i h[i] * W2[c][i] ),  c < d;  w2q [d][I/2], w2s [d][I/32]. */
int orc_mx_down(int d, int I, const uint16_t* h, const uint8_t* w2q, const uint8_t* w2s,
                uint16_t* y) {
  if (d <= 0 || I <= 0 || (I % 32) || !h || !w2q || !w2s || !y) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int c = 0; c < d; ++c) {
    const uint8_t* qr = w2q + (long)c * (I / 2);
    const uint8_t* sr = w2s + (long)c * (I / 32);
    double acc = 0.0;
    for (int i = 0; i < I; ++i) acc += orc_bf16_to_f64(h[i]) * orc_mx_elem(qr, sr, i);
    y[c] = orc_f64_to_bf16(acc);
  }
  return ORC_OK;
}

/* One token row through one MXFP4 expert: gate_up, SwiGLU, down. gu and h may
 * be NULL. */
int orc_expert_row(int d, int I, const uint16_t* x, const uint8_t* w13q,
                   const uint8_t* w13s, const uint8_t* w2q, const uint8_t* w2s,
                   uint16_t* gu_out, uint16_t* h_out, uint16_t* y) {
  if (I <= 0 || !y) return ORC_EINVAL;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)I);
  if (!h) return ORC_EINVAL;
  int rc = orc_mx_gate_up(d, I, x, w13q, w13s, gu_out, h);
  if (!rc) rc = orc_mx_down(d, I, h, w2q, w2s, y);
  if (!rc && h_out) memcpy(h_out, h, sizeof(uint16_t) * (size_t)I);
  free(h);
  return rc;
}

/* The same two steps with dense bf16 weights: ws13 [2 Is][d], ws2 [d][Is]. */
int orc_bf_gate_up(int d, int Is, const uint16_t* x, const uint16_t* ws13, uint16_t* gu_out,
                   uint16_t* h) {
  if (d <= 0 || Is <= 0 || !x || !ws13 || !h) return ORC_EINVAL;
  uint16_t* gu = (uint16_t*)malloc(sizeof(uint16_t) * 2 * (size_t)Is);
  if (!gu) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < 2 * Is; ++n) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j)
      acc += orc_bf16_to_f64(x[j]) * orc_bf16_to_f64(ws13[(long)n * d + j]);
    gu[n] = orc_f64_to_bf16(acc);
  }
  for (int i = 0; i < Is; ++i) {
    double g = orc_bf16_to_f64(gu[i]), u = orc_bf16_to_f64(gu[Is + i]);
    h[i] = orc_f64_to_bf16(silu(g) * u);
  }
  if (gu_out) memcpy(gu_out, gu, sizeof(uint16_t) * 2 * (size_t)Is);
  free(gu);
  return ORC_OK;
}

int orc_bf_down(int d, int Is, const uint16_t* h, const uint16_t* ws2, uint16_t* y) {
  if (d <= 0 || Is <= 0 || !h || !ws2 || !y) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int c = 0; c < d; ++c) {
    double acc = 0.0;
    for (int i = 0; i < Is; ++i)
      acc += orc_bf16_to_f64(h[i]) * orc_bf16_to_f64(ws2[(long)c * Is + i]);
    y[c] = orc_f64_to_bf16(acc);
  }
  return ORC_OK;
}

int orc_shared_row(int d, int Is, const uint16_t* x, const uint16_t* ws13,
                   const uint16_t* ws2, uint16_t* gu_out, uint16_t* h_out, uint16_t* y) {
  if (Is <= 0 || !y) return ORC_EINVAL;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)Is);
  if (!h) return ORC_EINVAL;
  int rc = orc_bf_gate_up(d, Is, x, ws13, gu_out, h);
  if (!rc) rc = orc_bf_down(d, Is, h, ws2, y);
  if (!rc && h_out) memcpy(h_out, h, sizeof(uint16_t) * (size_t)Is);
  free(h);
  return rc;
}

/* Every bucket row through its expert, then (Is > 0) every token through the
 * shared expert. y: [R_max + (Is ? S : 0)][d] with R_max = S * min(topk, n_loc);
 * bucket row r at row r, token t's shared output at row R_max + t. Rows past
 * the bucket total are left untouched. */
int orc_expert_ffn(int S, int d, int I, int n_loc, int topk, int Is, const uint16_t* x,
                   const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                   const uint8_t* w2s, const int32_t* counts, const int32_t* offsets,
                   const int32_t* rows, const uint16_t* ws13, const uint16_t* ws2,
                   uint16_t* y) {
  if (S < 0 || !x || !counts || !offsets || !rows || !y) return ORC_EINVAL;
  if (Is > 0 && (!ws13 || !ws2)) return ORC_EINVAL;
  int kk = topk < n_loc ? topk : n_loc;
  long R_max = (long)S * kk;
  size_t e13q = (size_t)2 * I * (d / 2), e13s = (size_t)2 * I * (d / 32);
  size_t e2q = (size_t)d * (I / 2), e2s = (size_t)d * (I / 32);
  /* the bucket rows to run, with their experts (checked before any work) */
  long n_rows = 0;
  for (int el = 0; el < n_loc; ++el) {
    if (counts[el] < 0 || offsets[el] < 0 || offsets[el] + counts[el] > R_max) return ORC_EINVAL;
    n_rows += counts[el];
  }
  int32_t* row_el = (int32_t*)malloc(sizeof(int32_t) * (size_t)(2 * n_rows + 1));
  if (!row_el) return ORC_EINVAL;
  int32_t* row_r = row_el + n_rows;
  long i = 0;
  for (int el = 0; el < n_loc; ++el)
    for (int r = offsets[el]; r < offsets[el] + counts[el]; ++r) {
      if (rows[r] < 0 || rows[r] >= S) {
        free(row_el);
        return ORC_EINVAL;
      }
      row_el[i] = el;
      row_r[i++] = r;
    }
  /* every bucket row, then every token through the shared expert: independent
   * rows, one thread each */
  long n_tasks = n_rows + (Is > 0 ? S : 0);
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long j = 0; j < n_tasks; ++j) {
    if (j < n_rows) {
      int el = row_el[j], r = row_r[j], t = rows[r];
      bad |= orc_expert_row(d, I, x + (long)t * d, w13q + el * e13q, w13s + el * e13s,
                            w2q + el * e2q, w2s + el * e2s, NULL, NULL, y + (long)r * d) != 0;
    } else {
      int t = (int)(j - n_rows);
      bad |= orc_shared_row(d, Is, x + (long)t * d, ws13, ws2, NULL, NULL,
                            y + (R_max + t) * d) != 0;
    }
  }
  free(row_el);
  return bad ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 4. per-pick RMSNorm, 5. weighted sum                                      */
/* ------------------------------------------------------------------------ */

/* z[c] = y[c] / sqrt(mean_c y^2 + eps) * gamma[c] (gamma NULL = ones) */
int orc_norm_row(int d, const uint16_t* y, const uint16_t* gamma, double eps, double* z) {
  if (d <= 0 || !y || !z) return ORC_EINVAL;
  double ss = 0.0;
  for (int c = 0; c < d; ++c) {
    double v = orc_bf16_to_f64(y[c]);
    ss += v * v;
  }
  double r = 1.0 / sqrt(ss / (double)d + eps);
  for (int c = 0; c < d; ++c)
    z[c] = orc_bf16_to_f64(y[c]) * r * (gamma ? orc_bf16_to_f64(gamma[c]) : 1.0);
  return ORC_OK;
}

/* out[t][c] = fp32( sum over t's picks in slot order with pick_pos >= 0 of
 *                   w[t][slot] * z_pick[c]  (+ y[R_max + t][c] if Is > 0) ).
 * Tokens without a local pick (and no shared expert) get 0. */
int orc_combine(int S, int d, int topk, int n_loc, int Is, float eps, const uint16_t* y,
                const float* w, const int32_t* pick_pos, const uint16_t* gamma, float* out) {
  if (S < 0 || d <= 0 || !y || !w || !pick_pos || !out) return ORC_EINVAL;
  int kk = topk < n_loc ? topk : n_loc;
  long R_max = (long)S * kk;
  for (long p = 0; p < (long)S * topk; ++p)
    if (pick_pos[p] >= R_max) return ORC_EINVAL;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int t = 0; t < S; ++t) {
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    double* z = (double*)malloc(sizeof(double) * (size_t)d);
    if (!acc || !z) {
      free(acc);
      free(z);
      bad = 1;
      continue;
    }
    for (int c = 0; c < d; ++c) acc[c] = 0.0;
    for (int i = 0; i < topk; ++i) {
      int p = pick_pos[t * topk + i];
      if (p < 0) continue;
      orc_norm_row(d, y + (long)p * d, gamma, (double)eps, z);
      double wt = (double)w[t * topk + i];
      for (int c = 0; c < d; ++c) acc[c] += wt * z[c];
    }
    if (Is > 0)
      for (int c = 0; c < d; ++c) acc[c] += orc_bf16_to_f64(y[(R_max + t) * d + c]);
    for (int c = 0; c < d; ++c) out[(long)t * d + c] = (float)acc[c];
    free(acc);
    free(z);
  }
  return bad ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 6. the latent projections around the block                                */
/* ------------------------------------------------------------------------ */

/* K5 page, HA routing tail: ffn_in feeds both the router and pre_expert_proj,
 * a dense bf16 projection into the latent the experts run on, and the
 * projection is normalised (pre_expert_norm) before the experts. K3 page,
 * stage "F", and K5 page, HB: post_expert_proj maps the summed expert partial
 * back. (The Kimi-K3 layer page's latent MoE has the same chain: "k2_launch"
 * takes w_ld, ln_w and w_up.) */

/* out[t][n] = bf16( sum_k in[t][k] * w[n][k] ), in [S][K] and w [N][K] bf16 */
int orc_dense_proj(int S, int K, int N, const uint16_t* in, const uint16_t* w, uint16_t* out) {
  if (S < 0 || K <= 0 || N <= 0 || !in || !w || !out) return ORC_EINVAL;
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < S; ++t)
    for (int n = 0; n < N; ++n) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k)
        acc += orc_bf16_to_f64(in[(long)t * K + k]) * orc_bf16_to_f64(w[(long)n * K + k]);
      out[(long)t * N + n] = orc_f64_to_bf16(acc);
    }
  return ORC_OK;
}

/* pre_expert_norm: h[t][c] = bf16( h_raw[t][c] * r_t * gamma[c] ) with
 * r_t = (sum_c h_raw[t][c]^2 / L + eps)^(-1/2); gamma NULL = ones */
int orc_latent_norm(int S, int L, double eps, const uint16_t* h_raw, const uint16_t* gamma,
                    uint16_t* h) {
  if (S < 0 || L <= 0 || !h_raw || !h) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int t = 0; t < S; ++t) {
    double ss = 0.0;
    for (int c = 0; c < L; ++c) {
      double v = orc_bf16_to_f64(h_raw[(long)t * L + c]);
      ss += v * v;
    }
    double r = 1.0 / sqrt(ss / (double)L + eps);
    for (int c = 0; c < L; ++c) {
      double g = gamma ? orc_bf16_to_f64(gamma[c]) : 1.0;
      h[(long)t * L + c] = orc_f64_to_bf16(orc_bf16_to_f64(h_raw[(long)t * L + c]) * r * g);
    }
  }
  return ORC_OK;
}

/* post_expert_proj: the fp32 partial is handed to the bf16 GEMM rounded to
 * bf16, then out = orc_dense_proj of it */
int orc_post_proj(int S, int K, int N, const float* partial, const uint16_t* w, uint16_t* out) {
  if (S < 0 || K <= 0 || N <= 0 || !partial || !w || !out) return ORC_EINVAL;
  uint16_t* in = (uint16_t*)malloc(sizeof(uint16_t) * ((size_t)S * K + 1));
  if (!in) return ORC_EINVAL;
  for (long i = 0; i < (long)S * K; ++i) in[i] = orc_f64_to_bf16((double)partial[i]);
  int rc = orc_dense_proj(S, K, N, in, w, out);
  free(in);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* the whole block                                                           */
/* ------------------------------------------------------------------------ */

/* route -> bucket -> expert FFN -> combine, all outputs caller-owned:
 * bias_mode 0: the bias is part of the logit; 1: it steers the selection only
 * (logits are then written without it);
 * logits [S][E] fp64, ids/w [S][topk], counts [n_loc], offsets [n_loc+1],
 * rows [R_max], pick_pos [S][topk], active [1+n_loc], y [R_max (+S)][d],
 * out [S][d]. */
int orc_forward(int S, int d, int E, int topk, int n_loc, int local_base, int I, int renorm,
                float eps, int Is, int bias_mode, const uint16_t* x, const float* wr,
                const float* bias,
                const uint8_t* w13q, const uint8_t* w13s, const uint8_t* w2q,
                const uint8_t* w2s, const uint16_t* gamma, const uint16_t* ws13,
                const uint16_t* ws2, double* logits, int32_t* ids, float* w, int32_t* counts,
                int32_t* offsets, int32_t* rows, int32_t* pick_pos, int32_t* active,
                uint16_t* y, float* out) {
  if (bias_mode != 0 && bias_mode != 1) return ORC_EINVAL;
  const int sel = bias_mode == 1 && bias;
  int rc = orc_router_logits(S, d, E, x, wr, sel ? NULL : bias, logits);
  if (!rc)
    rc = sel ? orc_topk_sel(S, E, topk, renorm, logits, bias, ids, w)
             : orc_topk(S, E, topk, renorm, logits, ids, w);
  if (!rc) rc = orc_bucket(S, topk, n_loc, local_base, ids, counts, offsets, rows, pick_pos, active);
  if (!rc)
    rc = orc_expert_ffn(S, d, I, n_loc, topk, Is, x, w13q, w13s, w2q, w2s, counts, offsets,
                        rows, ws13, ws2, y);
  if (!rc) rc = orc_combine(S, d, topk, n_loc, Is, eps, y, w, pick_pos, gamma, out);
  return rc;
}
