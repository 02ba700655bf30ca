/*
 * moe_oracle.c -- scalar CPU oracle of the routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg use it. It is independent of the GPU library:
 * no shared code, headers, tables or constants.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (every
 * floating-point operation below is a single correctly rounded IEEE
 * operation, and fused multiply-adds appear only where fmaf() is written
 * out). OpenMP only spreads the layer's independent (token, slot) pairs over
 * threads; it changes no arithmetic.
 *
 * Function-to-page map (full citations in moe_oracle.h):
 *  O1 quantise/pack rows ...... agentlenshq "Key features": packed int4 /
 *                               int8 / int2 with per-row scales.
 *  O2 activation quantisation . agentlenshq "Key features": int8 matmuls run
 *                               as integer dot products (int8 operands).
 *  O3 router .................. takumi3488 "self-test" section: a
 *                               DeepSeek-V3-family router; remio "How Colibri
 *                               runs GLM-5.2": a few experts per token.
 *  O4 bucketing ............... remio "The RAM wall became a storage
 *                               problem": one read per expert per batch.
 *  O5 expert FFN .............. agentlenshq "Key features" (dequantisation
 *                               on use, integer dot) and "Memory split"
 *                               (about 19 MB per int4 expert = three
 *                               6144 x 2048 matrices: gate, up, down).
 *  O6 shared expert ........... agentlenshq "Memory split": shared experts
 *                               are resident and always used.
 *  O7 combine ................. remio "How Colibri runs GLM-5.2".
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* O1 / O2: per-row symmetric absmax quantisation                            */
/* ------------------------------------------------------------------------ */

static int qmax_of(int bits) {
  switch (bits) {
    case 8: return 127;
    case 4: return 7;
    case 2: return 1;
    default: return -1;
  }
}

/* Quantise one row to signed codes (steps 1-2 of O1). */
static float quantize_row(const float *w, int cols, int qmax, int8_t *q) {
  float a = 0.0f;
  for (int c = 0; c < cols; ++c) {
    float v = fabsf(w[c]);
    if (v > a) a = v;
  }
  if (a == 0.0f) {
    memset(q, 0, (size_t)cols);
    return 0.0f;
  }
  float s = a / (float)qmax; /* one correctly rounded fp32 division */
  for (int c = 0; c < cols; ++c) {
    float r = rintf(w[c] / s); /* fp32 division, then round half to even */
    if (r > (float)qmax) r = (float)qmax;
    if (r < (float)-qmax) r = (float)-qmax;
    q[c] = (int8_t)r;
  }
  return s;
}

int orc_quantize_rows(int bits, const float *w, int64_t rows, int cols, uint8_t *packed, float *scales) {
  int qmax = qmax_of(bits);
  if (qmax < 0 || cols <= 0 || rows < 0 || (cols * bits) % 8 != 0) return -1;
  const int per_byte = 8 / bits;
  const int row_bytes = cols * bits / 8;
  int8_t *q = (int8_t *)malloc((size_t)cols);
  if (!q) return -2;
  for (int64_t r = 0; r < rows; ++r) {
    scales[r] = quantize_row(w + r * (int64_t)cols, cols, qmax, q);
    uint8_t *dst = packed + r * (int64_t)row_bytes;
    for (int b = 0; b < row_bytes; ++b) {
      unsigned byte = 0;
      for (int j = 0; j < per_byte; ++j) {
        int code = q[b * per_byte + j];
        unsigned field;
        if (bits == 8)
          field = (unsigned)(uint8_t)(int8_t)code; /* two's complement */
        else
          field = (unsigned)(code + qmax + 1);     /* offset binary: q+8 or q+2 */
        byte |= field << (j * bits);
      }
      dst[b] = (uint8_t)byte;
    }
  }
  free(q);
  return 0;
}

int orc_unpack_rows(int bits, const uint8_t *packed, int64_t rows, int cols, int8_t *q) {
  int qmax = qmax_of(bits);
  if (qmax < 0 || cols <= 0 || (cols * bits) % 8 != 0) return -1;
  const int per_byte = 8 / bits;
  const int row_bytes = cols * bits / 8;
  const unsigned mask = (1u << bits) - 1u;
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t *src = packed + r * (int64_t)row_bytes;
    int8_t *dst = q + r * (int64_t)cols;
    for (int c = 0; c < cols; ++c) {
      unsigned byte = src[c / per_byte];
      unsigned field = (byte >> ((c % per_byte) * bits)) & mask;
      if (bits == 8)
        dst[c] = (int8_t)(uint8_t)field;
      else
        dst[c] = (int8_t)((int)field - (qmax + 1));
    }
  }
  return 0;
}

int orc_quantize_act(const float *x, int T, int H, int8_t *xq, float *sx) {
  if (T < 0 || H <= 0) return -1;
  for (int t = 0; t < T; ++t) sx[t] = quantize_row(x + (int64_t)t * H, H, 127, xq + (int64_t)t * H);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* exp / SiLU in fp32                                                       */
/* ------------------------------------------------------------------------ */

/* Cody-Waite reduction constants derived from ln 2 = 0.693147180559945309417...:
 * LN2_HI is ln 2 truncated to 16 fractional bits (45426 / 2^16, exact in
 * fp32 with trailing zero bits); LN2_LO is the rest, rounded to fp32. */
#define ORC_LN2 0.6931471805599453094172321
#define ORC_LN2_HI_D (45426.0 / 65536.0)

float orc_exp_f32(float x) {
  const float log2e = (float)1.4426950408889634073599247;
  const float ln2_hi = (float)ORC_LN2_HI_D;
  const float ln2_lo = (float)(ORC_LN2 - ORC_LN2_HI_D);
  if (isnan(x)) return x;
  if (x > 88.75f) return INFINITY;
  if (x < -104.0f) return 0.0f;
  float n = rintf(x * log2e);
  float r = fmaf(-n, ln2_hi, x);
  r = fmaf(-n, ln2_lo, r);
  /* e^r = sum_{j=0..7} r^j / j!, Horner form starting at 1/7! = 1/5040 */
  float p = (float)(1.0 / 5040.0);
  p = fmaf(p, r, (float)(1.0 / 720.0));
  p = fmaf(p, r, (float)(1.0 / 120.0));
  p = fmaf(p, r, (float)(1.0 / 24.0));
  p = fmaf(p, r, (float)(1.0 / 6.0));
  p = fmaf(p, r, 0.5f);
  p = fmaf(p, r, 1.0f);
  p = fmaf(p, r, 1.0f);
  return ldexpf(p, (int)n);
}

float orc_silu_f32(float g) {
  float e = orc_exp_f32(-g);
  return g / (1.0f + e);
}

/* ------------------------------------------------------------------------ */
/* O3: router                                                               */
/* ------------------------------------------------------------------------ */

int orc_router(int logits_in, const float *x, const float *wr, const float *bias, int T, int H, int E, int k,
               double routed_scale, int32_t *idx, float *w, double *keys_out, double *sig_out) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  if (!logits_in && (H <= 0 || !wr)) return -1;
  double *sig = (double *)malloc(sizeof(double) * (size_t)E);
  double *key = (double *)malloc(sizeof(double) * (size_t)E);
  char *taken = (char *)malloc((size_t)E);
  if (!sig || !key || !taken) return -2;
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double z;
      if (logits_in) {
        z = (double)x[(int64_t)t * E + e];
      } else {
        z = 0.0;
        const float *xr = x + (int64_t)t * H;
        const float *wrow = wr + (int64_t)e * H;
        for (int h = 0; h < H; ++h) z += (double)xr[h] * (double)wrow[h];
      }
      sig[e] = 1.0 / (1.0 + exp(-z));
      key[e] = sig[e] + (bias ? (double)bias[e] : 0.0);
      if (keys_out) keys_out[(int64_t)t * E + e] = key[e];
      if (sig_out) sig_out[(int64_t)t * E + e] = sig[e];
    }
    /* k rounds of "largest remaining key, lowest id on equality" */
    memset(taken, 0, (size_t)E);
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || key[e] > key[best]) best = e;
      }
      taken[best] = 1;
      idx[(int64_t)t * k + j] = best;
      sum += sig[best];
    }
    for (int j = 0; j < k; ++j) {
      int e = idx[(int64_t)t * k + j];
      w[(int64_t)t * k + j] = (float)(routed_scale * sig[e] / sum);
    }
  }
  free(sig);
  free(key);
  free(taken);
  return 0;
}

/* Top-p truncation of a top-k selection (agentlenshq.com, "Colibri: running
 * GLM-5.2 744B MoE on consumer hardware", sections "Measured benchmarks" and
 * community insights: the --topp 0.7 setting that loads fewer experts per
 * token). Reading: in rank order, the normalised weights sigma_j / sum_k sigma
 * accumulate; the shortest prefix whose cumulative weight reaches top_p is
 * kept (all k if none does), its weights renormalised over the kept experts;
 * dropped slots get id -1 and weight 0. top_p <= 0 leaves the selection as it
 * is. sig: [T][E] sigmoids (fp64) as orc_router returns them; idx [T][k] in,
 * out; w [T][k] out; cum_out [T][k] (nullable) the cumulative weights. */
int orc_topp(int T, int E, int k, const double *sig, double routed_scale, double top_p, int32_t *idx, float *w,
             double *cum_out) {
  if (T < 0 || E <= 0 || k <= 0 || !sig || !idx || !w) return -1;
  for (int t = 0; t < T; ++t) {
    int32_t *id = idx + (int64_t)t * k;
    const double *sg = sig + (int64_t)t * E;
    double total = 0.0;
    for (int j = 0; j < k; ++j) total += sg[id[j]];
    double cum = 0.0;
    int keep = k;
    for (int j = 0; j < k; ++j) {
      cum += sg[id[j]] / total;
      if (cum_out) cum_out[(int64_t)t * k + j] = cum;
      if (keep == k && top_p > 0.0 && cum >= top_p) keep = j + 1;
    }
    if (top_p <= 0.0) continue;
    double kept = 0.0;
    for (int j = 0; j < keep; ++j) kept += sg[id[j]];
    for (int j = 0; j < k; ++j) {
      if (j < keep) {
        w[(int64_t)t * k + j] = (float)(routed_scale * sg[id[j]] / kept);
      } else {
        id[j] = -1;
        w[(int64_t)t * k + j] = 0.0f;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O4: bucketing                                                            */
/* ------------------------------------------------------------------------ */

int orc_bucket(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets, int32_t *perm) {
  if (T < 0 || k <= 0 || E <= 0) return -1;
  int64_t n = (int64_t)T * k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (idx[i] < 0 || idx[i] >= E) return -1;
    counts[idx[i]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!cursor) return -2;
  for (int64_t i = 0; i < n; ++i) { /* i = t*k + j, ascending (t, j) */
    int e = idx[i];
    perm[offsets[e] + cursor[e]++] = (int32_t)i;
  }
  free(cursor);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* O5 / O6: one expert on one token                                         */
/* ------------------------------------------------------------------------ */

/* Signed code of element c of a packed row (the inverse of O1's packing). */
static inline int code_at(int bits, const uint8_t *row, int c) {
  switch (bits) {
    case 8: return (int8_t)row[c];
    case 4: return (int)((row[c >> 1] >> ((c & 1) * 4)) & 0xF) - 8;
    default: return (int)((row[c >> 2] >> ((c & 3) * 2)) & 0x3) - 2;
  }
}

int orc_expert_token(int bits, const orc_expert *ex, const int8_t *xq_t, float sx_t, int H, int I, int32_t *accg,
                     int32_t *accu, float *a, int8_t *aq, float *sa, int32_t *accd, float *y) {
  if (qmax_of(bits) < 0 || H <= 0 || I <= 0 || !y) return -1;
  const int64_t rb_h = (int64_t)H * bits / 8; /* bytes per gate/up row */
  const int64_t rb_i = (int64_t)I * bits / 8; /* bytes per down row */
  float *av = (float *)malloc(sizeof(float) * (size_t)I);
  int8_t *aqv = (int8_t *)malloc((size_t)I);
  if (!av || !aqv) return -2;
  int rc = 0;
  for (int i = 0; i < I; ++i) {
    int64_t sg = 0, su = 0;
    const uint8_t *grow = ex->gate + i * rb_h;
    const uint8_t *urow = ex->up + i * rb_h;
    for (int h = 0; h < H; ++h) {
      sg += (int64_t)code_at(bits, grow, h) * xq_t[h];
      su += (int64_t)code_at(bits, urow, h) * xq_t[h];
    }
    if (sg > INT32_MAX || sg < INT32_MIN || su > INT32_MAX || su < INT32_MIN) rc = -3;
    if (accg) accg[i] = (int32_t)sg;
    if (accu) accu[i] = (int32_t)su;
    float g = (float)(int32_t)sg * ex->s_gate[i] * sx_t;
    float u = (float)(int32_t)su * ex->s_up[i] * sx_t;
    av[i] = orc_silu_f32(g) * u;
  }
  float s_a = quantize_row(av, I, 127, aqv);
  for (int r = 0; r < H; ++r) {
    int64_t sd = 0;
    const uint8_t *drow = ex->down + r * rb_i;
    for (int i = 0; i < I; ++i) sd += (int64_t)code_at(bits, drow, i) * aqv[i];
    if (sd > INT32_MAX || sd < INT32_MIN) rc = -3;
    if (accd) accd[r] = (int32_t)sd;
    y[r] = (float)(int32_t)sd * ex->s_down[r] * s_a;
  }
  if (a) memcpy(a, av, sizeof(float) * (size_t)I);
  if (aq) memcpy(aq, aqv, (size_t)I);
  if (sa) *sa = s_a;
  free(av);
  free(aqv);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* O7: combine                                                              */
/* ------------------------------------------------------------------------ */

int orc_combine(const float *y_slots, const float *w, int T, int k, int H, int has_shared, float *out) {
  if (T < 0 || k <= 0 || H <= 0) return -1;
  const int S = k + (has_shared ? 1 : 0);
  for (int t = 0; t < T; ++t) {
    const float *ys = y_slots + (int64_t)t * S * H;
    for (int h = 0; h < H; ++h) {
      double acc = has_shared ? (double)ys[(int64_t)k * H + h] : 0.0;
      for (int j = 0; j < k; ++j) acc += (double)w[(int64_t)t * k + j] * (double)ys[(int64_t)j * H + h];
      out[(int64_t)t * H + h] = (float)acc;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Full layer                                                               */
/* ------------------------------------------------------------------------ */

int orc_layer(const float *x, const float *logits, const float *wr, const float *bias, double routed_scale,
              const orc_expert *experts, const uint8_t *bits, const orc_expert *shared, int shared_bits, int T, int H,
              int I, int E, int k, double top_p, int8_t *xq, float *sx, int32_t *idx, float *w, float *y_slots,
              float *out) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k <= 0 || k > E || !out) return -1;
  double *sig = NULL;
  const int S = k + (shared ? 1 : 0);
  int8_t *xq_ = xq ? xq : (int8_t *)malloc((size_t)T * H);
  float *sx_ = sx ? sx : (float *)malloc(sizeof(float) * (size_t)T);
  int32_t *idx_ = idx ? idx : (int32_t *)malloc(sizeof(int32_t) * (size_t)T * k);
  float *w_ = w ? w : (float *)malloc(sizeof(float) * (size_t)T * k);
  float *ys_ = y_slots ? y_slots : (float *)malloc(sizeof(float) * (size_t)T * S * H);
  int rc = 0;
  if (!xq_ || !sx_ || !idx_ || !w_ || !ys_) { rc = -2; goto done; }
  if ((rc = orc_quantize_act(x, T, H, xq_, sx_)) != 0) goto done;
  if (top_p > 0.0 && !(sig = (double *)malloc(sizeof(double) * (size_t)T * E))) { rc = -2; goto done; }
  if (logits)
    rc = orc_router(1, logits, NULL, bias, T, H, E, k, routed_scale, idx_, w_, NULL, sig);
  else
    rc = orc_router(0, x, wr, bias, T, H, E, k, routed_scale, idx_, w_, NULL, sig);
  if (rc) goto done;
  if (top_p > 0.0 && (rc = orc_topp(T, E, k, sig, routed_scale, top_p, idx_, w_, NULL)) != 0) goto done;
  /* every (token, slot) pair is one expert applied to one token, independent
     of the others: with OpenMP they are spread over the threads (each pair
     still computed by one thread in the scalar order above) */
  {
    int prc = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(min : prc)
    for (int64_t p = 0; p < (int64_t)T * S; ++p) {
      const int64_t t = p / S;
      const int j = (int)(p - t * S);
      float *yp = ys_ + ((int64_t)t * S + j) * H;
      int r = 0;
      if (j < k) {
        const int e = idx_[t * k + j];
        if (e < 0) /* dropped by top-p: no expert, a zero slot */
          memset(yp, 0, sizeof(float) * (size_t)H);
        else
          r = orc_expert_token(bits[e], &experts[e], xq_ + t * H, sx_[t], H, I, NULL, NULL, NULL, NULL, NULL, NULL,
                               yp);
      } else {
        r = orc_expert_token(shared_bits, shared, xq_ + t * H, sx_[t], H, I, NULL, NULL, NULL, NULL, NULL, NULL, yp);
      }
      if (r < prc) prc = r;
    }
    if ((rc = prc) != 0) goto done;
  }
  rc = orc_combine(ys_, w_, T, k, H, shared ? 1 : 0, out);
done:
  free(sig);
  if (!xq) free(xq_);
  if (!sx) free(sx_);
  if (!idx) free(idx_);
  if (!w) free(w_);
  if (!y_slots) free(ys_);
  return rc;
}

/* Threads of the layer's (token, slot) loop (OpenMP builds; 1 otherwise). */
#ifdef _OPENMP
#include <omp.h>
#endif
int orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Unquantised fp64 SwiGLU (sanity figure only)                             */
/* ------------------------------------------------------------------------ */

int orc_swiglu_f64(const float *wg, const float *wu, const float *wd, const float *x, int H, int I, double *y) {
  double *a = (double *)malloc(sizeof(double) * (size_t)I);
  if (!a) return -2;
  for (int i = 0; i < I; ++i) {
    double g = 0.0, u = 0.0;
    for (int h = 0; h < H; ++h) {
      g += (double)wg[(int64_t)i * H + h] * (double)x[h];
      u += (double)wu[(int64_t)i * H + h] * (double)x[h];
    }
    a[i] = g / (1.0 + exp(-g)) * u;
  }
  for (int r = 0; r < H; ++r) {
    double s = 0.0;
    for (int i = 0; i < I; ++i) s += (double)wd[(int64_t)r * I + i] * a[i];
    y[r] = s;
  }
  free(a);
  return 0;
}
