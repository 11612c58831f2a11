/*
 * moe_oracle.c — fp64 CPU oracle of the mixture-of-experts layer.
 * TEST INFRASTRUCTURE ONLY (see moe_oracle.h): never part of the product path.
 *
 * Each function writes out the plain definition its header comment cites;
 * loops run in the order of the definition's sums, nothing is blocked,
 * fused or reordered, and threads only split independent outputs.
 */
#include "moe_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Element decoding                                                    */
/* ------------------------------------------------------------------ */

static double dec_f32(const void* buf, int64_t i) {
  float f;
  memcpy(&f, (const char*)buf + 4 * i, 4);
  return (double)f;
}

static double dec_bf16(const void* buf, int64_t i) {
  uint16_t h;
  memcpy(&h, (const char*)buf + 2 * i, 2);
  uint32_t u = (uint32_t)h << 16; /* bfloat16 is the upper half of a binary32 */
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3 (fn variant): s eeee mmm, exponent bias 7.
 * e == 0: subnormal, value = m/8 * 2^-6. e == 15 && m == 7: NaN. Otherwise
 * (1 + m/8) * 2^(e-7). No infinities; the largest finite value is 448. */
static double dec_e4m3(const void* buf, int64_t i) {
  uint8_t b = ((const uint8_t*)buf)[i];
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -v : v;
}

static double dec_f64(const void* buf, int64_t i) { return ((const double*)buf)[i]; }

double orc_decode(const void* buf, int dt, int64_t i) {
  switch (dt) {
    case ORC_F32: return dec_f32(buf, i);
    case ORC_BF16: return dec_bf16(buf, i);
    case ORC_E4M3: return dec_e4m3(buf, i);
    case ORC_F64: return dec_f64(buf, i);
    default: return NAN;
  }
}

int orc_decode_array(const void* buf, int dt, int64_t n, double* out) {
  if (!buf || !out || n < 0 || dt < 0 || dt > 3) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = orc_decode(buf, dt, i);
  return 0;
}

/* Nearest bfloat16 (8 significant bits, binary32 exponent range) to v,
 * ties to even, computed directly from v (no intermediate binary32). */
double orc_round_bf16(double v) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  int ex;
  frexp(v, &ex);     /* v = f * 2^ex, 0.5 <= |f| < 1 */
  int lead = ex - 1; /* exponent of the leading bit */
  if (lead < -126) lead = -126; /* subnormal range: fixed quantum 2^-133 */
  double q = ldexp(1.0, lead - 7);
  double r = rint(v / q) * q; /* rint rounds half to even in the default mode */
  double maxv = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > maxv) r = copysign(INFINITY, v);
  return r;
}

uint16_t orc_bf16_bits(double v) {
  double r = orc_round_bf16(v);
  float f = (float)r; /* exact: r is representable */
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(v)) return 0x7fc0;
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* Threads over independent outputs                                    */
/* ------------------------------------------------------------------ */

typedef void (*orc_task_fn)(void* ctx, int64_t i);
typedef struct {
  orc_task_fn fn;
  void* ctx;
  int64_t n;
  int nthreads;
  int tid;
} orc_par_arg;

static void* orc_par_worker(void* p) {
  orc_par_arg* a = (orc_par_arg*)p;
  for (int64_t i = a->tid; i < a->n; i += a->nthreads) a->fn(a->ctx, i);
  return NULL;
}

static void orc_parallel_for(int64_t n, int nthreads, orc_task_fn fn, void* ctx) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; ++i) fn(ctx, i);
    return;
  }
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  orc_par_arg args[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    args[t].fn = fn;
    args[t].ctx = ctx;
    args[t].n = n;
    args[t].nthreads = nthreads;
    args[t].tid = t;
    if (pthread_create(&th[t], NULL, orc_par_worker, &args[t]) != 0) break;
    started++;
  }
  if (started < nthreads) { /* could not start them all: finish inline */
    for (int t = started; t < nthreads; ++t) orc_par_worker(&args[t]);
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------ */
/* O1-O3 router                                                        */
/* ------------------------------------------------------------------ */

typedef struct {
  double v;
  int e;
} orc_score;

/* Larger score first; equal scores: lower expert index first. */
static int orc_score_cmp(const void* pa, const void* pb) {
  const orc_score* a = (const orc_score*)pa;
  const orc_score* b = (const orc_score*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->e > b->e) - (a->e < b->e);
}

/* O1 for token t (scores into sc[E], bias added), then either O2 (full
 * sort) or, when `given` holds K expert indices, that selection as it
 * stands; O3 over the selected scores in slot order. gap: the K-th minus the
 * (K+1)-th largest score of the full sort, in both cases. */
static int route_one(const void* x, const void* wr, int dt, const float* bias, int t, int H, int E,
                     int K, const int32_t* given, int32_t* idx, double* gate, double* logits, double* gap) {
  orc_score* s = (orc_score*)malloc(sizeof(orc_score) * (size_t)E);
  double* sc = (double*)malloc(sizeof(double) * (size_t)E);
  if (!s || !sc) {
    free(s);
    free(sc);
    return -2;
  }
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int h = 0; h < H; ++h)
      acc += orc_decode(x, dt, (int64_t)t * H + h) * orc_decode(wr, dt, (int64_t)h * E + e);
    if (bias) acc += (double)bias[e];
    s[e].v = acc;
    s[e].e = e;
    sc[e] = acc;
    if (logits) logits[(int64_t)t * E + e] = acc;
  }
  qsort(s, (size_t)E, sizeof(orc_score), orc_score_cmp); /* brute-force full sort */
  int rc = 0;
  for (int k = 0; k < K; ++k) {
    idx[k] = given ? given[k] : s[k].e;
    if (idx[k] < 0 || idx[k] >= E) rc = -1;
  }
  if (rc == 0) {
    double denom = 0.0;
    for (int k = 0; k < K; ++k) denom += exp(sc[idx[k]] - sc[idx[0]]);
    for (int k = 0; k < K; ++k) gate[k] = exp(sc[idx[k]] - sc[idx[0]]) / denom;
  }
  if (gap) *gap = (K < E) ? (s[K - 1].v - s[K].v) : INFINITY;
  free(s);
  free(sc);
  return rc;
}

int orc_route(const void* x, const void* wr, int dt, const float* bias, int T, int H, int E, int K,
              int32_t* topk_idx, double* topk_gate, double* logits, double* gap) {
  return orc_route_given(x, wr, dt, bias, T, H, E, K, NULL, topk_idx, topk_gate, logits, gap);
}

int orc_route_given(const void* x, const void* wr, int dt, const float* bias, int T, int H, int E, int K,
                    const int32_t* given, int32_t* topk_idx, double* topk_gate, double* logits,
                    double* gap) {
  if (!x || !wr || !topk_idx || !topk_gate) return -1;
  if (T < 0 || H <= 0 || E <= 0 || K <= 0 || K > E) return -1;
  for (int t = 0; t < T; ++t) {
    int rc = route_one(x, wr, dt, bias, t, H, E, K, given ? given + (int64_t)t * K : NULL,
                       topk_idx + (int64_t)t * K, topk_gate + (int64_t)t * K, logits, gap ? gap + t : NULL);
    if (rc) return rc;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* O4-O6 dispatch                                                      */
/* ------------------------------------------------------------------ */

int orc_permute(const int32_t* topk_idx, int T, int E, int K, int32_t* counts, int32_t* offsets,
                int32_t* perm_src, int32_t* perm_dst) {
  if (!topk_idx || !counts || !offsets || !perm_src || !perm_dst) return -1;
  if (T < 0 || E <= 0 || K <= 0) return -1;
  int64_t A = (int64_t)T * K;
  for (int64_t i = 0; i < A; ++i)
    if (topk_idx[i] < 0 || topk_idx[i] >= E) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < A; ++i) counts[topk_idx[i]]++;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* fill = (int32_t*)calloc((size_t)E, sizeof(int32_t));
  if (!fill) return -2;
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      int64_t i = (int64_t)t * K + k;
      int e = topk_idx[i];
      int32_t row = offsets[e] + fill[e]++;
      perm_src[row] = (int32_t)i;
      perm_dst[i] = row;
    }
  free(fill);
  return 0;
}

int orc_gather_rows(const void* x, int64_t row_bytes, const int32_t* perm_src, int A, int K, void* xp) {
  if (!x || !perm_src || !xp || row_bytes <= 0 || A < 0 || K <= 0) return -1;
  for (int r = 0; r < A; ++r) {
    int64_t t = perm_src[r] / K;
    memcpy((char*)xp + (int64_t)r * row_bytes, (const char*)x + t * row_bytes, (size_t)row_bytes);
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* O7 grouped GEMM                                                     */
/* ------------------------------------------------------------------ */

typedef struct {
  const void* a;
  int a_dt;
  double a_scale;
  const double* a_row_scale; /* NULL: a_scale for every row */
  const void* w;
  int w_dt;
  double w_scale;
  const int32_t* offsets;
  int e, Hin, N, act;
  const int32_t* rows;
  double* out;
  int bad;
} orc_gmm_ctx;

static void orc_gmm_row(void* p, int64_t j) {
  orc_gmm_ctx* c = (orc_gmm_ctx*)p;
  int64_t r = c->rows ? c->rows[j] : j;
  int ex = -1;
  for (int q = 0; q < c->e; ++q)
    if (c->offsets[q] <= r && r < c->offsets[q + 1]) {
      ex = q;
      break;
    }
  double* o = c->out + j * (int64_t)c->N;
  if (ex < 0) {
    c->bad = 1;
    for (int n = 0; n < c->N; ++n) o[n] = NAN;
    return;
  }
  for (int n = 0; n < c->N; ++n) o[n] = 0.0;
  const int64_t wbase = (int64_t)ex * c->Hin * c->N;
  for (int h = 0; h < c->Hin; ++h) { /* o[n] = sum over h, in ascending h, for every n */
    double av = orc_decode(c->a, c->a_dt, r * c->Hin + h);
    for (int n = 0; n < c->N; ++n) o[n] += av * orc_decode(c->w, c->w_dt, wbase + (int64_t)h * c->N + n);
  }
  double sc = (c->a_row_scale ? c->a_row_scale[r] : c->a_scale) * c->w_scale;
  for (int n = 0; n < c->N; ++n) {
    double v = o[n] * sc;
    if (c->act == ORC_ACT_RELU && v < 0.0) v = 0.0;
    o[n] = v;
  }
}

int orc_gmm(const void* a, int a_dt, double a_scale, const void* w, int w_dt, double w_scale,
            const int32_t* offsets, int e, int Hin, int N, int act, const int32_t* rows, int nrows,
            double* out, int nthreads) {
  if (!a || !w || !offsets || !out || e <= 0 || Hin <= 0 || N <= 0) return -1;
  if (act != ORC_ACT_NONE && act != ORC_ACT_RELU) return -1;
  if (offsets[0] != 0) return -1;
  for (int q = 0; q < e; ++q)
    if (offsets[q + 1] < offsets[q]) return -1;
  int64_t n_out = rows ? nrows : offsets[e];
  if (n_out < 0) return -1;
  orc_gmm_ctx c = {a, a_dt, a_scale, NULL, w, w_dt, w_scale, offsets, e, Hin, N, act, rows, out, 0};
  orc_parallel_for(n_out, nthreads, orc_gmm_row, &c);
  return c.bad ? -1 : 0;
}

int orc_gmm_row_scaled(const void* a, int a_dt, const double* a_row_scale, const void* w, int w_dt,
                       double w_scale, const int32_t* offsets, int e, int Hin, int N, int act,
                       const int32_t* rows, int nrows, double* out, int nthreads) {
  if (!a_row_scale || !a || !w || !offsets || !out || e <= 0 || Hin <= 0 || N <= 0) return -1;
  if (act != ORC_ACT_NONE && act != ORC_ACT_RELU) return -1;
  if (offsets[0] != 0) return -1;
  for (int q = 0; q < e; ++q)
    if (offsets[q + 1] < offsets[q]) return -1;
  int64_t n_out = rows ? nrows : offsets[e];
  if (n_out < 0) return -1;
  orc_gmm_ctx c = {a, a_dt, 1.0, a_row_scale, w, w_dt, w_scale, offsets, e, Hin, N, act, rows, out, 0};
  orc_parallel_for(n_out, nthreads, orc_gmm_row, &c);
  return c.bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* Per-token E4M3 quantisation                                          */
/* ------------------------------------------------------------------ */

static double e4m3_value(int code) {
  const uint8_t b = (uint8_t)code;
  return dec_e4m3(&b, 0);
}

/* The finite E4M3 value nearest to num/den, decided without forming the
 * quotient: |num| is compared with v*den for the E4M3 values v and with
 * m*den for the midpoints m between neighbours. E4M3 values have at most 4
 * significant bits and midpoints 5, so with den a binary32 number (24 bits)
 * every such product is exact in binary64 and every comparison is exact.
 * Codes 0x00 .. 0x7e are the non-negative finite values in increasing order
 * (the exponent field sits above the mantissa field), so a bisection over
 * the codes brackets |num|. Ties go to the even code (mantissa bit 0 clear);
 * |num/den| at or above 448 gives +-448; NaN gives 0x7f. */
uint8_t orc_e4m3_nearest_ratio(double num, double den) {
  if (isnan(num) || !(den > 0.0)) return 0x7f;
  const uint8_t sign = signbit(num) ? 0x80 : 0x00;
  const double a = fabs(num);
  if (a >= 448.0 * den) return sign | 0x7e;
  int lo = 0, hi = 0x7e; /* value(lo) * den <= a < value(hi) * den */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (e4m3_value(mid) * den <= a)
      lo = mid;
    else
      hi = mid;
  }
  const double m = 0.5 * (e4m3_value(lo) + e4m3_value(hi)) * den;
  int one;
  if (a < m)
    one = lo;
  else if (a > m)
    one = hi;
  else
    one = (lo & 1) ? hi : lo; /* tie: the even code */
  return sign | (uint8_t)one;
}

uint8_t orc_e4m3_nearest(float v) { return orc_e4m3_nearest_ratio((double)v, 1.0); }

int orc_e4m3_nearest_array(const float* v, int64_t n, uint8_t* out) {
  if (!v || !out || n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_nearest(v[i]);
  return 0;
}

static uint32_t f32_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

/* amax / 448 rounded to the nearest binary32 number, ties to even. A first
 * guess from one binary64 division is moved to whichever neighbour is nearer,
 * judged by comparing amax with 448 times the midpoint between two adjacent
 * binary32 numbers (25 significant bits times 3: exact in binary64). */
float orc_div448_f32(double amax) {
  float s = (float)(amax / 448.0);
  for (int guard = 0; guard < 4; ++guard) {
    const float up = nextafterf(s, INFINITY), dn = nextafterf(s, 0.0f);
    const double mu = 0.5 * ((double)s + (double)up) * 448.0;
    const double md = 0.5 * ((double)s + (double)dn) * 448.0;
    const int odd = (int)(f32_bits(s) & 1u);
    if (amax > mu || (amax == mu && odd))
      s = up;
    else if (dn != s && (amax < md || (amax == md && odd)))
      s = dn;
    else
      break;
  }
  return s;
}

int orc_quant_rows(const void* x, int x_dt, int x_rows, int H, const int32_t* src, int div, int rows,
                   uint8_t* q, float* scale) {
  if (!x || !q || !scale || x_rows < 0 || H <= 0 || rows < 0 || div < 1) return -1;
  if (x_dt != ORC_F32 && x_dt != ORC_BF16 && x_dt != ORC_F64) return -1;
  for (int r = 0; r < rows; ++r) {
    int64_t t = r;
    if (src) t = src[r] >= 0 ? src[r] / div : -1;
    uint8_t* qr = q + (int64_t)r * H;
    if (t < 0 || t >= x_rows) {
      memset(qr, 0, (size_t)H);
      scale[r] = 0.0f;
      continue;
    }
    double amax = 0.0;
    for (int h = 0; h < H; ++h) {
      const double v = fabs(orc_decode(x, x_dt, t * H + h));
      if (v > amax) amax = v;
    }
    const float s = orc_div448_f32(amax);
    scale[r] = s;
    for (int h = 0; h < H; ++h)
      qr[h] = (s > 0.0f) ? orc_e4m3_nearest_ratio(orc_decode(x, x_dt, t * H + h), (double)s) : 0;
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* O7, MX form: block-scaled operands                                   */
/* ------------------------------------------------------------------ */

/* E8M0 scale byte: 2^(s - 127); 255 encodes NaN (OCP MX). */
double orc_e8m0(int s) {
  if (s < 0 || s > 255) return NAN;
  return s == 255 ? NAN : ldexp(1.0, s - 127);
}

typedef struct {
  const void* a;
  int a_dt;
  const uint8_t* a_scale;
  const void* w;
  int w_dt;
  const uint8_t* w_scale;
  const int32_t* offsets;
  int e, Hin, N, act;
  const int32_t* rows;
  double* out;
  int bad;
} orc_gmm_mx_ctx;

static void orc_gmm_mx_row(void* p, int64_t j) {
  orc_gmm_mx_ctx* c = (orc_gmm_mx_ctx*)p;
  int64_t r = c->rows ? c->rows[j] : j;
  int ex = -1;
  for (int q = 0; q < c->e; ++q)
    if (c->offsets[q] <= r && r < c->offsets[q + 1]) {
      ex = q;
      break;
    }
  double* o = c->out + j * (int64_t)c->N;
  double* blk = (double*)malloc(sizeof(double) * (size_t)c->N);
  if (ex < 0 || !blk) {
    c->bad = 1;
    for (int n = 0; n < c->N; ++n) o[n] = NAN;
    free(blk);
    return;
  }
  const int nb = c->Hin / 32;
  const int64_t wbase = (int64_t)ex * c->Hin * c->N;
  for (int n = 0; n < c->N; ++n) o[n] = 0.0;
  for (int b = 0; b < nb; ++b) {
    /* the block's plain dot products, ascending h, then its two scales */
    for (int n = 0; n < c->N; ++n) blk[n] = 0.0;
    for (int h = 32 * b; h < 32 * b + 32; ++h) {
      double av = orc_decode(c->a, c->a_dt, r * c->Hin + h);
      for (int n = 0; n < c->N; ++n) blk[n] += av * orc_decode(c->w, c->w_dt, wbase + (int64_t)h * c->N + n);
    }
    double sa = orc_e8m0(c->a_scale[r * nb + b]);
    const uint8_t* swr = c->w_scale + ((int64_t)ex * nb + b) * c->N;
    for (int n = 0; n < c->N; ++n) o[n] += sa * orc_e8m0(swr[n]) * blk[n];
  }
  free(blk);
  if (c->act == ORC_ACT_RELU)
    for (int n = 0; n < c->N; ++n)
      if (o[n] < 0.0) o[n] = 0.0;
}

int orc_gmm_mx(const void* a, int a_dt, const uint8_t* a_scale, const void* w, int w_dt,
               const uint8_t* w_scale, const int32_t* offsets, int e, int Hin, int N, int act,
               const int32_t* rows, int nrows, double* out, int nthreads) {
  if (!a || !w || !a_scale || !w_scale || !offsets || !out || e <= 0 || Hin <= 0 || N <= 0) return -1;
  if (Hin % 32 != 0) return -1;
  if (act != ORC_ACT_NONE && act != ORC_ACT_RELU) return -1;
  if (offsets[0] != 0) return -1;
  for (int q = 0; q < e; ++q)
    if (offsets[q + 1] < offsets[q]) return -1;
  int64_t n_out = rows ? nrows : offsets[e];
  if (n_out < 0) return -1;
  orc_gmm_mx_ctx c = {a, a_dt, a_scale, w, w_dt, w_scale, offsets, e, Hin, N, act, rows, out, 0};
  orc_parallel_for(n_out, nthreads, orc_gmm_mx_row, &c);
  return c.bad ? -1 : 0;
}

/* MX with E2M1 (OCP FP4) elements: 1 sign, 2 exponent bits (bias 1), 1
 * mantissa bit; exponent 0 is subnormal (m * 0.5); largest value 6. Two
 * elements per byte along the reduction index, the even index in the low
 * nibble: a (A, Hin/2) bytes; w (e, Hin/2, N) bytes, byte (ex, h/2, n)
 * holding rows h (low nibble, h even) and h+1 of column n. */
double orc_e2m1(int code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

static double dec_e2m1_at(const uint8_t* buf, int64_t byte, int hi) {
  return orc_e2m1(hi ? (buf[byte] >> 4) : (buf[byte] & 15));
}

typedef struct {
  const uint8_t *a, *a_scale, *w, *w_scale;
  const int32_t* offsets;
  int e, Hin, N, act;
  const int32_t* rows;
  double* out;
  int bad;
} orc_gmm_mx4_ctx;

static void orc_gmm_mx4_row(void* p, int64_t j) {
  orc_gmm_mx4_ctx* c = (orc_gmm_mx4_ctx*)p;
  int64_t r = c->rows ? c->rows[j] : j;
  int ex = -1;
  for (int q = 0; q < c->e; ++q)
    if (c->offsets[q] <= r && r < c->offsets[q + 1]) {
      ex = q;
      break;
    }
  double* o = c->out + j * (int64_t)c->N;
  double* blk = (double*)malloc(sizeof(double) * (size_t)c->N);
  if (ex < 0 || !blk) {
    c->bad = 1;
    for (int n = 0; n < c->N; ++n) o[n] = NAN;
    free(blk);
    return;
  }
  const int nb = c->Hin / 32, hb = c->Hin / 2;
  for (int n = 0; n < c->N; ++n) o[n] = 0.0;
  for (int b = 0; b < nb; ++b) {
    /* the block's plain dot products, ascending h, then its two scales */
    for (int n = 0; n < c->N; ++n) blk[n] = 0.0;
    for (int h = 32 * b; h < 32 * b + 32; ++h) {
      const double av = dec_e2m1_at(c->a, r * hb + h / 2, h & 1);
      const int64_t wrow = ((int64_t)ex * hb + h / 2) * c->N;
      for (int n = 0; n < c->N; ++n) blk[n] += av * dec_e2m1_at(c->w, wrow + n, h & 1);
    }
    const double sa = orc_e8m0(c->a_scale[r * nb + b]);
    const uint8_t* swr = c->w_scale + ((int64_t)ex * nb + b) * c->N;
    for (int n = 0; n < c->N; ++n) o[n] += sa * orc_e8m0(swr[n]) * blk[n];
  }
  free(blk);
  if (c->act == ORC_ACT_RELU)
    for (int n = 0; n < c->N; ++n)
      if (o[n] < 0.0) o[n] = 0.0;
}

int orc_gmm_mx4(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                const int32_t* offsets, int e, int Hin, int N, int act, const int32_t* rows, int nrows,
                double* out, int nthreads) {
  if (!a || !w || !a_scale || !w_scale || !offsets || !out || e <= 0 || Hin <= 0 || N <= 0) return -1;
  if (Hin % 32 != 0) return -1;
  if (act != ORC_ACT_NONE && act != ORC_ACT_RELU) return -1;
  if (offsets[0] != 0) return -1;
  for (int q = 0; q < e; ++q)
    if (offsets[q + 1] < offsets[q]) return -1;
  int64_t n_out = rows ? nrows : offsets[e];
  if (n_out < 0) return -1;
  orc_gmm_mx4_ctx c = {a, a_scale, w, w_scale, offsets, e, Hin, N, act, rows, out, 0};
  orc_parallel_for(n_out, nthreads, orc_gmm_mx4_row, &c);
  return c.bad ? -1 : 0;
}

/* ------------------------------------------------------------------ */
/* O8 combine / Unpermute                                              */
/* ------------------------------------------------------------------ */

int orc_combine(const double* yp, const int32_t* perm_dst, const double* gate, int T, int K, int N,
                double* out) {
  if (!yp || !perm_dst || !out || T < 0 || K <= 0 || N <= 0) return -1;
  for (int t = 0; t < T; ++t) {
    if (gate) {
      double* o = out + (int64_t)t * N;
      for (int n = 0; n < N; ++n) o[n] = 0.0;
      for (int k = 0; k < K; ++k) {
        int64_t i = (int64_t)t * K + k;
        const double* src = yp + (int64_t)perm_dst[i] * N;
        for (int n = 0; n < N; ++n) o[n] += gate[i] * src[n];
      }
    } else {
      for (int k = 0; k < K; ++k) {
        int64_t i = (int64_t)t * K + k;
        memcpy(out + i * N, yp + (int64_t)perm_dst[i] * N, sizeof(double) * (size_t)N);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Expert FFN on one token, and the whole layer                         */
/* ------------------------------------------------------------------ */

int orc_expert_ffn(const double* x, const void* w1, const void* w2, int dt, int ex, int H, int F,
                   int act, double* out) {
  if (!x || !w1 || !w2 || !out || H <= 0 || F <= 0 || ex < 0) return -1;
  double* hid = (double*)calloc((size_t)F, sizeof(double));
  if (!hid) return -2;
  const int64_t b1 = (int64_t)ex * H * F, b2 = (int64_t)ex * F * H;
  for (int h = 0; h < H; ++h)
    for (int f = 0; f < F; ++f) hid[f] += x[h] * orc_decode(w1, dt, b1 + (int64_t)h * F + f);
  if (act == ORC_ACT_RELU)
    for (int f = 0; f < F; ++f)
      if (hid[f] < 0.0) hid[f] = 0.0;
  for (int h = 0; h < H; ++h) out[h] = 0.0;
  for (int f = 0; f < F; ++f)
    for (int h = 0; h < H; ++h) out[h] += hid[f] * orc_decode(w2, dt, b2 + (int64_t)f * H + h);
  free(hid);
  return 0;
}

int orc_layer(const void* x, const void* wr, const float* bias, const void* w1, const void* w2, int dt,
              int T, int H, int E, int K, int F, int act, double* y, int32_t* topk_idx,
              double* topk_gate, double* gap, int32_t* counts_out, int nthreads) {
  if (!x || !wr || !w1 || !w2 || !y) return -1;
  if (T <= 0 || H <= 0 || E <= 0 || K <= 0 || K > E || F <= 0) return -1;
  if (dt != ORC_F32 && dt != ORC_BF16) return -1;
  const int64_t A = (int64_t)T * K;
  const int64_t es = (dt == ORC_F32) ? 4 : 2;
  int rc = -2;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * A);
  double* g = (double*)malloc(sizeof(double) * A);
  int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * E);
  int32_t* offsets = (int32_t*)malloc(sizeof(int32_t) * (E + 1));
  int32_t* psrc = (int32_t*)malloc(sizeof(int32_t) * A);
  int32_t* pdst = (int32_t*)malloc(sizeof(int32_t) * A);
  void* xp = malloc((size_t)(A * H * es));
  double* hm = (double*)malloc(sizeof(double) * A * F);
  double* yp = (double*)malloc(sizeof(double) * A * H);
  if (!idx || !g || !counts || !offsets || !psrc || !pdst || !xp || !hm || !yp) goto done;
  if ((rc = orc_route(x, wr, dt, bias, T, H, E, K, idx, g, NULL, gap))) goto done;
  if ((rc = orc_permute(idx, T, E, K, counts, offsets, psrc, pdst))) goto done;
  if ((rc = orc_gather_rows(x, (int64_t)H * es, psrc, (int)A, K, xp))) goto done;
  if ((rc = orc_gmm(xp, dt, 1.0, w1, dt, 1.0, offsets, E, H, F, act, NULL, 0, hm, nthreads))) goto done;
  if ((rc = orc_gmm(hm, ORC_F64, 1.0, w2, dt, 1.0, offsets, E, F, H, ORC_ACT_NONE, NULL, 0, yp, nthreads)))
    goto done;
  if ((rc = orc_combine(yp, pdst, g, T, K, H, y))) goto done;
  if (topk_idx) memcpy(topk_idx, idx, sizeof(int32_t) * A);
  if (topk_gate) memcpy(topk_gate, g, sizeof(double) * A);
  if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * E);
  rc = 0;
done:
  free(idx); free(g); free(counts); free(offsets); free(psrc); free(pdst);
  free(xp); free(hm); free(yp);
  return rc;
}

typedef struct {
  const void *x, *wr, *w1, *w2;
  const float* bias;
  int dt, T, H, E, K, F, act;
  const int32_t* tokens;
  const int32_t* given;
  double* y;
  int32_t* idx;
  double* gate;
  double* gap;
  int bad;
} orc_tok_ctx;

static void orc_token_task(void* p, int64_t j) {
  orc_tok_ctx* c = (orc_tok_ctx*)p;
  int t = c->tokens[j];
  int32_t* idx = c->idx + j * c->K;
  double* gate = c->gate + j * c->K;
  double* yo = c->y + j * (int64_t)c->H;
  double* xv = (double*)malloc(sizeof(double) * c->H);
  double* eo = (double*)malloc(sizeof(double) * c->H);
  if (!xv || !eo || t < 0 || t >= c->T) {
    c->bad = 1;
    free(xv); free(eo);
    return;
  }
  if (route_one(c->x, c->wr, c->dt, c->bias, t, c->H, c->E, c->K, c->given ? c->given + j * c->K : NULL,
                idx, gate, NULL, c->gap ? c->gap + j : NULL)) {
    c->bad = 1;
  }
  for (int h = 0; h < c->H; ++h) {
    xv[h] = orc_decode(c->x, c->dt, (int64_t)t * c->H + h);
    yo[h] = 0.0;
  }
  for (int k = 0; k < c->K; ++k) {
    if (orc_expert_ffn(xv, c->w1, c->w2, c->dt, idx[k], c->H, c->F, c->act, eo)) c->bad = 1;
    for (int h = 0; h < c->H; ++h) yo[h] += gate[k] * eo[h];
  }
  free(xv);
  free(eo);
}

int orc_layer_tokens(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                     int dt, int T, int H, int E, int K, int F, int act, const int32_t* tokens,
                     int ntok, double* y, int32_t* topk_idx, double* topk_gate, double* gap,
                     int nthreads) {
  return orc_layer_tokens_given(x, wr, bias, w1, w2, dt, T, H, E, K, F, act, tokens, ntok, NULL, y, topk_idx,
                                topk_gate, gap, nthreads);
}

int orc_layer_tokens_given(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                           int dt, int T, int H, int E, int K, int F, int act, const int32_t* tokens,
                           int ntok, const int32_t* given, double* y, int32_t* topk_idx, double* topk_gate,
                           double* gap, int nthreads) {
  if (!x || !wr || !w1 || !w2 || !tokens || !y || ntok < 0) return -1;
  if (T <= 0 || H <= 0 || E <= 0 || K <= 0 || K > E || F <= 0) return -1;
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)malloc(sizeof(int32_t) * (size_t)ntok * K + 1);
  double* g = topk_gate ? topk_gate : (double*)malloc(sizeof(double) * (size_t)ntok * K + 1);
  if (!idx || !g) return -2;
  orc_tok_ctx c = {x, wr, w1, w2, bias, dt, T, H, E, K, F, act, tokens, given, y, idx, g, gap, 0};
  orc_parallel_for(ntok, nthreads, orc_token_task, &c);
  if (!topk_idx) free(idx);
  if (!topk_gate) free(g);
  return c.bad ? -1 : 0;
}

int orc_layer_dense(const void* x, const void* wr, const float* bias, const void* w1, const void* w2,
                    int dt, int T, int H, int E, int K, int F, int act, double* y) {
  if (!x || !wr || !w1 || !w2 || !y) return -1;
  if (T <= 0 || H <= 0 || E <= 0 || K <= 0 || K > E || F <= 0) return -1;
  int rc = -2;
  int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * K);
  double* g = (double*)malloc(sizeof(double) * (size_t)T * K);
  double* m = (double*)calloc((size_t)T * E, sizeof(double)); /* binary activation mask */
  double* G = (double*)calloc((size_t)T * E, sizeof(double)); /* gates scattered to (T,E) */
  double* xv = (double*)malloc(sizeof(double) * H);
  double* eo = (double*)malloc(sizeof(double) * H);
  if (!idx || !g || !m || !G || !xv || !eo) goto done;
  if ((rc = orc_route(x, wr, dt, bias, T, H, E, K, idx, g, NULL, NULL))) goto done;
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      m[(int64_t)t * E + idx[t * K + k]] = 1.0;
      G[(int64_t)t * E + idx[t * K + k]] = g[t * K + k];
    }
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < H; ++h) {
      xv[h] = orc_decode(x, dt, (int64_t)t * H + h);
      y[(int64_t)t * H + h] = 0.0;
    }
    for (int e = 0; e < E; ++e) {
      if ((rc = orc_expert_ffn(xv, w1, w2, dt, e, H, F, act, eo))) goto done;
      double coef = m[(int64_t)t * E + e] * G[(int64_t)t * E + e];
      for (int h = 0; h < H; ++h) y[(int64_t)t * H + h] += coef * eo[h];
    }
  }
  rc = 0;
done:
  free(idx); free(g); free(m); free(G); free(xv); free(eo);
  return rc;
}
