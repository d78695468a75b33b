/*
 * nf4_oracle.c -- plain, slow, obviously correct CPU oracle for the NF4-style
 * 4-bit weight-only linear layer  y = x . dequant(W)^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * includes this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg load it.  It shares no code, header, table or constant with the
 * HIP path.
 *
 * Sources (vibevoice.c README, "Quantization > Weights"): a projection is
 * stored as 4-bit codes in blocks of 64 along the input dimension with one
 * absmax scale per block; the codes index a non-uniform table ("Int8
 * activations" section: "its codes index a non-uniform table").  The table
 * itself is not printed on the pages; the reading taken here is the one the
 * task statement fixes: normal quantiles normalised to [-1, 1] with an exact
 * zero (7 negative, 8 positive entries), each rounded to the nearest bfloat16.
 *
 * Built with  gcc -O2 -fno-fast-math -ffp-contract=off  and nothing that
 * flushes denormals.  All reductions run in natural k order in double.
 *
 * Functions that are not pinned by an independent check say so here:
 *   - none.  Every function below is pinned by a CPU test (exact rationals,
 *     closed forms, scipy/numpy library routines); the one unpinned claim is
 *     bit-compatibility of the table with third-party NF4 tables, which no
 *     function here asserts.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_BLOCK 64

/* ------------------------------------------------------------------------ */
/* Standard normal CDF and its inverse.                                     */
/* Phi(z) = erfc(-z / sqrt 2) / 2  (textbook identity).  The inverse is      */
/* plain bisection on that monotone function: no rational approximation, so */
/* there is no published constant table to get wrong.                        */
/* ------------------------------------------------------------------------ */
double oracle_norm_cdf(double z) { return 0.5 * erfc(-z / sqrt(2.0)); }

double oracle_norm_ppf(double p) {
  if (!(p > 0.0 && p < 1.0)) return NAN;
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 400; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid == lo || mid == hi) break; /* bracket is two adjacent doubles */
    if (oracle_norm_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

/* Round a double to the nearest bfloat16 value (8 significant bits), ties to
 * even, returned as a double.  Valid for normal-range magnitudes, which is all
 * the codebook needs. */
double oracle_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  double m = frexp(v, &e);       /* v = m * 2^e, 0.5 <= |m| < 1 */
  double r = nearbyint(ldexp(m, 8)); /* default rounding mode: ties to even */
  return ldexp(r, e - 8);
}

/* Codebook: 16 sorted values.  With tail probability delta,
 *   positives  q_j^+ =  Phi^-1(1/2 + (delta - 1/2) j/8) / Phi^-1(delta), j=1..8
 *   negatives  q_j^- = -Phi^-1(1/2 + (delta - 1/2) j/7) / Phi^-1(delta), j=1..7
 *   plus an exact 0.
 * Sorted ascending: q_7^-, ..., q_1^-, 0, q_1^+, ..., q_8^+.  The endpoints are
 * +-1 exactly because j/n == 1 exactly for j == n.  `unrounded` receives the
 * double values; `out` the bf16-rounded values as fp32. */
void oracle_nf4_codebook(double delta, float out[16], double unrounded[16]) {
  double d = oracle_norm_ppf(delta);
  double v[16];
  for (int j = 1; j <= 7; ++j) {
    double p = 0.5 + (delta - 0.5) * ((double)j / 7.0);
    v[7 - j] = -oracle_norm_ppf(p) / d;
  }
  v[7] = 0.0;
  for (int j = 1; j <= 8; ++j) {
    double p = 0.5 + (delta - 0.5) * ((double)j / 8.0);
    v[7 + j] = oracle_norm_ppf(p) / d;
  }
  for (int i = 0; i < 16; ++i) {
    if (unrounded) unrounded[i] = v[i];
    out[i] = (float)oracle_round_bf16(v[i]);
  }
}

/* ------------------------------------------------------------------------ */
/* Quantizer.  Per row n and 64-block b:                                     */
/*   s = max |w|  (exact);                                                   */
/*   s == 0  -> every code is the index z of the +0.0 entry;                 */
/*   else    idx = #{ i in 0..14 : (double)w > m_i * (double)s },            */
/*           m_i = ((double)c_i + (double)c_{i+1}) / 2.                       */
/* This is the nearest code to w/s with an exact midpoint going to the       */
/* lower index.  codes_out is one code per byte, [N][K].                     */
/* ------------------------------------------------------------------------ */
typedef struct {
  const float *W;
  int64_t N, K;
  const float *cb;
  uint8_t *codes;
  float *absmax;
  int zero_index;
  int64_t r0, r1;
} quant_job;

static void quantize_rows(const quant_job *j) {
  double mid[15];
  for (int i = 0; i < 15; ++i) mid[i] = ((double)j->cb[i] + (double)j->cb[i + 1]) / 2.0;
  const int64_t nb = j->K / ORACLE_BLOCK;
  for (int64_t n = j->r0; n < j->r1; ++n) {
    for (int64_t b = 0; b < nb; ++b) {
      const float *w = j->W + n * j->K + b * ORACLE_BLOCK;
      uint8_t *q = j->codes + n * j->K + b * ORACLE_BLOCK;
      float s = 0.0f;
      for (int k = 0; k < ORACLE_BLOCK; ++k) {
        float a = fabsf(w[k]);
        if (a > s) s = a;
      }
      j->absmax[n * nb + b] = s;
      for (int k = 0; k < ORACLE_BLOCK; ++k) {
        if (s == 0.0f) {
          q[k] = (uint8_t)j->zero_index;
          continue;
        }
        int count = 0;
        for (int i = 0; i < 15; ++i)
          if ((double)w[k] > mid[i] * (double)s) ++count;
        q[k] = (uint8_t)count;
      }
    }
  }
}

static void *quantize_thread(void *arg) {
  quantize_rows((const quant_job *)arg);
  return NULL;
}

/* Returns 0 on success, -1 on a bad shape or a codebook without +0.0. */
int oracle_quantize(const float *W, int64_t N, int64_t K, const float cb[16], uint8_t *codes,
                    float *absmax, int nthreads) {
  if (N < 1 || K < ORACLE_BLOCK || K % ORACLE_BLOCK) return -1;
  int z = -1;
  for (int i = 0; i < 16; ++i)
    if (cb[i] == 0.0f && !signbit(cb[i])) z = i;
  if (z < 0) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > N) nthreads = (int)N;
  pthread_t th[256];
  quant_job jobs[256];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (quant_job){W, N, K, cb, codes, absmax, z, N * t / nthreads, N * (t + 1) / nthreads};
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, quantize_thread, &jobs[t]);
  quantize_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Canonical packed format: byte[n][j] = code[n][2j] | code[n][2j+1] << 4    */
/* (low nibble holds the even k).                                            */
/* ------------------------------------------------------------------------ */
void oracle_pack_canonical(const uint8_t *codes, int64_t N, int64_t K, uint8_t *packed) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K / 2; ++j) {
      uint8_t lo = codes[n * K + 2 * j] & 0xF;
      uint8_t hi = codes[n * K + 2 * j + 1] & 0xF;
      packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
    }
}

void oracle_unpack_canonical(const uint8_t *packed, int64_t N, int64_t K, uint8_t *codes) {
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K / 2; ++j) {
      uint8_t byte = packed[n * (K / 2) + j];
      codes[n * K + 2 * j] = byte & 0xF;
      codes[n * K + 2 * j + 1] = byte >> 4;
    }
}

/* Code of element (n, k) from the canonical packed bytes. */
static inline int code_at(const uint8_t *packed, int64_t K, int64_t n, int64_t k) {
  uint8_t byte = packed[n * (K / 2) + k / 2];
  return (k & 1) ? (byte >> 4) : (byte & 0xF);
}

/* ------------------------------------------------------------------------ */
/* Dequant: W'[n,k] = fl32(c[idx] * s), one binary32 multiply.               */
/* ------------------------------------------------------------------------ */
static void dequant_row(const uint8_t *packed, const float *absmax, const float cb[16], int64_t K,
                        int64_t n, float *out_row) {
  const int64_t nb = K / ORACLE_BLOCK;
  for (int64_t k = 0; k < K; ++k) {
    float c = cb[code_at(packed, K, n, k)];
    float s = absmax[n * nb + k / ORACLE_BLOCK];
    float w = c * s;
    out_row[k] = w;
  }
}

void oracle_dequant(const uint8_t *packed, const float *absmax, const float cb[16], int64_t N,
                    int64_t K, float *W_out) {
  for (int64_t n = 0; n < N; ++n) dequant_row(packed, absmax, cb, K, n, W_out + n * K);
}

/* bfloat16 bit pattern -> value (exact widening). */
static inline double bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Linear: y[m,n] = sum_k (double)x[m,k] * (double)W'[n,k] in natural k      */
/* order, and bound[m,n] = sum_k |x[m,k] * W'[n,k]|.  Each product of a      */
/* bf16 and a binary32 value is exact in double.  Only the output rows n     */
/* listed in `rows` (nrows of them) are computed; outputs are [M][nrows].    */
/* rows == NULL means all N rows in order.                                   */
/* ------------------------------------------------------------------------ */
typedef struct {
  const uint16_t *x;
  int64_t M;
  const uint8_t *packed;
  const float *absmax;
  const float *cb;
  int64_t N, K;
  const int64_t *rows;
  int64_t nrows;
  double *y, *bound;
  int64_t r0, r1;
} linear_job;

static void linear_part(const linear_job *j) {
  float *w = (float *)malloc(sizeof(float) * (size_t)j->K);
  if (!w) return;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t n = j->rows ? j->rows[r] : r;
    dequant_row(j->packed, j->absmax, j->cb, j->K, n, w);
    for (int64_t m = 0; m < j->M; ++m) {
      const uint16_t *xr = j->x + m * j->K;
      double acc = 0.0, b = 0.0;
      for (int64_t k = 0; k < j->K; ++k) {
        double p = bf16_to_double(xr[k]) * (double)w[k];
        acc += p;
        b += fabs(p);
      }
      j->y[m * j->nrows + r] = acc;
      if (j->bound) j->bound[m * j->nrows + r] = b;
    }
  }
  free(w);
}

static void *linear_thread(void *arg) {
  linear_part((const linear_job *)arg);
  return NULL;
}

int oracle_linear(const uint16_t *x, int64_t M, const uint8_t *packed, const float *absmax,
                  const float cb[16], int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
                  double *y, double *bound, int nthreads) {
  if (M < 1 || N < 1 || K < ORACLE_BLOCK || K % ORACLE_BLOCK) return -1;
  if (!rows) nrows = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = (int)nrows;
  pthread_t th[256];
  linear_job jobs[256];
  for (int t = 0; t < nthreads; ++t)
    jobs[t] = (linear_job){x,    M,     packed, absmax, cb, N, K, rows, nrows,
                           y,    bound, nrows * t / nthreads, nrows * (t + 1) / nthreads};
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, linear_thread, &jobs[t]);
  linear_part(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* ======================================================================== */
/* Second format: asymmetric int4 in groups of 128 along K (vibevoice.c     */
/* README, "Quantization" > "Weights", the AWQ/GPTQ paragraph): a weight is */
/* (q - z) * s with a 4-bit integer q, an exact integer zero point z per    */
/* group and an FP16 scale s per group.                                     */
/* ======================================================================== */
#define ORACLE_GROUP 128

/* Nearest binary16 value of a double, ties to even; the result as a double.
 * Written from the IEEE 754 binary16 format: 11 significant bits for
 * normal values (exponent -14..15), a fixed quantum of 2^-24 below 2^-14,
 * and overflow past the largest finite value 65504 to infinity. */
double oracle_round_fp16(double v) {
  if (v != v || v == 0.0) return v;
  const double a = fabs(v);
  if (a >= 65520.0) return v > 0 ? INFINITY : -INFINITY;  /* halfway to 2^16 and above */
  int e;
  frexp(a, &e);                      /* a = f * 2^e with f in [0.5, 1) */
  int q_exp = e - 11;                /* quantum of an 11-bit significand */
  if (q_exp < -24) q_exp = -24;      /* subnormal range: fixed quantum */
  const double quantum = ldexp(1.0, q_exp);
  const double r = nearbyint(a / quantum) * quantum;  /* a / quantum is exact */
  return v > 0 ? r : -r;
}

/* Per row and group of 128: wmin, wmax; s = fp16(max(wmax - wmin, 1e-5) / 15);
 * z = clamp(rint(-wmin / s), 0, 15); q = clamp(rint(w / s) + z, 0, 15), all
 * in double with round-half-even (the rounding mode in force).  codes: one
 * per byte [N][K]; scales fp32 [N][K/128] (each fp16-exact); zeros uint8
 * [N][K/128].  Returns -1 on a bad shape. */
typedef struct {
  const float *W;
  int64_t N, K;
  uint8_t *codes;
  float *scales;
  uint8_t *zeros;
  int64_t r0, r1;
} awq_job;

static void awq_rows(const awq_job *j) {
  const int64_t ng = j->K / ORACLE_GROUP;
  for (int64_t n = j->r0; n < j->r1; ++n)
    for (int64_t g = 0; g < ng; ++g) {
      const float *w = j->W + n * j->K + g * ORACLE_GROUP;
      uint8_t *q = j->codes + n * j->K + g * ORACLE_GROUP;
      float lo = w[0], hi = w[0];
      for (int k = 1; k < ORACLE_GROUP; ++k) {
        if (w[k] < lo) lo = w[k];
        if (w[k] > hi) hi = w[k];
      }
      double range = (double)hi - (double)lo;
      if (range < 1e-5) range = 1e-5;
      const double s = oracle_round_fp16(range / 15.0);
      double z = nearbyint(-(double)lo / s);
      if (z < 0) z = 0;
      if (z > 15) z = 15;
      j->scales[n * ng + g] = (float)s;
      j->zeros[n * ng + g] = (uint8_t)z;
      for (int k = 0; k < ORACLE_GROUP; ++k) {
        double v = nearbyint((double)w[k] / s) + z;
        if (v < 0) v = 0;
        if (v > 15) v = 15;
        q[k] = (uint8_t)v;
      }
    }
}

static void *awq_thread(void *arg) {
  awq_rows((const awq_job *)arg);
  return NULL;
}

int oracle_awq_quantize(const float *W, int64_t N, int64_t K, uint8_t *codes, float *scales,
                        uint8_t *zeros, int nthreads) {
  if (N < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > N) nthreads = (int)N;
  pthread_t th[256];
  awq_job jobs[256];
  for (int t = 0; t < nthreads; ++t)
    jobs[t] = (awq_job){W, N, K, codes, scales, zeros, N * t / nthreads, N * (t + 1) / nthreads};
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, awq_thread, &jobs[t]);
  awq_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* W'[n,k] = fl32((q - z) * s): the integer q - z (exact in binary32) times s,
 * one binary32 multiply.  packed: canonical bytes [N][K/2]. */
static void awq_dequant_row(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                            int64_t K, int64_t n, float *out_row) {
  const int64_t ng = K / ORACLE_GROUP;
  for (int64_t k = 0; k < K; ++k) {
    const int q = code_at(packed, K, n, k);
    const int z = zeros[n * ng + k / ORACLE_GROUP];
    const float d = (float)(q - z);
    const float s = scales[n * ng + k / ORACLE_GROUP];
    out_row[k] = d * s;
  }
}

void oracle_awq_dequant(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                        int64_t N, int64_t K, float *W_out) {
  for (int64_t n = 0; n < N; ++n) awq_dequant_row(packed, scales, zeros, K, n, W_out + n * K);
}

/* y[m,n] = sum_k x[m,k] * W'[n,k] in double, natural k order, and
 * bound[m,n] = sum_k |x[m,k] * W'[n,k]|, as oracle_linear. */
typedef struct {
  const uint16_t *x;
  int64_t M;
  const uint8_t *packed;
  const float *scales;
  const uint8_t *zeros;
  int64_t N, K;
  const int64_t *rows;
  int64_t nrows;
  double *y, *bound;
  int64_t r0, r1;
} awq_linear_job;

static void awq_linear_part(const awq_linear_job *j) {
  float *w = (float *)malloc(sizeof(float) * (size_t)j->K);
  if (!w) return;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t n = j->rows ? j->rows[r] : r;
    awq_dequant_row(j->packed, j->scales, j->zeros, j->K, n, w);
    for (int64_t m = 0; m < j->M; ++m) {
      const uint16_t *xr = j->x + m * j->K;
      double acc = 0.0, b = 0.0;
      for (int64_t k = 0; k < j->K; ++k) {
        double p = bf16_to_double(xr[k]) * (double)w[k];
        acc += p;
        b += fabs(p);
      }
      j->y[m * j->nrows + r] = acc;
      if (j->bound) j->bound[m * j->nrows + r] = b;
    }
  }
  free(w);
}

static void *awq_linear_thread(void *arg) {
  awq_linear_part((const awq_linear_job *)arg);
  return NULL;
}

int oracle_awq_linear(const uint16_t *x, int64_t M, const uint8_t *packed, const float *scales,
                      const uint8_t *zeros, int64_t N, int64_t K, const int64_t *rows,
                      int64_t nrows, double *y, double *bound, int nthreads) {
  if (M < 1 || N < 1 || K < ORACLE_GROUP || K % ORACLE_GROUP) return -1;
  if (!rows) nrows = N;
  for (int64_t r = 0; rows && r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= N) return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > nrows) nthreads = (int)nrows;
  pthread_t th[256];
  awq_linear_job jobs[256];
  for (int t = 0; t < nthreads; ++t)
    jobs[t] = (awq_linear_job){x, M, packed, scales, zeros, N, K, rows, nrows,
                               y, bound, nrows * t / nthreads, nrows * (t + 1) / nthreads};
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, awq_linear_thread, &jobs[t]);
  awq_linear_part(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}
