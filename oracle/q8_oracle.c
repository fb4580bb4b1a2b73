/*
 * q8_oracle.c - CPU oracle for the Q8_0 decode matvec.  TEST INFRASTRUCTURE:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load it.  The product path (libq8dec) never calls it and shares no code,
 * header, table or helper with it.
 *
 * What it computes (inferno.rs "IV.4: One command buffer per token"):
 *   - "Eight kernels", the q8_matvec listing and its prose: a weight row is a
 *     run of n/32 Q8_0 blocks; block b holds a little-endian binary16 scale
 *     and 32 signed 8-bit quants covering x[32b .. 32b+31]; the output is
 *     y[r] = sum_b scale_b * sum_j q_bj * x[32b+j].
 *   - "The decoder: kernels and helpers", embed_row: dequantised weight is
 *     scale * q.
 *   - "Eight kernels", argmax_row and its prose: the largest value wins and
 *     equal values go to the lower index.
 * The oracle evaluates the plain definition, not any kernel's schedule: every
 * term scale*q*x is exact in binary64 (11 + 8 + 24 = 43 significant bits) and
 * the terms are summed in natural order (b, then j) in binary64.  The
 * per-output tolerance of the parity bar, 1e-4 * sum|scale*q*x| + 1e-6, is
 * returned beside each value.
 *
 * Readings where the pages are silent: binary16 subnormal scales are decoded
 * exactly; quant byte 0x80 is the int8 value -128; NaN logits never win the
 * argmax and an all-NaN row gives -1; -0 and +0 compare equal.
 *
 * The int8-activation variant (inferno.rs "IV.4", the prose after the
 * q8_matvec listing in "Eight kernels" and "The correctness ladder": the
 * CPU's sdot kernel quantises the activations and multiplies integers).  The
 * pages do not give the quantiser; the reading used here is the Q8_0 rule
 * applied to x, per block of 32, in binary32: amax = max |x_j|, d = amax/127,
 * q_j = x_j * (1/d) rounded to the nearest integer, ties to even (so
 * |q_j| <= 127); d = 0 gives q = 0; a block holding a NaN or an infinity gets
 * d = NaN and q = 0.  The product is then
 *   y[r] = sum_b scale_b * d_b * sum_j qw_bj * qx_bj
 * with the integer sums exact and the rest in binary64, natural order.
 *
 * Build: plain C11, no -ffast-math, floating contraction off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>

/* IEEE-754 binary16 -> binary64, from the format's definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 holds zero and the
 * subnormals f * 2^-24, exponent 31 holds the infinities and NaNs. */
double q8o_half_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1F;
  int frac = h & 0x3FF;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) 2^(e-15) */
  }
  return sign ? -v : v;
}

/* Rows [r0, r1) of y = W x for one activation row x (length n). */
static void matvec_rows(const uint8_t *w, const float *x, int64_t n,
                        int64_t r0, int64_t r1, double *y, double *tol) {
  const int64_t blocks = n / 32;
  for (int64_t r = r0; r < r1; r++) {
    const uint8_t *row = w + (size_t)r * (size_t)blocks * 34u;
    double sum = 0.0, mag = 0.0;
    for (int64_t b = 0; b < blocks; b++) {
      const uint8_t *blk = row + (size_t)b * 34u;
      double scale = q8o_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
      for (int j = 0; j < 32; j++) {
        double q = (double)(int8_t)blk[2 + j];
        double t = scale * q * (double)x[32 * b + j];
        sum += t;
        mag += fabs(t);
      }
    }
    y[r] = sum;
    if (tol) tol[r] = 1e-4 * mag + 1e-6;
  }
}

/* y[p] (and tol[p] if non-NULL) for w = p rows of n/32 blocks, x[n]. */
void q8o_matvec(const uint8_t *w, const float *x, int64_t n, int64_t p,
                double *y, double *tol) {
  matvec_rows(w, x, n, 0, p, y, tol);
}

/* Batched: x is [m][n] row-major, y and tol are [m][p] row-major. */
void q8o_matvec_batched(const uint8_t *w, const float *x, int64_t m, int64_t n,
                        int64_t p, double *y, double *tol) {
  for (int64_t i = 0; i < m; i++)
    matvec_rows(w, x + (size_t)i * (size_t)n, n, 0, p, y + (size_t)i * (size_t)p,
                tol ? tol + (size_t)i * (size_t)p : 0);
}

/* Same arithmetic per row, rows split over `threads` POSIX threads; results
 * are bit-identical to q8o_matvec because each row is computed alone. */
typedef struct {
  const uint8_t *w;
  const float *x;
  int64_t n, r0, r1;
  double *y, *tol;
} q8o_job;

static void *q8o_run(void *arg) {
  q8o_job *j = (q8o_job *)arg;
  matvec_rows(j->w, j->x, j->n, j->r0, j->r1, j->y, j->tol);
  return 0;
}

int q8o_matvec_mt(const uint8_t *w, const float *x, int64_t n, int64_t p,
                  double *y, double *tol, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  pthread_t th[256];
  q8o_job jobs[256];
  int made[256];
  for (int t = 0; t < threads; t++) {
    jobs[t].w = w;
    jobs[t].x = x;
    jobs[t].n = n;
    jobs[t].r0 = p * t / threads;
    jobs[t].r1 = p * (t + 1) / threads;
    jobs[t].y = y;
    jobs[t].tol = tol;
    made[t] = threads > 1 && pthread_create(&th[t], 0, q8o_run, &jobs[t]) == 0;
    if (!made[t]) q8o_run(&jobs[t]);
  }
  for (int t = 0; t < threads; t++)
    if (made[t]) pthread_join(th[t], 0);
  return threads;
}

/* Index of the largest value; equal values go to the lower index; NaN is
 * skipped; -1 when every value is NaN or p == 0. */
int64_t q8o_argmax_f64(const double *v, int64_t p) {
  int64_t best = -1;
  double bv = 0.0;
  for (int64_t i = 0; i < p; i++) {
    if (isnan(v[i])) continue;
    if (best < 0 || v[i] > bv) {
      best = i;
      bv = v[i];
    }
  }
  return best;
}

/* The same rule over binary32 values (for logits already held in f32). */
int64_t q8o_argmax_f32(const float *v, int64_t p) {
  int64_t best = -1;
  float bv = 0.0f;
  for (int64_t i = 0; i < p; i++) {
    if (isnan(v[i])) continue;
    if (best < 0 || v[i] > bv) {
      best = i;
      bv = v[i];
    }
  }
  return best;
}

/* ---- int8-activation variant ---------------------------------------------- */

/* Q8_0 quantisation of n activations (n % 32 == 0): d[n/32], q[n]. */
void q8o_quantize_x(const float *x, int64_t n, float *d, int8_t *q) {
  for (int64_t b = 0; b < n / 32; b++) {
    const float *xb = x + 32 * b;
    float amax = 0.0f;
    int bad = 0;
    for (int j = 0; j < 32; j++) {
      float a = fabsf(xb[j]);
      if (!isfinite(a)) bad = 1;
      else if (a > amax) amax = a;
    }
    if (bad) {
      d[b] = NAN;
      for (int j = 0; j < 32; j++) q[32 * b + j] = 0;
      continue;
    }
    float db = amax / 127.0f;
    float inv = db != 0.0f ? 1.0f / db : 0.0f;
    d[b] = db;
    for (int j = 0; j < 32; j++) q[32 * b + j] = (int8_t)rintf(xb[j] * inv);
  }
}

/* y[p] (and tol[p] if non-NULL) from quantised activations d[n/32], q[n]:
 * y = sum_b scale*d*isum, isum = sum_j qw*qx (exact integer); tol =
 * 1e-4 * sum_b |scale*d| * sum_j |qw*qx| + 1e-6. */
void q8o_matvec_i8x(const uint8_t *w, const float *d, const int8_t *q,
                    int64_t n, int64_t p, double *y, double *tol) {
  const int64_t blocks = n / 32;
  for (int64_t r = 0; r < p; r++) {
    const uint8_t *row = w + (size_t)r * (size_t)blocks * 34u;
    double acc = 0.0, size = 0.0;
    for (int64_t b = 0; b < blocks; b++) {
      const uint8_t *blk = row + (size_t)b * 34u;
      const double sd = q8o_half_to_double((uint16_t)(blk[0] | (blk[1] << 8))) * (double)d[b];
      int64_t isum = 0, iabs = 0;
      for (int j = 0; j < 32; j++) {
        const int64_t prod = (int64_t)(int8_t)blk[2 + j] * (int64_t)q[32 * b + j];
        isum += prod;
        iabs += prod < 0 ? -prod : prod;
      }
      acc += sd * (double)isum;
      size += fabs(sd) * (double)iabs;
    }
    y[r] = acc;
    if (tol) tol[r] = 1e-4 * size + 1e-6;
  }
}
