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
 * The rest of the decode step (inferno.rs "IV.4": "Eight kernels" for
 * rms_norm_row, rope_row, append_kv, attention_decode, add_inplace and
 * silu_hadamard; "One command buffer" for their order in a layer) is
 * evaluated in binary64 from the listings' definitions, except the RoPE
 * angle, which the listing types in binary32 and which is reproduced in
 * binary32 (q8o_rope_angle).
 *
 * Build: plain C11, no -ffast-math, floating contraction off.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

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

/* ---- the rest of the decode step ---------------------------------------------
 * inferno.rs "IV.4", "Eight kernels": rms_norm_row, rope_row, append_kv,
 * attention_decode, add_inplace and silu_hadamard; "One command buffer": the
 * order in which a layer runs them.  Activations are binary64 throughout;
 * the weights are the Q8_0 bytes and the binary32 norm weights, widened
 * exactly.  The one step the pages type in binary32 on purpose, the RoPE
 * angle, is reproduced in binary32 (q8o_rope_angle). */

/* q8_matvec with binary64 activations: y[r] = sum_b scale_b sum_j q_bj x_j,
 * natural order; mag[r] = sum of |scale*q*x| (if non-NULL). */
void q8o_matvec_f64(const uint8_t *w, const double *x, int64_t n, int64_t p,
                    double *y, double *mag) {
  const int64_t blocks = n / 32;
  for (int64_t r = 0; r < p; r++) {
    const uint8_t *row = w + (size_t)r * (size_t)blocks * 34u;
    double sum = 0.0, size = 0.0;
    for (int64_t b = 0; b < blocks; b++) {
      const uint8_t *blk = row + (size_t)b * 34u;
      double scale = q8o_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
      for (int j = 0; j < 32; j++) {
        double t = scale * (double)(int8_t)blk[2 + j] * x[32 * b + j];
        sum += t;
        size += fabs(t);
      }
    }
    y[r] = sum;
    if (mag) mag[r] = size;
  }
}

/* rms_norm_row: every row of dim values is divided by the root of (its mean
 * square + eps) and multiplied element-wise by the weight. */
void q8o_rms_norm(const double *x, const double *w, double *out, int64_t rows,
                  int64_t dim, double eps) {
  for (int64_t r = 0; r < rows; r++) {
    const double *xr = x + r * dim;
    double ss = 0.0;
    for (int64_t i = 0; i < dim; i++) ss += xr[i] * xr[i];
    const double inv = 1.0 / sqrt(ss / (double)dim + eps);
    for (int64_t i = 0; i < dim; i++) out[r * dim + i] = xr[i] * inv * w[i];
  }
}

/* rope_row's angle for pair i of a head (half = head_dim / 2) at position
 * pos.  The listing types it in binary32: the frequency is 1 over
 * theta^(i/half), the power correctly rounded (its precise:: functions) and
 * the quotient rounded to binary32, and the angle is pos times that
 * frequency, rounded to binary32. */
float q8o_rope_angle(int64_t pos, int64_t i, int64_t half, float theta) {
  const float e = (float)i / (float)half;
  const float pw = (float)pow((double)theta, (double)e);
  const float freq = 1.0f / pw;
  return (float)pos * freq;
}

/* rope_row: in each of `heads` heads, element i and element i + half turn
 * together by the angle of pair i: (a, b) -> (a cos - b sin, a sin + b cos). */
void q8o_rope(double *x, int64_t heads, int64_t head_dim, int64_t pos, float theta) {
  const int64_t half = head_dim / 2;
  for (int64_t h = 0; h < heads; h++) {
    double *xh = x + h * head_dim;
    for (int64_t i = 0; i < half; i++) {
      const double ang = (double)q8o_rope_angle(pos, i, half, theta);
      const double c = cos(ang), s = sin(ang);
      const double a = xh[i], b = xh[i + half];
      xh[i] = a * c - b * s;
      xh[i + half] = a * s + b * c;
    }
  }
}

/* attention_decode: query head h reads key/value head h / kv_group of the
 * seq cached rows (row t of head g starts at t * kv_width + g * head_dim);
 * score_t = q . k_t / sqrt(head_dim); weights = softmax of the scores with
 * their maximum subtracted; out = sum_t weight_t v_t.  probs, if non-NULL,
 * receives the weights, [n_heads][seq]. */
void q8o_attention(const double *q, const double *kc, const double *vc, double *out,
                   double *probs, int64_t seq, int64_t kv_width, int64_t head_dim,
                   int64_t kv_group, int64_t n_heads) {
  const double scale = 1.0 / sqrt((double)head_dim);
  for (int64_t h = 0; h < n_heads; h++) {
    const int64_t off = (h / kv_group) * head_dim;
    const double *qh = q + h * head_dim;
    double *sc = probs ? probs + h * seq : (double *)malloc(sizeof(double) * (size_t)(seq > 0 ? seq : 1));
    double mx = -INFINITY;
    for (int64_t t = 0; t < seq; t++) {
      const double *kr = kc + t * kv_width + off;
      double d = 0.0;
      for (int64_t j = 0; j < head_dim; j++) d += qh[j] * kr[j];
      sc[t] = d * scale;
      if (sc[t] > mx) mx = sc[t];
    }
    double sum = 0.0;
    for (int64_t t = 0; t < seq; t++) {
      sc[t] = exp(sc[t] - mx);
      sum += sc[t];
    }
    for (int64_t t = 0; t < seq; t++) sc[t] /= sum;
    for (int64_t j = 0; j < head_dim; j++) {
      double acc = 0.0;
      for (int64_t t = 0; t < seq; t++) acc += sc[t] * vc[t * kv_width + off + j];
      out[h * head_dim + j] = acc;
    }
    if (!probs) free(sc);
  }
}

/* silu_hadamard: out = gate / (1 + e^-gate) * up, element-wise. */
void q8o_silu_mul(const double *g, const double *u, double *out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
}

/* Shapes of a decoder layer. */
typedef struct {
  int64_t hidden, n_heads, n_kv_heads, head_dim, inter;
  double eps;
  float theta;
} q8o_dims;

/* One layer's weights: Q8_0 bytes of the seven projections ([out][in/32]
 * blocks) and the binary64 norm weights. */
typedef struct {
  const uint8_t *wq, *wk, *wv, *wo, *wg, *wu, *wd;
  const double *attn_norm, *q_norm, *k_norm, *ffn_norm;
} q8o_layer;

/* The layer's intermediate values, each sized for its role. */
typedef struct {
  double *xn, *q, *k, *v, *attn, *attn_out, *xn2, *gate, *up, *h, *ffn_out;
} q8o_acts;

/* One layer of the decode step at position pos, in the order the command
 * buffer encodes it: norm -> q, k, v -> QK-norm -> RoPE on q and k -> append
 * k, v as cache row pos -> attention over rows 0..pos -> o projection, added
 * into x -> norm -> gate, up -> SwiGLU -> down projection, added into x.
 * x [hidden] is updated in place; kc, vc are [>= pos + 1][kv_width]. */
void q8o_decode_layer(const q8o_dims *dm, const q8o_layer *L, double *x, double *kc,
                      double *vc, int64_t pos, const q8o_acts *a) {
  const int64_t H = dm->hidden, hd = dm->head_dim;
  const int64_t qw = dm->n_heads * hd, kvw = dm->n_kv_heads * hd;
  q8o_rms_norm(x, L->attn_norm, a->xn, 1, H, dm->eps);
  q8o_matvec_f64(L->wq, a->xn, H, qw, a->q, 0);
  q8o_matvec_f64(L->wk, a->xn, H, kvw, a->k, 0);
  q8o_matvec_f64(L->wv, a->xn, H, kvw, a->v, 0);
  q8o_rms_norm(a->q, L->q_norm, a->q, dm->n_heads, hd, dm->eps);
  q8o_rms_norm(a->k, L->k_norm, a->k, dm->n_kv_heads, hd, dm->eps);
  q8o_rope(a->q, dm->n_heads, hd, pos, dm->theta);
  q8o_rope(a->k, dm->n_kv_heads, hd, pos, dm->theta);
  for (int64_t i = 0; i < kvw; i++) {
    kc[pos * kvw + i] = a->k[i];
    vc[pos * kvw + i] = a->v[i];
  }
  q8o_attention(a->q, kc, vc, a->attn, 0, pos + 1, kvw, hd,
                dm->n_heads / dm->n_kv_heads, dm->n_heads);
  q8o_matvec_f64(L->wo, a->attn, qw, H, a->attn_out, 0);
  for (int64_t i = 0; i < H; i++) x[i] += a->attn_out[i];
  q8o_rms_norm(x, L->ffn_norm, a->xn2, 1, H, dm->eps);
  q8o_matvec_f64(L->wg, a->xn2, H, dm->inter, a->gate, 0);
  q8o_matvec_f64(L->wu, a->xn2, H, dm->inter, a->up, 0);
  q8o_silu_mul(a->gate, a->up, a->h, dm->inter);
  q8o_matvec_f64(L->wd, a->h, dm->inter, H, a->ffn_out, 0);
  for (int64_t i = 0; i < H; i++) x[i] += a->ffn_out[i];
}
