/*
 * q8_gen.c - seeded synthetic inputs for the Q8_0 decode-matvec workloads.
 *
 * This module only draws numbers.  It holds none of the matvec's arithmetic
 * (no scale decoding, no dot products, no reductions) and is shared by the
 * HIP path's tests/bench and by the CPU oracle's tests as a pure data source.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  The i-th output of a stream with key K is
 * mix(K + (i+1)*GAMMA), so every value is a function of (key, counter) and
 * any slice can be produced independently (counter-based, thread-parallel).
 *
 * Distributions (the Q8_0 workloads of the matvec pages, synthetic stand-ins
 * for the real Qwen3-0.6B weights which are not available):
 *   x       : N(0,1) by Box-Muller (cosine branch) in double, rounded to f32.
 *   quants  : uniform integers in [-127, 127]; each 32-bit half of one
 *             64-bit draw is mapped by multiply-shift (Lemire) to [0, 254].
 *   scale   : binary16 round-to-nearest-even of |N(0, 0.02)| / 127.
 * A Q8_0 block is 34 bytes: a little-endian binary16 scale, then 32 int8
 * quants (inferno.rs "IV.4: One command buffer per token", "Eight kernels").
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL
#define QBLK 32
#define QBYTES 34

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output (i >= 0) of the SplitMix64 stream whose seed is `key`. */
static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * GAMMA);
}

/* Stream key for one tensor: role 1 = weight blocks, 2 = activations x.
 * `index` names the matvec (0..196 in a decode step), `row` the row of x. */
uint64_t q8g_stream_key(uint64_t seed, uint32_t role, uint32_t index,
                        uint32_t row) {
  uint64_t tag = ((uint64_t)role << 56) ^ ((uint64_t)index << 28) ^ (uint64_t)row;
  return mix64(seed ^ mix64(tag + GAMMA));
}

uint64_t q8g_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* Standard normal from draws 2i and 2i+1 of the stream. */
static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t r1 = draw(key, 2 * i), r2 = draw(key, 2 * i + 1);
  double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;       /* [0, 1) */
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* Round a double to IEEE-754 binary16, nearest-even, subnormals kept. */
uint16_t q8g_f16_rne(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return 0x7E00u;
  double a = fabs(v);
  if (isinf(a)) return sign | 0x7C00u;
  if (a < 0x1.0p-14) {
    /* subnormal range: value = k * 2^-24, k = 0..1024 (1024 = min normal) */
    double k = rint(a * 0x1.0p24);
    return sign | (uint16_t)k;
  }
  int e;
  double f = frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
  double m = rint(ldexp(f, 11)); /* 11 significant bits: [1024, 2048] */
  if (m == 2048.0) { m = 1024.0; e += 1; }
  int biased = e - 1 + 15;
  if (biased >= 31) return sign | 0x7C00u;
  return sign | (uint16_t)(biased << 10) | (uint16_t)((int)m - 1024);
}

/* ---- block fill ------------------------------------------------------- */

/* Draws used by global block g: 2 (scale normal) + 16 (quants). */
#define DRAWS_PER_BLOCK 18

/* Blocks g0..g1-1 of the stream; `out` holds block g0. */
static void fill_blocks(uint64_t key, int64_t g0, int64_t g1, uint8_t *out) {
  for (int64_t g = g0; g < g1; g++) {
    uint8_t *blk = out + (size_t)(g - g0) * QBYTES;
    uint64_t base = (uint64_t)g * DRAWS_PER_BLOCK;
    double z = normal_at(key, base / 2); /* draws base, base+1 */
    uint16_t s = q8g_f16_rne(fabs(z) * 0.02 / 127.0);
    blk[0] = (uint8_t)(s & 0xFF);
    blk[1] = (uint8_t)(s >> 8);
    for (int t = 0; t < 16; t++) {
      uint64_t r = draw(key, base + 2 + t);
      uint32_t lo = (uint32_t)r, hi = (uint32_t)(r >> 32);
      int q0 = (int)(((uint64_t)lo * 255u) >> 32) - 127;
      int q1 = (int)(((uint64_t)hi * 255u) >> 32) - 127;
      blk[2 + 2 * t] = (uint8_t)(int8_t)q0;
      blk[3 + 2 * t] = (uint8_t)(int8_t)q1;
    }
  }
}

/* Normals i0..i1-1 of the stream; `out` holds normal i0. */
static void fill_normals(uint64_t key, int64_t i0, int64_t i1, float *out) {
  for (int64_t i = i0; i < i1; i++) out[i - i0] = (float)normal_at(key, (uint64_t)i);
}

typedef struct {
  int kind; /* 0 blocks, 1 normals */
  uint64_t key;
  int64_t a, b; /* element range [a, b) of the stream */
  void *out;    /* storage of element a */
} job_t;

static void *run_job(void *arg) {
  job_t *j = (job_t *)arg;
  if (j->kind == 0) fill_blocks(j->key, j->a, j->b, (uint8_t *)j->out);
  else fill_normals(j->key, j->a, j->b, (float *)j->out);
  return NULL;
}

static void parallel_fill(int kind, uint64_t key, int64_t first, int64_t count,
                          void *out, int nthreads) {
  size_t elem = kind == 0 ? QBYTES : sizeof(float);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (count < 4096) nthreads = 1;
  pthread_t th[64];
  job_t jobs[64];
  int created[64] = {0};
  for (int t = 0; t < nthreads; t++) {
    int64_t a = count * t / nthreads, b = count * (t + 1) / nthreads;
    jobs[t].kind = kind;
    jobs[t].key = key;
    jobs[t].a = first + a;
    jobs[t].b = first + b;
    jobs[t].out = (uint8_t *)out + (size_t)a * elem;
    if (nthreads > 1 && pthread_create(&th[t], NULL, run_job, &jobs[t]) == 0)
      created[t] = 1;
    else
      run_job(&jobs[t]);
  }
  for (int t = 0; t < nthreads; t++)
    if (created[t]) pthread_join(th[t], NULL);
}

/* Blocks first..first+nblocks-1 of the stream `key` (34 bytes each). */
void q8g_blocks(uint64_t key, int64_t first, int64_t nblocks, uint8_t *out,
                int nthreads) {
  parallel_fill(0, key, first, nblocks, out, nthreads);
}

/* Normals first..first+count-1 of the stream `key`, rounded to f32. */
void q8g_normals(uint64_t key, int64_t first, int64_t count, float *out,
                 int nthreads) {
  parallel_fill(1, key, first, count, out, nthreads);
}
