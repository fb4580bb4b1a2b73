// The decode step's attention and norms on gfx950 (inferno.rs "IV.4",
// "Eight kernels": rms_norm_row, rope_row, append_kv, attention_decode).
//
// attention_decode is split over the cache the way MI355X wants it: the
// pages run one 128-thread group per query head over every cached row, which
// keeps 16 of 256 compute units busy; here a workgroup takes 64 cached rows
// of one key/value head for all the query heads that share it (GQA), writes
// a partial softmax (its maximum, its sum and its weighted value sum), and
// the last workgroup of that head to finish merges the partials.  The QK-norm
// and the RoPE of q and k are folded into each workgroup's prologue (a head
// is 128 values, cheaper to recompute than to hand over through another
// launch), and the workgroup that holds row pos writes this token's key and
// value into the cache (append_kv); rows below pos come from the cache, row
// pos from registers, so no workgroup reads a row another one writes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q8dec_decode_dev.h"
#include "q8dec_internal.h"

namespace q8 {
namespace {

constexpr int HD = kAttnHeadDim;
constexpr int CH = kAttnChunk;
static_assert(HD == 128 && CH == 64, "the lane mappings below assume these");

// Sum over the 16 lanes of each 16-lane row.
__device__ __forceinline__ float row16_sum(float v) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) v += __shfl_xor(v, m, 16);
  return v;
}

__device__ __forceinline__ void load8(const float *p, float (&d)[8]) {
  const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
  d[0] = a.x; d[1] = a.y; d[2] = a.z; d[3] = a.w;
  d[4] = b.x; d[5] = b.y; d[6] = b.z; d[7] = b.w;
}

// Merge of key/value head g's nc chunk partials by one workgroup: out =
// sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c, M the maximum of the m_c.
// Chunks go in rounds of R, each issuing all of its loads at once: thread
// (h, i) loads chunk c0 + i's maximum and sum of head h, and every (h, d)
// thread its R sums of dimension d.  Wave h then takes the round's maximum,
// the running maximum M, the factor that rescales the earlier rounds and
// the chunk weights e^(m_c - M) into LDS; each (h, d) thread rescales its
// running sum and adds the weighted chunk sums in chunk order.  lds: 3 G R +
// 4 G floats, not in use.
template <int G, int R>
__device__ __forceinline__ void merge_partials(const AttnArgs &a, int g, int nc, float *lds) {
  constexpr int IT = (G * HD + dec::kThreads - 1) / dec::kThreads;  // (h, d) items per thread
  static_assert(G <= 4 && R <= 64, "one wave per head, one lane per chunk");
  const int tid = (int)threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float *mw = lds;         // [G][R]: the round's chunk maxima, then weights
  float *ls = mw + G * R;  // [G][R]: the round's chunk sums
  float *hs = ls + G * R;  // [G][4]: running maximum, running sum, rescale
  if (tid < G) {
    hs[4 * tid] = -INFINITY;
    hs[4 * tid + 1] = 0.f;
  }
  float A[IT];
#pragma unroll
  for (int e = 0; e < IT; e++) A[e] = 0.f;
  const float *ph = a.part + (size_t)(g * G) * a.chunks * kAttnPart;
  for (int c0 = 0; c0 < nc; c0 += R) {
    const int k = nc - c0 < R ? nc - c0 : R;
    float pm = -INFINITY, pl = 0.f;
    if (tid < G * R && tid % R < k) {
      const float *p = ph + ((size_t)(tid / R) * a.chunks + c0 + tid % R) * kAttnPart;
      pm = dec::ld_dev(p);
      pl = dec::ld_dev(p + 1);
    }
    float pa[IT][R];
#pragma unroll
    for (int e = 0; e < IT; e++) {
      const int it = tid + e * dec::kThreads, h = it / HD, d = it % HD;
#pragma unroll
      for (int i = 0; i < R; i++) {
        pa[e][i] = 0.f;
        if (it < G * HD && i < k)
          pa[e][i] = dec::ld_dev(ph + ((size_t)h * a.chunks + c0 + i) * kAttnPart + 4 + d);
      }
    }
    if (tid < G * R) {
      mw[tid] = pm;
      ls[tid] = pl;
    }
    __syncthreads();
    if (wave < G) {
      const float m = lane < R ? mw[wave * R + lane] : -INFINITY;
      const float l = lane < R ? ls[wave * R + lane] : 0.f;
      const float mo = hs[4 * wave], mn = fmaxf(mo, dec::wave_maxf(m));
      const float r = mo == mn ? 1.f : expf(mo - mn);
      const float w = lane < k ? expf(m - mn) : 0.f;
      const float sl = dec::wave_sum(w * l);
      if (lane < R) mw[wave * R + lane] = w;
      if (lane == 0) {
        hs[4 * wave] = mn;
        hs[4 * wave + 1] = hs[4 * wave + 1] * r + sl;
        hs[4 * wave + 2] = r;
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < IT; e++) {
      const int it = tid + e * dec::kThreads, h = it < G * HD ? it / HD : 0;
      float v = A[e] * hs[4 * h + 2];
#pragma unroll
      for (int i = 0; i < R; i++) v += mw[h * R + i] * pa[e][i];
      A[e] = v;
    }
    __syncthreads();  // before the next round rewrites mw, ls and hs
  }
#pragma unroll
  for (int e = 0; e < IT; e++) {
    const int it = tid + e * dec::kThreads;
    if (it < G * HD) a.out[(size_t)(g * G) * HD + it] = A[e] / hs[4 * (it / HD) + 1];
  }
}

// G query heads per key/value head.  Every load the workgroup needs (its
// vectors, the norm weights, the rotation table and its 64 cached key and
// value rows) is issued as soon as pos is known, so the whole prologue costs
// one memory round trip.
template <int G>
__global__ void __launch_bounds__(dec::kThreads) attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) float qs[G][HD];  // normed, rotated queries
  __shared__ __attribute__((aligned(16))) float kn[HD];     // this token's key, normed, rotated
  __shared__ __attribute__((aligned(16))) float vn[HD];     // this token's value
  __shared__ float sc[G][CH];                               // scores, then weights
  __shared__ float ml[G][2];                                // chunk maximum and sum
  __shared__ __attribute__((aligned(16))) float red[4][G][HD];
  __shared__ uint32_t flag;
  const int g = (int)blockIdx.x / a.chunks, c = (int)blockIdx.x % a.chunks;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int pos = *a.pos;
  if (pos < 0 || pos >= a.cache_rows) {  // no such row: the heads read NaN
    if (c == 0)
      for (int t = (int)threadIdx.x; t < G * HD; t += dec::kThreads)
        a.out[(size_t)(g * G) * HD + t] = __builtin_nanf("");
    return;
  }
  const int seq = pos + 1;
  const int nc = (seq + CH - 1) / CH;
  if (c >= nc) return;  // beyond the cached rows: no arrival either
  const int t0 = c * CH;
  const int len = seq - t0 < CH ? seq - t0 : CH;
  const bool owner = pos < t0 + CH;  // this chunk holds row pos
  const size_t kvw = (size_t)a.n_kv * HD;

  // Vectors: wave w takes vectors w and w + 4 of the G queries, the key (G)
  // and the value (G + 1); lane l holds elements l and l + 64 (RoPE pair l).
  constexpr int NV = (G + 2 + 3) / 4;
  float x0[NV], x1[NV];
#pragma unroll
  for (int j = 0; j < NV; j++) {
    const int vec = wave + 4 * j;
    x0[j] = x1[j] = 0.f;
    if (vec < G + 2) {
      const float *src = vec < G ? a.q + (size_t)(g * G + vec) * HD
                                 : (vec == G ? a.k : a.v) + (size_t)g * HD;
      x0[j] = src[lane];
      x1[j] = src[lane + 64];
    }
  }
  const float wq0 = a.q_norm[lane], wq1 = a.q_norm[lane + 64];
  const float wk0 = a.k_norm[lane], wk1 = a.k_norm[lane + 64];
  const float cs = a.rope[2 * lane], sn = a.rope[2 * lane + 1];
  // cached rows below pos: 16 lanes per row (8 dimensions each), 4 passes
  const int slot = (int)threadIdx.x >> 4, sub = (int)threadIdx.x & 15;
  float kr[4][8], vr[4][8];
#pragma unroll
  for (int ps = 0; ps < 4; ps++) {
    const int tl = slot + 16 * ps, t = t0 + tl;
#pragma unroll
    for (int i = 0; i < 8; i++) kr[ps][i] = vr[ps][i] = 0.f;
    if (tl < len && t != pos) {
      const size_t off = (size_t)t * kvw + (size_t)g * HD + 8 * sub;
      load8(a.kc + off, kr[ps]);
      load8(a.vc + off, vr[ps]);
    }
  }

  // QK-norm and RoPE of the queries and the key; the value as it is.  The
  // chunk holding row pos appends this token's key and value to the cache.
#pragma unroll
  for (int j = 0; j < NV; j++) {
    const int vec = wave + 4 * j;
    if (vec <= G) {
      const float w0 = vec < G ? wq0 : wk0, w1 = vec < G ? wq1 : wk1;
      const float ss = dec::wave_sum(x0[j] * x0[j] + x1[j] * x1[j]);
      const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
      const float u0 = x0[j] * inv * w0, u1 = x1[j] * inv * w1;
      const float r0 = u0 * cs - u1 * sn, r1 = u0 * sn + u1 * cs;
      float *dst = vec < G ? qs[vec] : kn;
      dst[lane] = r0;
      dst[lane + 64] = r1;
      if (vec == G && owner) {
        float *row = a.kc + (size_t)pos * kvw + (size_t)g * HD;
        row[lane] = r0;
        row[lane + 64] = r1;
      }
    } else if (vec == G + 1) {
      vn[lane] = x0[j];
      vn[lane + 64] = x1[j];
      if (owner) {
        float *row = a.vc + (size_t)pos * kvw + (size_t)g * HD;
        row[lane] = x0[j];
        row[lane + 64] = x1[j];
      }
    }
  }
  __syncthreads();
  if (owner) {  // row pos comes from LDS
#pragma unroll
    for (int ps = 0; ps < 4; ps++) {
      const int tl = slot + 16 * ps;
      if (tl < len && t0 + tl == pos) {
        load8(kn + 8 * sub, kr[ps]);
        load8(vn + 8 * sub, vr[ps]);
      }
    }
  }

  // Scores q . k_t / sqrt(128).
  const float scale = 1.0f / sqrtf((float)HD);
#pragma unroll
  for (int h = 0; h < G; h++) {
    float qr[8];
    load8(qs[h] + 8 * sub, qr);
#pragma unroll
    for (int ps = 0; ps < 4; ps++) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) d += qr[i] * kr[ps][i];
      d = row16_sum(d);
      const int tl = slot + 16 * ps;
      if (sub == 0 && tl < len) sc[h][tl] = d * scale;
    }
  }
  __syncthreads();

  // Softmax of the chunk, one wave per query head.
  for (int h = wave; h < G; h += 4) {
    const float s = lane < len ? sc[h][lane] : -INFINITY;
    const float m = dec::wave_maxf(s);
    const float e = lane < len ? expf(s - m) : 0.f;
    const float l = dec::wave_sum(e);
    sc[h][lane] = e;
    if (lane == 0) {
      ml[h][0] = m;
      ml[h][1] = l;
    }
  }
  __syncthreads();

  // Weighted value rows.
#pragma unroll
  for (int h = 0; h < G; h++) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = 0.f;
#pragma unroll
    for (int ps = 0; ps < 4; ps++) {
      const int tl = slot + 16 * ps;
      const float e = tl < len ? sc[h][tl] : 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += e * vr[ps][i];
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      acc[i] += __shfl_xor(acc[i], 16, 64);
      acc[i] += __shfl_xor(acc[i], 32, 64);
    }
    if (lane < 16) {
#pragma unroll
      for (int i = 0; i < 8; i++) red[wave][h][8 * sub + i] = acc[i];
    }
  }
  __syncthreads();
  for (int t = (int)threadIdx.x; t < G * HD; t += dec::kThreads) {
    const int h = t / HD, d = t % HD;
    const float s = (red[0][h][d] + red[1][h][d]) + (red[2][h][d] + red[3][h][d]);
    float *p = a.part + ((size_t)(g * G + h) * a.chunks + c) * kAttnPart;
    dec::st_dev(p + 4 + d, s);
    if (d == 0) {
      dec::st_dev(p, ml[h][0]);
      dec::st_dev(p + 1, ml[h][1]);
    }
  }

  // The last workgroup of this key/value head merges the nc partials.
  if (!dec::arrive_last(a.arrive + g, (uint32_t)c, (uint32_t)nc, &flag)) return;
  constexpr int IT = (G * HD + dec::kThreads - 1) / dec::kThreads;  // (h, d) items per thread
  static_assert(3 * G * 64 + 4 * G <= 4 * G * HD, "the merge's state fits in red");
  if (nc <= 16)
    merge_partials<G, 16>(a, g, nc, &red[0][0][0]);
  else
    merge_partials<G, 64 / IT>(a, g, nc, &red[0][0][0]);
}

// The step's first node: x = x_in and xn = rms_norm_row(x_in) (first
// layer's weight), and the RoPE cos/sin pairs of position *pos (the same for
// every layer), rope[2i] = cos(pos * freq[i]), rope[2i + 1] = sin(...).
__global__ void __launch_bounds__(dec::kThreads)
step_start_kernel(const float *x_in, const float *w, float *xn, float *x, int dim, float eps,
                  const int32_t *pos, const float *freq, float *rope) {
  __shared__ float red[4];
  __shared__ float vs[kNormMaxDim];
  if (threadIdx.x < HD / 2) {
    const float ang = (float)*pos * freq[threadIdx.x];
    float sn, cs;
    sincosf(ang, &sn, &cs);
    rope[2 * threadIdx.x] = cs;
    rope[2 * threadIdx.x + 1] = sn;
  }
  dec::norm_row(x_in, nullptr, x, w, xn, dim, eps, vs, red);
}

__global__ void rope_freq_kernel(float theta, float *freq) {
  const int i = (int)threadIdx.x;
  if (i < HD / 2) {
    const float e = (float)i / (float)(HD / 2);
    const float pw = (float)pow((double)theta, (double)e);
    freq[i] = 1.0f / pw;
  }
}

}  // namespace

int attn_chunks(int cache_rows) { return (cache_rows + CH - 1) / CH; }

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.n_kv * a.chunks));
  switch (a.n_heads / a.n_kv) {
    case 1: hipLaunchKernelGGL(attention_kernel<1>, grid, dim3(dec::kThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL(attention_kernel<2>, grid, dim3(dec::kThreads), 0, s, a); break;
    case 3: hipLaunchKernelGGL(attention_kernel<3>, grid, dim3(dec::kThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL(attention_kernel<4>, grid, dim3(dec::kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_step_start(const float *x_in, const float *w, float *xn, float *x,
                             int dim, float eps, const int32_t *pos, const float *freq,
                             float *rope, hipStream_t s) {
  if (dim < 1 || dim > kNormMaxDim) return hipErrorInvalidValue;
  hipLaunchKernelGGL(step_start_kernel, dim3(1), dim3(dec::kThreads), 0, s, x_in, w, xn, x,
                     dim, eps, pos, freq, rope);
  return hipGetLastError();
}

hipError_t launch_rope_freq(float theta, float *freq, hipStream_t s) {
  hipLaunchKernelGGL(rope_freq_kernel, dim3(1), dim3(64), 0, s, theta, freq);
  return hipGetLastError();
}

}  // namespace q8
