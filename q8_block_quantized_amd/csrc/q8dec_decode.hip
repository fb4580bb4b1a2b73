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

// G query heads per key/value head.
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

  // QK-norm and RoPE of the G queries and the key; lane l holds pair
  // (l, l + 64) of a head.  The value is copied as it is.
  for (int vec = wave; vec < G + 2; vec += 4) {
    if (vec <= G) {
      const float *src = vec < G ? a.q + (size_t)(g * G + vec) * HD : a.k + (size_t)g * HD;
      const float *wn = vec < G ? a.q_norm : a.k_norm;
      const float x0 = src[lane], x1 = src[lane + 64];
      const float ss = dec::wave_sum(x0 * x0 + x1 * x1);
      const float inv = 1.0f / sqrtf(ss / (float)HD + a.eps);
      const float u0 = x0 * inv * wn[lane], u1 = x1 * inv * wn[lane + 64];
      const float ang = (float)pos * a.freq[lane];
      float sn, cs;
      sincosf(ang, &sn, &cs);
      const float r0 = u0 * cs - u1 * sn, r1 = u0 * sn + u1 * cs;
      float *dst = vec < G ? qs[vec] : kn;
      dst[lane] = r0;
      dst[lane + 64] = r1;
      if (vec == G && owner) {
        float *row = a.kc + (size_t)pos * kvw + (size_t)g * HD;
        row[lane] = r0;
        row[lane + 64] = r1;
      }
    } else {
      const float v0 = a.v[(size_t)g * HD + lane], v1 = a.v[(size_t)g * HD + lane + 64];
      vn[lane] = v0;
      vn[lane + 64] = v1;
      if (owner) {
        float *row = a.vc + (size_t)pos * kvw + (size_t)g * HD;
        row[lane] = v0;
        row[lane + 64] = v1;
      }
    }
  }
  __syncthreads();

  // Scores: 16 lanes per cached row (8 dimensions each), 16 rows per pass.
  const int slot = (int)threadIdx.x >> 4, sub = (int)threadIdx.x & 15;
  float kr[4][8];
#pragma unroll
  for (int ps = 0; ps < 4; ps++) {
    const int tl = slot + 16 * ps, t = t0 + tl;
#pragma unroll
    for (int i = 0; i < 8; i++) kr[ps][i] = 0.f;
    if (tl < len) {
      if (t != pos) load8(a.kc + (size_t)t * kvw + (size_t)g * HD + 8 * sub, kr[ps]);
      else load8(kn + 8 * sub, kr[ps]);
    }
  }
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

  // Weighted value rows, same lane mapping as the scores.
  float vr[4][8];
#pragma unroll
  for (int ps = 0; ps < 4; ps++) {
    const int tl = slot + 16 * ps, t = t0 + tl;
#pragma unroll
    for (int i = 0; i < 8; i++) vr[ps][i] = 0.f;
    if (tl < len) {
      if (t != pos) load8(a.vc + (size_t)t * kvw + (size_t)g * HD + 8 * sub, vr[ps]);
      else load8(vn + 8 * sub, vr[ps]);
    }
  }
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
    p[4 + d] = s;
    if (d == 0) {
      p[0] = ml[h][0];
      p[1] = ml[h][1];
    }
  }

  // The last workgroup of this key/value head merges the nc partials, in
  // chunk order: out = sum_c e^(m_c - M) acc_c / sum_c e^(m_c - M) l_c.
  if (!dec::arrive_last(a.arrive + g, (uint32_t)c, (uint32_t)nc, &flag)) return;
  for (int t = (int)threadIdx.x; t < G * HD; t += dec::kThreads) {
    const int h = t / HD, d = t % HD;
    const float *ph = a.part + (size_t)(g * G + h) * a.chunks * kAttnPart;
    float M = -INFINITY;
    for (int cc = 0; cc < nc; cc++) M = fmaxf(M, ph[(size_t)cc * kAttnPart]);
    float L = 0.f, A = 0.f;
    for (int cc = 0; cc < nc; cc++) {
      const float *p = ph + (size_t)cc * kAttnPart;
      const float w = expf(p[0] - M);
      L += p[1] * w;
      A += p[4 + d] * w;
    }
    a.out[(size_t)(g * G + h) * HD + d] = A / L;
  }
}

__global__ void __launch_bounds__(dec::kThreads)
rms_norm_kernel(const float *x, const float *w, float *out, float *copy, int dim,
                float eps) {
  __shared__ float red[4];
  const size_t off = (size_t)blockIdx.x * dim;
  dec::norm_row(x + off, nullptr, copy ? copy + off : nullptr, w, out + off, dim, eps, red);
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

hipError_t launch_rms_norm(const float *x, const float *w, float *out, float *copy,
                           int rows, int dim, float eps, hipStream_t s) {
  if (rows < 1 || dim < 1 || dim > kNormMaxDim) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rms_norm_kernel, dim3((unsigned)rows), dim3(dec::kThreads), 0, s, x, w,
                     out, copy, dim, eps);
  return hipGetLastError();
}

hipError_t launch_rope_freq(float theta, float *freq, hipStream_t s) {
  hipLaunchKernelGGL(rope_freq_kernel, dim3(1), dim3(64), 0, s, theta, freq);
  return hipGetLastError();
}

}  // namespace q8
