// The decode step's attention and norm nodes on gfx950 (inferno.rs "IV.4",
// "Eight kernels": rms_norm_row, rope_row, append_kv, attention_decode).
// The attention itself (attention_block, q8dec_decode_dev.h) is shared with
// the persistent decode step; here it runs as one graph node, one block per
// workgroup.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "q8dec_decode_dev.h"
#include "q8dec_internal.h"

namespace q8 {
namespace {

using dec::CH;
using dec::HD;

// The attention node of the decode graph: one block per workgroup.
template <int G>
__global__ void __launch_bounds__(dec::kThreads) attention_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) dec::AttnLds<G> S;
  dec::attention_block<G, false>(a, (int)blockIdx.x, S, [] {});
}

// The step's first node: the RoPE cos/sin pairs of position *pos (the same
// for every layer), rope[2i] = cos(pos * freq[i]), rope[2i + 1] = sin(...),
// and, when x_in is set, x = x_in and xn = rms_norm_row(x_in) (the first
// layer's weight; otherwise the first q/k/v launch's prologue computes xn).
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
  if (x_in) dec::norm_row(x_in, nullptr, x, w, xn, dim, eps, vs, red);
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
