// Device helpers of the decode step's non-matvec work (inferno.rs "IV.4",
// "Eight kernels": rms_norm_row, add_inplace, silu_hadamard), shared by the
// kernel sources: cross-workgroup completion, 256-thread reductions, the
// row norm and the SwiGLU product.  Every function is inline.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8dec_internal.h"

namespace q8 {
namespace dec {

constexpr int kThreads = 256;  // workgroup size of every decode kernel

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

__device__ __forceinline__ float wave_maxf(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// Sum over the 256 threads, the same value returned to every thread, in a
// fixed order (butterfly in each wave, then the four wave sums pairwise).
// red: 4 floats of LDS.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Completion of a launch: every workgroup wg in [0, nwg) calls this once,
// with all of its threads, after its last global store.  It returns true in
// every thread of the one workgroup that arrives last, which then reads what
// all the others wrote.  Arrivals go through team counters (workgroup wg
// joins team wg % kArgmaxTeams), so no counter takes more than one arrival
// per team member; each counter is back at zero when the last arrival
// returns.  flag: one word of LDS.
__device__ __forceinline__ bool arrive_last(ArgmaxSlot *s, uint32_t wg, uint32_t nwg,
                                            uint32_t *flag) {
  // each wave's stores are complete and written back at device scope
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t T = kArgmaxTeams;
    const uint32_t j = wg % T;
    const uint32_t size = (nwg - j + T - 1) / T, nteams = nwg < T ? nwg : T;
    uint32_t last = 0;
    ArgmaxGroup *g = &s->team[j];
    const uint32_t prev = __hip_atomic_fetch_add(&g->counter, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == size - 1u) {
      __hip_atomic_store(&g->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t p2 = __hip_atomic_fetch_add(&s->top.counter, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
      if (p2 == nteams - 1u) {
        __hip_atomic_store(&s->top.counter, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        last = 1u;
      }
    }
    *flag = last;
  }
  __syncthreads();
  const bool last = *flag != 0u;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// rms_norm_row by one workgroup over n <= kNormMaxDim values: v = src (+ r
// when r is set), dst = v (when dst is set), out = v / sqrt(mean(v^2) + eps)
// * g.  src and dst may be the same array.  red: 4 floats of LDS.
__device__ __forceinline__ void norm_row(const float *src, const float *r, float *dst,
                                         const float *g, float *out, int n, float eps,
                                         float *red) {
  constexpr int K = kNormMaxDim / kThreads;
  float v[K];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < K; k++) {
    const int i = (int)threadIdx.x + k * kThreads;
    v[k] = 0.f;
    if (i < n) v[k] = r ? src[i] + r[i] : src[i];
  }
#pragma unroll
  for (int k = 0; k < K; k++) {
    const int i = (int)threadIdx.x + k * kThreads;
    if (i < n && dst) dst[i] = v[k];
    ss += v[k] * v[k];
  }
  ss = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(ss / (float)n + eps);
#pragma unroll
  for (int k = 0; k < K; k++) {
    const int i = (int)threadIdx.x + k * kThreads;
    if (i < n) out[i] = v[k] * inv * g[i];
  }
}

// silu_hadamard by one workgroup: out = gate / (1 + e^-gate) * up.
__device__ __forceinline__ void silu_mul(const float *gate, const float *up, float *out,
                                         int n) {
  for (int i = (int)threadIdx.x; i < n; i += kThreads) {
    const float gv = gate[i];
    out[i] = gv / (1.0f + expf(-gv)) * up[i];
  }
}

// The epilogue of a persistent step launch (see Epilogue): called by every
// workgroup after its tiles.  lds: at least 8 words no longer in use.
__device__ __forceinline__ void run_epilogue(const Epilogue *e, uint32_t wg, uint32_t nwg,
                                             float *lds) {
  if (!arrive_last(e->arrive, wg, nwg, (uint32_t *)lds)) return;
  if (e->op == kEpiAddNorm)
    norm_row(e->x, e->r, e->x, e->g, e->out, e->n, e->eps, lds + 4);
  else if (e->op == kEpiSiluMul)
    silu_mul(e->g, e->r, e->out, e->n);
}

}  // namespace dec
}  // namespace q8
