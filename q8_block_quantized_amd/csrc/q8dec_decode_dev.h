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

// Values one workgroup hands to another inside a launch travel with
// device-scope (agent) accesses: the store writes through to the point where
// every XCD's L2 sees it, the load does not take a stale L2 copy.  These are
// the accesses the AMDGPU memory model uses for agent-scope atomics, and
// they avoid the agent-scope fences, whose L2 write-back and invalidate cost
// microseconds when every wave of a launch issues them.
__device__ __forceinline__ void st_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

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
// with all of its threads, after its last device-scope store (st_dev or the
// matvec's output stores).  It returns true in every thread of the one
// workgroup that arrives last, which can then read with ld_dev what all the
// others stored.  Each wave first waits until its stores are complete (on
// gfx9 the vector memory counter covers stores), then one thread counts the
// arrival; a workgroup's arrival is therefore ordered after its stores, and
// the last arrival's loads after every arrival.  Arrivals go through team
// counters (workgroup wg joins team wg % kArgmaxTeams), so no counter takes
// more than one arrival per team member; each counter is back at zero when
// the last arrival returns.  flag: one word of LDS.
__device__ __forceinline__ bool arrive_last(ArgmaxSlot *s, uint32_t wg, uint32_t nwg,
                                            uint32_t *flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t T = kArgmaxTeams;
    const uint32_t j = wg % T;
    const uint32_t size = (nwg - j + T - 1) / T, nteams = nwg < T ? nwg : T;
    uint32_t last = 0;
    ArgmaxGroup *g = &s->team[j];
    // with at most T arrivals every team has one member: count at the top only
    const uint32_t prev = nwg <= T ? 0u
                                   : __hip_atomic_fetch_add(&g->counter, 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
    if (prev == size - 1u) {
      if (nwg > T)
        __hip_atomic_store(&g->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t p2 = __hip_atomic_fetch_add(&s->top.counter, 1u, __ATOMIC_RELAXED,
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
  return *flag != 0u;
}

// rms_norm_row by one workgroup over n <= kNormMaxDim values: v = src (+ r
// when r is set; r is read with ld_dev), dst = v (when dst is set), out = v /
// sqrt(mean(v^2) + eps) * g.  src and dst may be the same array.  Rounds of
// 4 values per thread, each round's loads issued together (device-scope
// loads keep their order, so interleaving them with arithmetic would wait
// once per value); v is kept in LDS between the two passes.  vs: n floats
// of LDS; red: 4 floats of LDS.
__device__ __forceinline__ void norm_row(const float *src, const float *r, float *dst,
                                         const float *g, float *out, int n, float eps,
                                         float *vs, float *red) {
  constexpr int K = 4;
  float ss = 0.f;
  for (int i0 = 0; i0 < n; i0 += K * kThreads) {
    float a[K], b[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      b[k] = 0.f;
      if (r && i < n) b[k] = ld_dev(r + i);
    }
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      a[k] = i < n ? src[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      const float v = r ? a[k] + b[k] : a[k];
      if (i < n) {
        vs[i] = v;
        if (dst) dst[i] = v;
      }
      ss += v * v;
    }
  }
  ss = block_sum(ss, red);  // its barriers also publish vs
  const float inv = 1.0f / sqrtf(ss / (float)n + eps);
  for (int i0 = 0; i0 < n; i0 += K * kThreads) {
    float gv[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      gv[k] = i < n ? g[i] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      if (i < n) out[i] = vs[i] * inv * gv[k];
    }
  }
}

// silu_hadamard by one workgroup: out = gate / (1 + e^-gate) * up (gate and
// up read with ld_dev, 6 of each per thread per round, loaded together).
__device__ __forceinline__ void silu_mul(const float *gate, const float *up, float *out,
                                         int n) {
  constexpr int K = 6;
  for (int i0 = 0; i0 < n; i0 += K * kThreads) {
    float gv[K], uv[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      gv[k] = uv[k] = 0.f;
      if (i < n) {
        gv[k] = ld_dev(gate + i);
        uv[k] = ld_dev(up + i);
      }
    }
#pragma unroll
    for (int k = 0; k < K; k++) {
      const int i = i0 + (int)threadIdx.x + k * kThreads;
      if (i < n) out[i] = gv[k] / (1.0f + expf(-gv[k])) * uv[k];
    }
  }
}

// The epilogue of a persistent step launch (see Epilogue): called by every
// workgroup after its tiles.  lds: at least 8 + kNormMaxDim floats no longer
// in use.
__device__ __forceinline__ void run_epilogue(const Epilogue *e, uint32_t wg, uint32_t nwg,
                                             float *lds) {
  if (!arrive_last(e->arrive, wg, nwg, (uint32_t *)lds)) return;
  if (e->op == kEpiAddNorm)
    norm_row(e->x, e->r, e->x, e->g, e->out, e->n, e->eps, lds + 8, lds + 4);
  else if (e->op == kEpiSiluMul)
    silu_mul(e->g, e->r, e->out, e->n);
}

}  // namespace dec
}  // namespace q8
