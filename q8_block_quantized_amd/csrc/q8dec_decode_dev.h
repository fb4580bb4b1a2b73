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

// Cross-lane steps without LDS: DPP permutations within rows of 16 lanes
// cost a cycle or two, where a __shfl_xor (ds_bpermute) waits for an LDS
// round trip, and v_readlane moves a lane's value to a scalar register.
// Every lane of the wave must be active.  A DPP step combines a lane with
// its partner in the same operand order on both sides (a + b, not b + a),
// so the lanes of a row end with the same bits.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lanef(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum over each row of 16 lanes, in every lane of the row: pairs, quads,
// half-rows, rows.
__device__ __forceinline__ float row16_sum(float v) {
  v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);  // row_half_mirror
  v += dppf<0x140>(v);  // row_mirror
  return v;
}

// Sum over the wave (the row sums, then rows (0 + 1) + (2 + 3)), the same
// value in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}

__device__ __forceinline__ float wave_maxf(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}

// Sum over the 256 threads, the same value returned to every thread, in a
// fixed order (wave_sum in each wave, then the four wave sums pairwise).
// red: 4 floats of LDS.
// A workgroup barrier that orders LDS accesses only: every LDS write before
// it is complete (lgkmcnt) before any wave passes it, and the compiler moves
// no memory access across it.  __syncthreads() also waits for the wave's
// vector memory requests (its fence counts them, as they may be LDS writes),
// and with them for weight loads in flight that the code after the barrier
// does not yet need.
constexpr int kWaitLgkm0 = 0xC07F;  // s_waitcnt lgkmcnt(0), as the builtin's operand
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// block_sum with LDS-only barriers: for callers whose values before and
// after the sum are registers and LDS only.
__device__ __forceinline__ float block_sum_lds(float v, float *red) {
  v = wave_sum(v);
  lds_barrier();  // earlier readers of red are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  lds_barrier();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

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

// ---- attention_decode (inferno.rs "IV.4", "Eight kernels": rope_row,
// append_kv, attention_decode), split over the cache the way MI355X wants
// it: a workgroup takes 64 cached rows of one key/value head for all the
// query heads that share it (GQA), writes a partial softmax (its maximum,
// its sum and its weighted value sum), and the last workgroup of that head
// to finish merges the partials.  The QK-norm and the RoPE of q and k are
// folded into each workgroup's prologue, and the workgroup that holds row
// pos writes this token's key and value into the cache (append_kv); rows
// below pos come from the cache, row pos from registers, so no workgroup
// reads a row another one writes.

constexpr int HD = kAttnHeadDim;
constexpr int CH = kAttnChunk;
static_assert(HD == 128 && CH == 64, "the lane mappings below assume these");

// Sum over the 16 lanes of each 16-lane row.

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
template <int G, int R, bool COH>
__device__ __forceinline__ void merge_partials(const AttnArgs &a, int g, int nc, float *lds) {
  constexpr int IT = (G * HD + kThreads - 1) / kThreads;  // (h, d) items per thread
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
      pm = ld_dev(p);
      pl = ld_dev(p + 1);
    }
    float pa[IT][R];
#pragma unroll
    for (int e = 0; e < IT; e++) {
      const int it = tid + e * kThreads, h = it / HD, d = it % HD;
#pragma unroll
      for (int i = 0; i < R; i++) {
        pa[e][i] = 0.f;
        if (it < G * HD && i < k)
          pa[e][i] = ld_dev(ph + ((size_t)h * a.chunks + c0 + i) * kAttnPart + 4 + d);
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
      const float mo = hs[4 * wave], mn = fmaxf(mo, wave_maxf(m));
      const float r = mo == mn ? 1.f : expf(mo - mn);
      const float w = lane < k ? expf(m - mn) : 0.f;
      const float sl = wave_sum(w * l);
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
      const int it = tid + e * kThreads, h = it < G * HD ? it / HD : 0;
      float v = A[e] * hs[4 * h + 2];
#pragma unroll
      for (int i = 0; i < R; i++) v += mw[h * R + i] * pa[e][i];
      A[e] = v;
    }
    __syncthreads();  // before the next round rewrites mw, ls and hs
  }
#pragma unroll
  for (int e = 0; e < IT; e++) {
    const int it = tid + e * kThreads;
    if (it < G * HD) {
      const float v = A[e] / hs[4 * (it / HD) + 1];
      if (COH) st_dev(&a.out[(size_t)(g * G) * HD + it], v);
      else a.out[(size_t)(g * G) * HD + it] = v;
    }
  }
}

// The LDS of one attention block (G query heads per key/value head).
template <int G>
struct AttnLds {
  float qs[G][HD];      // normed, rotated queries
  float kn[HD];         // this token's key, normed, rotated
  float vn[HD];         // this token's value
  float sc[G][CH];      // scores, then weights
  float ml[G][2];       // chunk maximum and sum
  alignas(16) float red[16][G][HD];  // value sums per 16-lane row, then the merge's state
  uint32_t flag;
};

// Attention block blk = (key/value head g, chunk c) of one token, G query
// heads per key/value head.  Every load the block needs (its vectors, the
// norm weights, the rotation and its 64 cached key and value rows) is issued
// as soon as pos is known, so the whole prologue costs one memory round
// trip.  `wait` is called once, after the cached rows' loads are issued and
// before anything this token's step produced is read (a persistent launch
// waits there for the rest of the grid; the cached rows are older).  COH
// (the persistent launch): the output is stored at device scope (workgroups
// on other XCDs read it in the next phase), and the rotation comes from
// freq instead of the rope table.  q, k, v are plain loads in both forms:
// the persistent launch writes each of them once, before this phase.
template <int G, bool COH, class Wait>
__device__ __forceinline__ void attention_block(const AttnArgs &a, int blk, AttnLds<G> &S,
                                                Wait &&wait) {
  auto &qs = S.qs;
  auto &kn = S.kn;
  auto &vn = S.vn;
  auto &sc = S.sc;
  auto &ml = S.ml;
  auto &red = S.red;
  const int g = blk / a.chunks, c = blk % a.chunks;
  const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
  const int pos = *a.pos;
  if (pos < 0 || pos >= a.cache_rows) {  // no such row: the heads read NaN
    wait();
    if (c == 0)
      for (int t = (int)threadIdx.x; t < G * HD; t += kThreads) {
        if (COH) st_dev(&a.out[(size_t)(g * G) * HD + t], __builtin_nanf(""));
        else a.out[(size_t)(g * G) * HD + t] = __builtin_nanf("");
      }
    return;
  }
  const int seq = pos + 1;
  const int nc = (seq + CH - 1) / CH;
  if (c >= nc) {  // beyond the cached rows: no arrival either
    wait();
    return;
  }
  const int t0 = c * CH;
  const int len = seq - t0 < CH ? seq - t0 : CH;
  const bool owner = pos < t0 + CH;  // this chunk holds row pos
  const size_t kvw = (size_t)a.n_kv * HD;

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
  // the norm weights and the rotation do not depend on the step's values:
  // read and computed while the barrier completes
  const float wq0 = a.q_norm[lane], wq1 = a.q_norm[lane + 64];
  const float wk0 = a.k_norm[lane], wk1 = a.k_norm[lane + 64];
  float cs, sn;
  if (COH) {  // the rotation of this position (as the step's first node computes it)
    const float ang = (float)pos * a.freq[lane];
    sincosf(ang, &sn, &cs);
  } else {
    cs = a.rope[2 * lane];
    sn = a.rope[2 * lane + 1];
  }
  wait();  // everything below reads this step's values
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

  // QK-norm and RoPE of the queries and the key; the value as it is.  The
  // chunk holding row pos appends this token's key and value to the cache.
#pragma unroll
  for (int j = 0; j < NV; j++) {
    const int vec = wave + 4 * j;
    if (vec <= G) {
      const float w0 = vec < G ? wq0 : wk0, w1 = vec < G ? wq1 : wk1;
      const float ss = wave_sum(x0[j] * x0[j] + x1[j] * x1[j]);
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
    const float m = wave_maxf(s);
    const float e = lane < len ? expf(s - m) : 0.f;
    const float l = wave_sum(e);
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
    *(float4 *)&red[slot][h][8 * sub] = float4{acc[0], acc[1], acc[2], acc[3]};
    *(float4 *)&red[slot][h][8 * sub + 4] = float4{acc[4], acc[5], acc[6], acc[7]};
  }
  __syncthreads();
  for (int t = (int)threadIdx.x; t < G * HD; t += kThreads) {
    const int h = t / HD, d = t % HD;
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; k++)
      q[k] = (red[4 * k][h][d] + red[4 * k + 1][h][d]) + (red[4 * k + 2][h][d] + red[4 * k + 3][h][d]);
    const float s = (q[0] + q[1]) + (q[2] + q[3]);
    float *p = a.part + ((size_t)(g * G + h) * a.chunks + c) * kAttnPart;
    st_dev(p + 4 + d, s);
    if (d == 0) {
      st_dev(p, ml[h][0]);
      st_dev(p + 1, ml[h][1]);
    }
  }

  // The last workgroup of this key/value head merges the nc partials.
  if (!arrive_last(a.arrive + g, (uint32_t)c, (uint32_t)nc, &S.flag)) return;
  constexpr int IT = (G * HD + kThreads - 1) / kThreads;  // (h, d) items per thread
  static_assert(3 * G * 64 + 4 * G <= 4 * G * HD, "the merge's state fits in red");
  if (nc <= 16)
    merge_partials<G, 16, COH>(a, g, nc, &red[0][0][0]);
  else
    merge_partials<G, 64 / IT, COH>(a, g, nc, &red[0][0][0]);
}


}  // namespace dec
}  // namespace q8
