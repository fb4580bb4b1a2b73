// gfx950 kernels of libq8dec: the Q8_0 decode matvec, its batched form, the
// argmax, and the fused matvec + argmax.
//
// Q8_0 layout (inferno.rs "IV.4: One command buffer per token", "Eight
// kernels"): a weight row is n/32 blocks of 34 bytes, each a little-endian
// binary16 scale followed by 32 int8 quants covering x[32b .. 32b+31]; the
// kernels read the raw bytes in place (no repacking).
//
// Mapping to CDNA4 (64-lane wavefronts):
//  * A half-wave (32 lanes) owns one weight row; lane k handles blocks
//    k, k+32, k+64, ... of that row, so one wave reads two rows and a load
//    instruction covers contiguous bytes.
//  * A block starts at an even byte offset a.  Each lane loads the nine
//    dwords [a & ~3, (a & ~3) + 36) with dword-aligned dwordx4/dword loads;
//    one v_perm_b32 per quant dword then realigns the quants (byte shift 2
//    or 4), and a shift picks the scale half-word.  The quants convert to
//    f32 with sign extension (SDWA) and accumulate with x by FMA.
//  * The block sum is scaled once per block, as in the page's kernel.
//  * The 32 lane partials of a row reduce with DPP (quad_perm, row mirrors,
//    row_bcast15) without touching memory; the page's simd_sum step.
//  * m = 1 is bandwidth-bound GEMV work, so no MFMA is used.
// The fused argmax keeps a 64-bit key per lane, (order-preserving bits of
// the logit) << 32 | (0xFFFFFFFF - row), so that an unsigned max picks the
// largest logit and, among equal logits, the lowest row (the page's argmax
// tie rule); NaN never enters and -0 is folded onto +0.  Workgroups combine
// with one 64-bit atomic max each; the last workgroup to arrive (an arrival
// counter) writes the index and clears the workspace for the next launch, so
// the result does not depend on workgroup timing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8dec_internal.h"

namespace q8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
typedef uint32_t u32_a4 __attribute__((aligned(4)));
typedef uint16_t u16_a2 __attribute__((aligned(2)));

constexpr int kWG = 256;           // threads per workgroup
constexpr int kWaves = kWG / 64;   // wavefronts per workgroup
constexpr int kMaxGrid = 2048;     // 8 workgroups per CU on 256 CUs

// ---- block decoding ------------------------------------------------------

// The nine dwords covering the 34-byte block at byte offset a of w (a even,
// w 16-byte aligned).  The window may extend two bytes past the block when
// a % 4 == 0; callers use this form only where a next block follows.
__device__ __forceinline__ void load_window(const uint8_t *__restrict__ w,
                                            uint64_t a, uint32_t (&d)[9]) {
  const uint8_t *base = w + (a & ~(uint64_t)3);
  u32x4 lo = __builtin_nontemporal_load((const u32x4_a4 *)base);
  u32x4 hi = __builtin_nontemporal_load((const u32x4_a4 *)(base + 16));
  d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
  d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
  d[8] = __builtin_nontemporal_load((const u32_a4 *)(base + 32));
}

// Same window, but never reads outside the block: the last dword is built
// from two half-word loads, the second only when it lies inside the block.
__device__ __forceinline__ void load_window_exact(const uint8_t *__restrict__ w,
                                                  uint64_t a, uint32_t (&d)[9]) {
  const uint8_t *base = w + (a & ~(uint64_t)3);
  u32x4 lo = __builtin_nontemporal_load((const u32x4_a4 *)base);
  u32x4 hi = __builtin_nontemporal_load((const u32x4_a4 *)(base + 16));
  d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
  d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
  uint32_t t0 = *(const u16_a2 *)(base + 32);
  uint32_t t1 = (a & 2) ? *(const u16_a2 *)(base + 34) : 0u;
  d[8] = t0 | (t1 << 16);
}

// v_perm_b32 selectors that extract quant dword t from (d[t+1]:d[t]): the
// quants start at window byte 2 when a % 4 == 0 and at byte 4 otherwise.
__device__ __forceinline__ uint32_t quant_sel(uint32_t a_mod4) {
  return a_mod4 ? 0x07060504u : 0x05040302u;
}

__device__ __forceinline__ float scale_of(const uint32_t (&d)[9], uint32_t a_mod4) {
  uint16_t bits = (uint16_t)(d[0] >> (a_mod4 ? 16 : 0));
  return (float)__builtin_bit_cast(_Float16, bits);
}

// sum_j q_j * x_j over one block, x_j from registers; two FMA chains.
__device__ __forceinline__ float block_dot(const uint32_t (&d)[9], uint32_t sel,
                                           const float *xr) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int t = 0; t < 8; t++) {
    uint32_t q = __builtin_amdgcn_perm(d[t + 1], d[t], sel);
    float &acc = (t & 1) ? a1 : a0;
    acc = fmaf((float)(int8_t)(q), xr[4 * t + 0], acc);
    acc = fmaf((float)(int8_t)(q >> 8), xr[4 * t + 1], acc);
    acc = fmaf((float)(int8_t)(q >> 16), xr[4 * t + 2], acc);
    acc = fmaf((float)(int8_t)(q >> 24), xr[4 * t + 3], acc);
  }
  return a0 + a1;
}

// The 32 quants of a block as f32, for reuse across activation rows.
__device__ __forceinline__ void block_quants(const uint32_t (&d)[9], uint32_t sel,
                                             float *qf) {
#pragma unroll
  for (int t = 0; t < 8; t++) {
    uint32_t q = __builtin_amdgcn_perm(d[t + 1], d[t], sel);
    qf[4 * t + 0] = (float)(int8_t)(q);
    qf[4 * t + 1] = (float)(int8_t)(q >> 8);
    qf[4 * t + 2] = (float)(int8_t)(q >> 16);
    qf[4 * t + 3] = (float)(int8_t)(q >> 24);
  }
}

__device__ __forceinline__ void load_x32(const float *__restrict__ x, float *xr) {
  const float4 *xv = (const float4 *)x;
#pragma unroll
  for (int t = 0; t < 8; t++) {
    float4 v = xv[t];
    xr[4 * t + 0] = v.x; xr[4 * t + 1] = v.y;
    xr[4 * t + 2] = v.z; xr[4 * t + 3] = v.w;
  }
}

// ---- cross-lane reductions ---------------------------------------------

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         ROW_MASK, 0xF, false));
}

// Sum over each half-wave: afterwards lanes 16..31 hold the sum of lanes
// 0..31 and lanes 48..63 the sum of lanes 32..63.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_shift<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v += dpp_shift<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v += dpp_shift<0x141, 0xF>(v);  // row_half_mirror
  v += dpp_shift<0x140, 0xF>(v);  // row_mirror
  v += dpp_shift<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long u = __shfl_xor(v, o);
    v = u > v ? u : v;
  }
  return v;
}

// ---- argmax keys --------------------------------------------------------

__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t row) {
  if (v != v) return 0ull;  // NaN never wins
  uint32_t b = __builtin_bit_cast(uint32_t, v);
  if ((b & 0x7FFFFFFFu) == 0u) b = 0u;  // -0 == +0
  uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (unsigned long long)(0xFFFFFFFFu - row);
}

__device__ __forceinline__ int32_t key_index(unsigned long long k) {
  return k ? (int32_t)(0xFFFFFFFFu - (uint32_t)k) : -1;
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a,
                                                     unsigned long long b) {
  return a > b ? a : b;
}

// Combines the per-thread keys best[0..m-1] of this workgroup into the slot;
// the `arrivals`-th workgroup to get here writes idx[0..m-1] and clears the
// slot.  Every workgroup of the launch must call it exactly once.
__device__ void argmax_finish(const unsigned long long *best, int m,
                              ArgmaxSlot *__restrict__ slot,
                              int32_t *__restrict__ idx, uint32_t arrivals) {
  __shared__ unsigned long long red[kWaves][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    if (i < m) {
      unsigned long long v = wave_max_u64(best[i]);
      if (lane == 0) red[wave][i] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < m; i++) {
      unsigned long long v = red[0][i];
      for (int s = 1; s < kWaves; s++) v = umax64(v, red[s][i]);
      if (v)
        __hip_atomic_fetch_max(&slot->keys[i], v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    uint32_t prev = __hip_atomic_fetch_add(&slot->counter, 1u, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
    if (prev == arrivals - 1u) {
      for (int i = 0; i < m; i++) {
        unsigned long long k = __hip_atomic_exchange(
            &slot->keys[i], 0ull, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        idx[i] = key_index(k);
      }
      __hip_atomic_store(&slot->counter, 0u, __ATOMIC_RELEASE,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- m = 1, n = 1024 * NB (the model's widths) --------------------------
//
// x is staged once per workgroup through LDS (4 pad floats after every 32,
// so the per-lane 128-byte reads hit distinct banks) into 32 * NB registers
// per lane: lane k's columns never change, so x is read from LDS once.
// Each wave handles RPW row pairs per iteration (grid-stride loop).
template <int NB, int RPW, bool ARGMAX>
__global__ void __launch_bounds__(kWG)
mv1_fast(const uint8_t *__restrict__ w, const float *__restrict__ x,
         float *__restrict__ y, int32_t p, ArgmaxSlot *__restrict__ slot,
         int32_t *__restrict__ idx) {
  constexpr int BPR = 32 * NB;
  constexpr uint32_t PITCH = BPR * 34u;
  __shared__ __attribute__((aligned(16))) float xs[BPR * 36];
  const int tid = threadIdx.x, lane = tid & 63, k = lane & 31, half = lane >> 5;

  for (int c = tid; c < BPR * 8; c += kWG) {
    float4 v = ((const float4 *)x)[c];
    *(float4 *)&xs[(c >> 3) * 36 + (c & 7) * 4] = v;
  }
  __syncthreads();
  float xr[NB][32];
#pragma unroll
  for (int i = 0; i < NB; i++) {
#pragma unroll
    for (int t = 0; t < 8; t++) {
      float4 v = *(const float4 *)&xs[(k + 32 * i) * 36 + 4 * t];
      xr[i][4 * t + 0] = v.x; xr[i][4 * t + 1] = v.y;
      xr[i][4 * t + 2] = v.z; xr[i][4 * t + 3] = v.w;
    }
  }
  // a % 4 of every block this lane reads (row pitch is a multiple of 16)
  const uint32_t amod = (uint32_t)(k & 1) * 2u;
  const uint32_t sel = quant_sel(amod);
  const int32_t pairs = (p + 1) >> 1;
  const int32_t wave_id = blockIdx.x * kWaves + (tid >> 6);
  const int32_t stride = gridDim.x * kWaves * RPW;
  unsigned long long best = 0ull;

  for (int32_t pb = wave_id * RPW; pb < pairs; pb += stride) {
    uint32_t d[RPW][NB][9];
#pragma unroll
    for (int j = 0; j < RPW; j++) {
      int32_t r = 2 * (pb + j) + half;
      int32_t rc = r < p ? r : p - 1;
#pragma unroll
      for (int i = 0; i < NB; i++)
        load_window(w, (uint64_t)rc * PITCH + (uint32_t)(k + 32 * i) * 34u,
                    d[j][i]);
    }
#pragma unroll
    for (int j = 0; j < RPW; j++) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NB; i++)
        acc = fmaf(scale_of(d[j][i], amod), block_dot(d[j][i], sel, xr[i]), acc);
      acc = half_wave_sum(acc);
      int32_t r = 2 * (pb + j) + half;
      if (k == 31 && r < p) {
        if (y) y[r] = acc;
        if (ARGMAX) best = umax64(best, argmax_key(acc, (uint32_t)r));
      }
    }
  }
  if (ARGMAX) argmax_finish(&best, 1, slot, idx, gridDim.x);
}

// ---- any n (n % 32 == 0), 1 <= m <= 8 --------------------------------
//
// Same row mapping; x is read from global memory per block (it stays in the
// caches), and for m > 1 each block's quants are converted once and reused
// for all m activation rows.
template <bool ARGMAX>
__global__ void __launch_bounds__(kWG)
mv_generic(const uint8_t *__restrict__ w, const float *__restrict__ x,
           float *__restrict__ y, int32_t m, int32_t n, int32_t p,
           ArgmaxSlot *__restrict__ slot, int32_t *__restrict__ idx) {
  const int tid = threadIdx.x, lane = tid & 63, k = lane & 31, half = lane >> 5;
  const int32_t bpr = n >> 5;
  const uint64_t pitch = (uint64_t)bpr * 34u;
  const int32_t pairs = (p + 1) >> 1;
  const int32_t wave_id = blockIdx.x * kWaves + (tid >> 6);
  const int32_t stride = gridDim.x * kWaves;
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};

  for (int32_t pb = wave_id; pb < pairs; pb += stride) {
    const int32_t r = 2 * pb + half;
    const int32_t rc = r < p ? r : p - 1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int32_t b = k; b < bpr; b += 32) {
      const uint64_t a = (uint64_t)rc * pitch + (uint64_t)b * 34u;
      uint32_t d[9];
      load_window_exact(w, a, d);
      const uint32_t amod = (uint32_t)a & 2u;
      const uint32_t sel = quant_sel(amod);
      const float s = scale_of(d, amod);
      if (m == 1) {
        float xr[32];
        load_x32(x + 32 * (int64_t)b, xr);
        acc[0] = fmaf(s, block_dot(d, sel, xr), acc[0]);
      } else {
        float qf[32];
        block_quants(d, sel, qf);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (i < m) {
            float xr[32];
            load_x32(x + (int64_t)i * n + 32 * (int64_t)b, xr);
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int j = 0; j < 32; j += 2) {
              a0 = fmaf(qf[j], xr[j], a0);
              a1 = fmaf(qf[j + 1], xr[j + 1], a1);
            }
            acc[i] = fmaf(s, a0 + a1, acc[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i < m) {
        float v = half_wave_sum(acc[i]);
        if (k == 31 && r < p) {
          if (y) y[(int64_t)i * p + r] = v;
          if (ARGMAX) best[i] = umax64(best[i], argmax_key(v, (uint32_t)r));
        }
      }
    }
  }
  if (ARGMAX) argmax_finish(best, m, slot, idx, gridDim.x);
}

// ---- argmax over f32 logits ---------------------------------------------
// grid.y = activation row; every workgroup of the grid arrives once.
__global__ void __launch_bounds__(kWG)
argmax_rows(const float *__restrict__ logits, int32_t m, int32_t p,
            ArgmaxSlot *__restrict__ slot, int32_t *__restrict__ idx) {
  const float *row = logits + (int64_t)blockIdx.y * p;
  unsigned long long key = 0ull;
  for (int32_t e = blockIdx.x * kWG + threadIdx.x; e < p; e += gridDim.x * kWG)
    key = umax64(key, argmax_key(row[e], (uint32_t)e));
  // per-row keys: only entry blockIdx.y is live in this workgroup
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int i = 0; i < 8; i++)
    if (i == (int)blockIdx.y) best[i] = key;
  argmax_finish(best, m, slot, idx, gridDim.x * gridDim.y);
}

int grid_for_pairs(int32_t pairs, int pairs_per_wave) {
  int64_t waves = ((int64_t)pairs + pairs_per_wave - 1) / pairs_per_wave;
  int64_t wgs = (waves + kWaves - 1) / kWaves;
  if (wgs < 1) wgs = 1;
  return (int)(wgs < kMaxGrid ? wgs : kMaxGrid);
}

template <int NB, int RPW>
hipError_t launch_fast(const uint8_t *w, const float *x, float *y, int p,
                       ArgmaxSlot *slot, int32_t *idx, hipStream_t s) {
  const int grid = grid_for_pairs((p + 1) / 2, RPW);
  if (slot)
    hipLaunchKernelGGL((mv1_fast<NB, RPW, true>), dim3(grid), dim3(kWG), 0, s,
                       w, x, y, p, slot, idx);
  else
    hipLaunchKernelGGL((mv1_fast<NB, RPW, false>), dim3(grid), dim3(kWG), 0, s,
                       w, x, y, p, slot, idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_matvec(const uint8_t *w, const float *x, float *y, int m,
                         int n, int p, ArgmaxSlot *slot, int32_t *idx,
                         hipStream_t s) {
  if (p <= 0) return hipSuccess;
  if (m == 1) {
    switch (n) {
      case 1024: return launch_fast<1, 2>(w, x, y, p, slot, idx, s);
      case 2048: return launch_fast<2, 1>(w, x, y, p, slot, idx, s);
      case 3072: return launch_fast<3, 1>(w, x, y, p, slot, idx, s);
      default: break;
    }
  }
  const int grid = grid_for_pairs((p + 1) / 2, 1);
  if (slot)
    hipLaunchKernelGGL((mv_generic<true>), dim3(grid), dim3(kWG), 0, s, w, x,
                       y, m, n, p, slot, idx);
  else
    hipLaunchKernelGGL((mv_generic<false>), dim3(grid), dim3(kWG), 0, s, w, x,
                       y, m, n, p, slot, idx);
  return hipGetLastError();
}

hipError_t launch_argmax(const float *logits, int m, int p, ArgmaxSlot *slot,
                         int32_t *idx, hipStream_t s) {
  int64_t per = ((int64_t)p + kWG * 8 - 1) / (kWG * 8);  // ~8 values per thread
  int gx = (int)(per < 1 ? 1 : (per > 512 ? 512 : per));
  hipLaunchKernelGGL(argmax_rows, dim3(gx, m), dim3(kWG), 0, s, logits, m, p,
                     slot, idx);
  return hipGetLastError();
}

const void *probe_kernel() { return (const void *)&argmax_rows; }

// The persistent step kernel is added separately; until then these report
// that no persistent mode exists.
int step_rows_per_tile(int, int) { return 0; }
int step_grid(int) { return 0; }
hipError_t launch_step(const StepDesc *, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace q8
