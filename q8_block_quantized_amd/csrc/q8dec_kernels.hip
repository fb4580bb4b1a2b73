// gfx950 kernels of libq8dec: the Q8_0 decode matvec, its batched form, the
// argmax, the fused matvec + argmax, and the persistent decode-step kernel.
//
// Q8_0 layout (inferno.rs "IV.4: One command buffer per token", "Eight
// kernels"): a weight row is n/32 blocks of 34 bytes, each a little-endian
// binary16 scale followed by 32 int8 quants covering x[32b .. 32b+31]; the
// kernels read the raw bytes in place (no repacking).
//
// Mapping to CDNA4 (64-lane wavefronts):
//  * Work is cut into tiles: a run of consecutive rows of one matvec.  A
//    workgroup (4 waves) processes a tile 8 rows at a time: each half-wave
//    (32 lanes) owns one row and lane k handles blocks k, k+32, k+64 of it,
//    so one load instruction of a wave covers contiguous bytes.  Each lane
//    keeps the blocks of several rows in flight before it computes.
//  * A block starts at an even byte offset a.  Each lane loads the nine
//    dwords [a & ~3, (a & ~3) + 36) with dword-aligned dwordx4/dword loads;
//    one v_perm_b32 per quant dword then realigns the quants (byte shift 2
//    or 4) and a shift picks the scale half-word.  The quants convert to f32
//    with sign extension (SDWA) and accumulate with x by FMA; the block sum
//    is scaled once per block (the q8_matvec listing of inferno.rs "IV.4:
//    One command buffer per token", section "Eight kernels").
//  * x is staged once per matvec in LDS with 4 pad floats after every 32,
//    so the 128-byte per-lane reads of one block hit distinct banks.
//  * The 32 lane partials of a row reduce with DPP (quad_perm, row mirrors,
//    row_bcast15) without touching memory (the simd_sum step of the same
//    listing).
//  * m = 1 is bandwidth-bound GEMV work, so no MFMA is used.
// The fused argmax keeps a 64-bit key per lane, (order-preserving bits of
// the logit) << 32 | (0xFFFFFFFF - row), so an unsigned max picks the
// largest logit and, among equal logits, the lowest row (the argmax_row
// tie rule); NaN never enters and -0 is folded onto +0.  Each arrival (a
// workgroup, or a tile of the step) adds its key with one 64-bit atomic max;
// the last arrival (an arrival counter) writes the index and clears the
// workspace for the next launch, so the result does not depend on timing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8dec_internal.h"

namespace q8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef u32x4 u32x4_a4 __attribute__((aligned(4)));
typedef uint32_t u32_a4 __attribute__((aligned(4)));
typedef uint16_t u16_a2 __attribute__((aligned(2)));

// Pointers read from descriptors are generic; these casts tell the compiler
// they address global memory, so it emits global_load/global_store rather
// than flat accesses.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *gp(const T *p) {
  return (const __attribute__((address_space(1))) T *)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gpw(T *p) {
  return (__attribute__((address_space(1))) T *)p;
}

constexpr int kWG = 256;           // threads per workgroup
constexpr int kWaves = kWG / 64;   // wavefronts per workgroup
constexpr int kRowsPerPass = 2 * kWaves;

// ---- block decoding ------------------------------------------------------

// The nine dwords covering the 34-byte block at byte offset a of w (a even,
// w 16-byte aligned).  When a % 4 == 0 the window ends two bytes past the
// block, so this form is used only where more bytes follow.
__device__ __forceinline__ void load_window(const uint8_t *__restrict__ w,
                                            uint64_t a, uint32_t (&d)[9]) {
  const uint8_t *base = w + (a & ~(uint64_t)3);
  u32x4 lo = __builtin_nontemporal_load((const u32x4_a4 *)base);
  u32x4 hi = __builtin_nontemporal_load((const u32x4_a4 *)(base + 16));
  d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
  d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
  d[8] = __builtin_nontemporal_load((const u32_a4 *)(base + 32));
}

// Same window, never reading outside the block: the last dword is built from
// two half-word loads, the second only when it lies inside the block.
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

// The window of block a of a weight matrix of `wbytes` bytes.
__device__ __forceinline__ void fetch_block(const uint8_t *__restrict__ w,
                                            uint64_t wbytes, uint64_t a,
                                            uint32_t (&d)[9]) {
  if ((a & 2) || a + 36 <= wbytes) load_window(w, a, d);
  else load_window_exact(w, a, d);
}

// v_perm_b32 selector extracting quant dword t from (d[t+1]:d[t]): quants
// start at window byte 2 when a % 4 == 0 and at byte 4 when a % 4 == 2.
__device__ __forceinline__ uint32_t quant_sel(uint32_t amod) {
  return amod ? 0x07060504u : 0x05040302u;
}

__device__ __forceinline__ float scale_of(const uint32_t (&d)[9], uint32_t amod) {
  uint16_t bits = (uint16_t)(d[0] >> (amod ? 16 : 0));
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

__device__ __forceinline__ float dot32(const float *qf, const float *xr) {
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    a0 = fmaf(qf[j], xr[j], a0);
    a1 = fmaf(qf[j + 1], xr[j + 1], a1);
  }
  return a0 + a1;
}

// 32 consecutive floats (16-byte aligned), global or LDS.
__device__ __forceinline__ void load_x32(const float *x, float *xr) {
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

// Adds this workgroup's keys best[0..m-1] to the slot.  Workgroup `wg` of a
// grid of `nwg` joins team wg % kArgmaxTeams; the team's last arrival moves
// the team keys to the top group, and the top group's last arrival writes
// idx[0..m-1].  Arrival counts come from the groups' `expected` fields, or,
// when those are 0, from "every workgroup arrives once".  Atomics are
// relaxed: each counter increment is issued only after the key updates
// before it have returned (performed at the memory side), which orders them
// without L2 write-back or invalidation.  Called by every thread of the
// workgroup.
// `scratch` is kWaves * 8 * 8 bytes of LDS that no thread reads or writes
// meanwhile.
__device__ void argmax_finish(const unsigned long long *best, int m,
                              ArgmaxSlot *__restrict__ slot,
                              int32_t *__restrict__ idx, uint32_t wg,
                              uint32_t nwg, void *scratch) {
  unsigned long long(*red)[8] = (unsigned long long(*)[8])scratch;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < 8; r++) {
    if (r < m) {
      unsigned long long v = wave_max_u64(best[r]);
      if (lane == 0) red[wave][r] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t T = kArgmaxTeams;
    const uint32_t j = wg % T;
    ArgmaxGroup *g = &slot->team[j];
    uint32_t size = gp(&g->expected)[0], nteams = gp(&slot->top.expected)[0];
    if (size == 0u) {
      size = (nwg - j + T - 1) / T;
      nteams = nwg < T ? nwg : T;
    }
    unsigned long long v[8];
    unsigned long long dep = 0ull;
    for (int r = 0; r < m; r++) {
      v[r] = red[0][r];
      for (int w = 1; w < kWaves; w++) v[r] = umax64(v[r], red[w][r]);
      dep |= __hip_atomic_fetch_max(&g->keys[r], v[r], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("" ::"v"(dep));  // the maxima have returned
    const uint32_t prev = __hip_atomic_fetch_add(&g->counter, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == size - 1u) {
      dep = 0ull;
      for (int r = 0; r < m; r++) {
        const unsigned long long tk = __hip_atomic_exchange(
            &g->keys[r], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        dep |= __hip_atomic_fetch_max(&slot->top.keys[r], tk, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      }
      __hip_atomic_store(&g->counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asm volatile("" ::"v"(dep));
      const uint32_t p2 = __hip_atomic_fetch_add(&slot->top.counter, 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (p2 == nteams - 1u) {
        for (int r = 0; r < m; r++)
          idx[r] = key_index(__hip_atomic_exchange(&slot->top.keys[r], 0ull,
                                                   __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT));
        __hip_atomic_store(&slot->top.counter, 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();  // the scratch is free again
}

// ---- matvec geometry ---------------------------------------------------------

// How the tiles of a matvec are processed.
//  kStaged : the tile's rows are streamed with coalesced, 16-byte aligned
//            loads (whole rows are contiguous) into registers one tile ahead,
//            written to LDS, and each lane reads its blocks' windows from LDS.
//            Needs a row pitch that is a multiple of 16 (n/32 % 8 == 0).
//  kDirect : each lane loads its blocks' windows straight from global
//            memory (dword aligned, 34-byte lane stride); any row pitch.
//  kGeneric: as kDirect, but x is read from global memory (large m * n).
enum Path : int { kStaged = 0, kDirect = 1, kGeneric = 2 };

#ifndef Q8_TILE_BYTES
#define Q8_TILE_BYTES 26112  // 8 rows of 3072 columns
#endif
#ifndef Q8_MIN_WGS_PER_CU
#define Q8_MIN_WGS_PER_CU 1
#endif
constexpr int kTileMaxBytes = Q8_TILE_BYTES;
constexpr int kStageChunks = (kTileMaxBytes + 16 * kWG - 1) / (16 * kWG);
constexpr int kXMaxFloats = 8192;     // m * n of x kept in LDS (32 KB)
constexpr int kMaxLdsBlocks = 96;     // n <= 3072 for the LDS paths

__host__ __device__ inline int path_of(int m, int n) {
  const int bpr = n >> 5;
  if (bpr == 0 || bpr > kMaxLdsBlocks || m * n > kXMaxFloats) return kGeneric;
  return (bpr % 8 == 0) ? kStaged : kDirect;
}

__host__ __device__ inline int nbl_of(int n) { return ((n >> 5) + 31) >> 5; }

// Rows per tile: staged tiles fill up to kTileMaxBytes (at least one pass of
// 8 rows); direct and generic tiles are two or four passes.
__host__ __device__ inline int tile_rows_of(int m, int n) {
  const int path = path_of(m, n);
  if (path == kStaged) {
    const int r = kTileMaxBytes / ((n >> 5) * 34);
    return r >= 64 ? 64 : (r < 1 ? 1 : r);
  }
  return path == kDirect && m == 1 ? 32 : 16;
}

// LDS floats of staged x for m rows of width n (4 pad floats per block).
__host__ __device__ inline int x_lds_floats(int m, int n) {
  return m * (n >> 5) * 36;
}

// ---- direct paths (x in LDS or global, weights straight from global) ------

struct Tile {
  const uint8_t *w;
  uint64_t wbytes;
  const float *xg;  // x in global memory, [m][n]
  const float *xs;  // x staged in LDS (padded), or nullptr
  float *y;         // [m][p] or nullptr
  int32_t n, bpr, p, m;
  int32_t r0, r1;   // rows [r0, r1) of this tile, r1 <= p
};

// Direct path, m = 1, x in LDS.  NBL = blocks per lane per row (ceil(bpr / 32)); each
// half-wave keeps U rows (U * NBL blocks per lane) in flight.  The loads are
// unconditional (row and block indices are clamped into the matrix, and the
// contributions of clamped lanes are masked afterwards) so the compiler can
// issue all of them before the first wait.  Needs a full window for every
// block: see needs_exact_tail.
template <int NBL, int U>
__device__ __forceinline__ void direct_m1(const Tile &c, unsigned long long &best,
                                        bool keys) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const uint64_t pitch = (uint64_t)c.bpr * 34u;
  for (int32_t rb = c.r0 + 2 * wave; rb < c.r1; rb += kRowsPerPass * U) {
    uint32_t d[U][NBL][9];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int32_t r = rb + kRowsPerPass * u + half;
      const int32_t rc = r < c.r1 ? r : c.r1 - 1;
#pragma unroll
      for (int i = 0; i < NBL; i++) {
        const int32_t b = min(k + 32 * i, c.bpr - 1);
        load_window(c.w, (uint64_t)rc * pitch + (uint64_t)b * 34u, d[u][i]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int32_t r = rb + kRowsPerPass * u + half;
      const int32_t rc = r < c.r1 ? r : c.r1 - 1;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NBL; i++) {
        const int32_t b = min(k + 32 * i, c.bpr - 1);
        const uint32_t amod = (uint32_t)(((int64_t)rc * c.bpr + b) & 1) * 2u;
        float xr[32];
        load_x32(c.xs + 36 * b, xr);
        const float v = scale_of(d[u][i], amod) * block_dot(d[u][i], quant_sel(amod), xr);
        acc += (k + 32 * i < c.bpr) ? v : 0.f;
      }
      acc = half_wave_sum(acc);
      if (k == 31 && r < c.r1) {
        if (c.y) c.y[r] = acc;
        if (keys) best = umax64(best, argmax_key(acc, (uint32_t)r));
      }
    }
  }
}

// Direct path, 1 < m <= 8, x in LDS: each block's quants convert once and serve m rows.
// Same load scheme as direct_m1.
template <int NBL, int U>
__device__ __forceinline__ void direct_mb(const Tile &c, unsigned long long *best,
                                        bool keys) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const uint64_t pitch = (uint64_t)c.bpr * 34u;
  const int xstride = 36 * c.bpr;
  for (int32_t rb = c.r0 + 2 * wave; rb < c.r1; rb += kRowsPerPass * U) {
    uint32_t d[U][NBL][9];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int32_t r = rb + kRowsPerPass * u + half;
      const int32_t rc = r < c.r1 ? r : c.r1 - 1;
#pragma unroll
      for (int i = 0; i < NBL; i++) {
        const int32_t b = min(k + 32 * i, c.bpr - 1);
        load_window(c.w, (uint64_t)rc * pitch + (uint64_t)b * 34u, d[u][i]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      const int32_t r = rb + kRowsPerPass * u + half;
      const int32_t rc = r < c.r1 ? r : c.r1 - 1;
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NBL; i++) {
        const int32_t b = min(k + 32 * i, c.bpr - 1);
        const bool live = k + 32 * i < c.bpr;
        const uint32_t amod = (uint32_t)(((int64_t)rc * c.bpr + b) & 1) * 2u;
        const float s = live ? scale_of(d[u][i], amod) : 0.f;
        float qf[32];
        block_quants(d[u][i], quant_sel(amod), qf);
#pragma unroll
        for (int j = 0; j < 8; j++) {
          if (j < c.m) {
            float xr[32];
            load_x32(c.xs + j * xstride + 36 * b, xr);
            acc[j] = fmaf(s, dot32(qf, xr), acc[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (j < c.m) {
          const float v = half_wave_sum(acc[j]);
          if (k == 31 && r < c.r1) {
            if (c.y) c.y[(int64_t)j * c.p + r] = v;
            if (keys) best[j] = umax64(best[j], argmax_key(v, (uint32_t)r));
          }
        }
      }
    }
  }
}

// Any n and m: x read from global memory per block (it stays in the caches).
__device__ void rows_generic(const Tile &c, unsigned long long *best, bool keys) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const uint64_t pitch = (uint64_t)c.bpr * 34u;
  for (int32_t rb = c.r0 + 2 * wave; rb < c.r1; rb += kRowsPerPass) {
    const int32_t r = rb + half;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (r < c.r1) {
      for (int32_t b = k; b < c.bpr; b += 32) {
        const uint64_t a = (uint64_t)r * pitch + (uint64_t)b * 34u;
        uint32_t d[9];
        fetch_block(c.w, c.wbytes, a, d);
        const uint32_t amod = (uint32_t)a & 2u;
        const float s = scale_of(d, amod);
        float qf[32];
        block_quants(d, quant_sel(amod), qf);
        for (int j = 0; j < c.m; j++) {
          float xr[32];
          load_x32(c.xg + (int64_t)j * c.n + 32 * (int64_t)b, xr);
          acc[j] = fmaf(s, dot32(qf, xr), acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      if (j < c.m) {
        const float v = half_wave_sum(acc[j]);
        if (k == 31 && r < c.r1) {
          if (c.y) c.y[(int64_t)j * c.p + r] = v;
          if (keys) best[j] = umax64(best[j], argmax_key(v, (uint32_t)r));
        }
      }
    }
  }
}


// True when the last block of the matrix starts at a byte offset that is a
// multiple of 4 (p * bpr odd) and lies in this tile: its full window would
// read two bytes past the weights, so the tile takes rows_generic.
__device__ __forceinline__ bool needs_exact_tail(const Tile &c) {
  return c.r1 == c.p && (c.wbytes & 2);
}

// Direct path dispatch for one tile.
template <bool M1>
__device__ void run_direct(const Tile &c, int path, unsigned long long *best,
                           bool keys) {
  if (path == kGeneric || needs_exact_tail(c)) {
    rows_generic(c, best, keys);
    return;
  }
  const int nbl = nbl_of(c.n);
  if (M1) {
    if (nbl == 1) direct_m1<1, 4>(c, best[0], keys);
    else if (nbl == 2) direct_m1<2, 2>(c, best[0], keys);
    else direct_m1<3, 2>(c, best[0], keys);
  } else {
    if (nbl == 1) direct_mb<1, 2>(c, best, keys);
    else if (nbl == 2) direct_mb<2, 1>(c, best, keys);
    else direct_mb<3, 1>(c, best, keys);
  }
}

// ---- staged path ---------------------------------------------------------------

// Rows [0, rows) of a staged tile (LDS `tl`, row pitch 34 * bpr bytes), m = 1.
// Lane k of each half-wave reads the windows of blocks k, k+32, k+64 of its
// row from LDS, and the block's 32 x values from LDS.
template <int NBL>
__device__ __forceinline__ void staged_m1(const uint32_t *tl, int32_t bpr,
                                          int32_t rows, const float *xs,
                                          float *y, int32_t r0, bool keys,
                                          unsigned long long &best) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int32_t pitch = bpr * 34;
  for (int32_t rr0 = 2 * wave; rr0 < rows; rr0 += kRowsPerPass) {
    const int32_t rr = rr0 + half;
    const int32_t rc = rr < rows ? rr : rows - 1;
    float acc = 0.f;
    // keeps the x reads inside the loop (hoisted, they would pin 32 * NBL
    // registers for the whole tile)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int32_t b = min(k + 32 * i, bpr - 1);
      const int32_t o = rc * pitch + 34 * b;
      const uint32_t *wp = tl + (o >> 2);
      uint32_t d[9];
#pragma unroll
      for (int q = 0; q < 9; q++) d[q] = wp[q];
      const uint32_t amod = (uint32_t)o & 2u;
      float xb[32];
      load_x32(xs + 36 * b, xb);
      const float v = scale_of(d, amod) * block_dot(d, quant_sel(amod), xb);
      acc += (k + 32 * i < bpr) ? v : 0.f;
    }
    acc = half_wave_sum(acc);
    if (k == 31 && rr < rows) {
      if (y) gpw(y)[r0 + rr] = acc;
      if (keys) best = umax64(best, argmax_key(acc, (uint32_t)(r0 + rr)));
    }
  }
}

// Same for 1 < m <= 8: each block's quants convert once and serve m rows of
// x from LDS (row j at float offset j * 36 * bpr).
template <int NBL>
__device__ __forceinline__ void staged_mb(const uint32_t *tl, int32_t bpr,
                                          int32_t rows, int32_t m, int32_t p,
                                          const float *xs, float *y, int32_t r0,
                                          bool keys, unsigned long long *best) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int32_t pitch = bpr * 34;
  const int32_t xstride = 36 * bpr;
  for (int32_t rr0 = 2 * wave; rr0 < rows; rr0 += kRowsPerPass) {
    const int32_t rr = rr0 + half;
    const int32_t rc = rr < rows ? rr : rows - 1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int32_t b = min(k + 32 * i, bpr - 1);
      const int32_t o = rc * pitch + 34 * b;
      const uint32_t *wp = tl + (o >> 2);
      uint32_t d[9];
#pragma unroll
      for (int q = 0; q < 9; q++) d[q] = wp[q];
      const uint32_t amod = (uint32_t)o & 2u;
      const float s = (k + 32 * i < bpr) ? scale_of(d, amod) : 0.f;
      float qf[32];
      block_quants(d, quant_sel(amod), qf);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (j < m) {
          float xb[32];
          load_x32(xs + j * xstride + 36 * b, xb);
          acc[j] = fmaf(s, dot32(qf, xb), acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      if (j < m) {
        const float v = half_wave_sum(acc[j]);
        if (k == 31 && rr < rows) {
          if (y) gpw(y)[(int64_t)j * p + r0 + rr] = v;
          if (keys) best[j] = umax64(best[j], argmax_key(v, (uint32_t)(r0 + rr)));
        }
      }
    }
  }
}

// Registers that carry the next tile's weights (and x, when the next tile
// belongs to another matvec) while the current tile is computed.
template <int XC>
struct Prefetch {
  u32x4 w[kStageChunks];
  f32x4 x[XC];

  // `bytes` (a multiple of 16, >= 16) contiguous bytes at base (16-aligned).
  // Every chunk is loaded (offsets past the end repeat the last chunk), so
  // the loads are straight-line code the compiler can count.
  __device__ __forceinline__ void load_w(const uint8_t *base, int32_t bytes) {
    const __attribute__((address_space(1))) uint8_t *b = gp(base);
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      w[j] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4 *)(b + off));
    }
  }
  __device__ __forceinline__ void store_w(uint32_t *tl, int32_t bytes) const {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;  // repeats write equal data
      *(u32x4 *)((uint8_t *)tl + off) = w[j];
    }
  }
  // m rows of n floats (m * n <= 4 * XC * kWG), [m][n] contiguous.
  __device__ __forceinline__ void load_x(const float *src, int32_t floats) {
    const int32_t chunks = floats >> 2;
#pragma unroll
    for (int j = 0; j < XC; j++) {
      if (j * kWG < chunks) {
        int32_t c = j * kWG + (int32_t)threadIdx.x;
        c = c < chunks ? c : chunks - 1;
        x[j] = gp((const f32x4 *)src)[c];
      }
    }
  }
  // Into the padded LDS layout: row i, block b at i*36*bpr + 36*b.
  __device__ __forceinline__ void store_x(float *xs, int32_t m, int32_t n) const {
    const int32_t chunks = (m * n) >> 2, row_chunks = n >> 2;
    const int32_t bpr = n >> 5;
#pragma unroll
    for (int j = 0; j < XC; j++) {
      const int32_t c = j * kWG + (int32_t)threadIdx.x;
      if (c < chunks) {
        const int32_t i = c / row_chunks, e = (c - i * row_chunks) * 4;
        *(f32x4 *)&xs[i * 36 * bpr + 36 * (e >> 5) + (e & 31)] = x[j];
      }
    }
  }
};

// Where a launch's descriptors live: by value (one matvec) or in a
// device-side table (the step).  A workgroup of the step meets only a few
// matvecs, so the table is searched in memory.
struct OneSrc {
  StepDesc d;
  __device__ __forceinline__ int32_t find(int32_t, int32_t) const { return 0; }
  __device__ __forceinline__ StepDesc get(int32_t) const { return d; }
};

struct TableSrc {
  const StepDesc *tab;
  int32_t count;
  // Last descriptor at or after `lo` with tile_begin <= t.
  __device__ __forceinline__ int32_t find(int32_t t, int32_t lo) const {
    int32_t hi = count - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (tab[mid].tile_begin <= t) lo = mid;
      else hi = mid - 1;
    }
    return lo;
  }
  __device__ __forceinline__ StepDesc get(int32_t i) const { return tab[i]; }
};

__host__ __device__ inline int32_t tiles_of(const StepDesc &d) {
  return (d.p + d.rows_per_tile - 1) / d.rows_per_tile;
}

struct Job {
  int32_t desc;
  StepDesc d;
  int32_t path, r0, rows;
};

__device__ __forceinline__ Job job_at(int32_t desc, const StepDesc &d, int32_t t,
                                      int32_t m) {
  Job j;
  j.desc = desc;
  j.d = d;
  j.path = path_of(m, d.n);
  j.r0 = (t - d.tile_begin) * d.rows_per_tile;
  j.rows = min(d.rows_per_tile, d.p - j.r0);
  return j;
}

// Tiles first, first + stride, ... (< end) of the launch, in order.  Each
// tile's weights (and x, when the tile opens another matvec) are loaded into
// registers while the previous tile is computed.  Tiles of one matvec are
// contiguous, so a workgroup meets each matvec in one run of tiles; the run
// adds its argmax keys, if any, as one arrival.  LDS: the staged tile, then
// the padded x.
template <bool M1, bool ANY, class Src>
__device__ void run_tiles(const Src &src, int32_t first, int32_t end,
                          int32_t stride, int32_t d_hint, int32_t m,
                          float *tl_lds, float *xs) {
  constexpr int XC = M1 ? 3 : 8;  // float4 chunks of x per thread
  uint32_t *tl = (uint32_t *)tl_lds;
  int32_t t = first;
  if (t >= end) return;
  Prefetch<XC> pf;
  int32_t di = src.find(t, d_hint);
  Job cur = job_at(di, src.get(di), t, m);
  if (cur.path == kStaged)
    pf.load_w(cur.d.w + (uint64_t)cur.r0 * (cur.d.n >> 5) * 34u,
              cur.rows * (cur.d.n >> 5) * 34);
  if (cur.path != kGeneric) pf.load_x(cur.d.x, m * cur.d.n);
  int32_t xdesc = -1;
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
  for (;;) {
    const int32_t tn = t + stride;
    const bool more = tn < end;
    Job nxt = cur;
    if (more) {
      if (tn < cur.d.tile_begin + tiles_of(cur.d)) {
        nxt = job_at(cur.desc, cur.d, tn, m);
      } else {
        const int32_t dn = src.find(tn, cur.desc + 1);
        nxt = job_at(dn, src.get(dn), tn, m);
      }
    }
    const int32_t bpr = cur.d.n >> 5;
    const bool new_x = cur.path != kGeneric && cur.desc != xdesc;
    __syncthreads();  // the previous tile's readers of LDS are done
    if (cur.path == kStaged) pf.store_w(tl, cur.rows * bpr * 34);
    if (new_x) pf.store_x(xs, m, cur.d.n);
    __syncthreads();
    if (new_x) xdesc = cur.desc;
    if (more) {  // next tile's bytes go out before this tile is computed
      if (nxt.path == kStaged)
        pf.load_w(nxt.d.w + (uint64_t)nxt.r0 * (nxt.d.n >> 5) * 34u,
                  nxt.rows * (nxt.d.n >> 5) * 34);
      if (nxt.path != kGeneric && nxt.desc != cur.desc)
        pf.load_x(nxt.d.x, m * nxt.d.n);
    }
    const bool keys = cur.d.idx != nullptr;
    if (cur.path == kStaged) {
      const int nbl = nbl_of(cur.d.n);
      if (M1) {
        if (nbl == 1) staged_m1<1>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
        else if (nbl == 2) staged_m1<2>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
        else staged_m1<3>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
      } else {
        if (nbl == 1) staged_mb<1>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
        else if (nbl == 2) staged_mb<2>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
        else staged_mb<3>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
      }
    } else if (ANY) {
      Tile c;
      c.w = cur.d.w;
      c.bpr = bpr;
      c.wbytes = (uint64_t)cur.d.p * (uint64_t)bpr * 34u;
      c.xg = cur.d.x;
      c.xs = xs;
      c.y = cur.d.y;
      c.n = cur.d.n;
      c.p = cur.d.p;
      c.m = m;
      c.r0 = cur.r0;
      c.r1 = cur.r0 + cur.rows;
      run_direct<M1>(c, cur.path, best, keys);
    }
    if (keys && (!more || nxt.desc != cur.desc)) {
      argmax_finish(best, m, cur.d.slot, cur.d.idx, blockIdx.x, gridDim.x, tl_lds);
#pragma unroll
      for (int r = 0; r < 8; r++) best[r] = 0ull;
    }
    if (!more) break;
    t = tn;
    cur = nxt;
  }
}

// Two-deep variant of run_tiles: two register sets carry the weights of the
// next two tiles, so each workgroup keeps two tiles of HBM reads in flight
// while it computes a third from LDS (x stays one tile ahead).
struct WStage {
  u32x4 w[kStageChunks];
  __device__ __forceinline__ void load(const uint8_t *base, int32_t bytes) {
    const __attribute__((address_space(1))) uint8_t *b = gp(base);
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      w[j] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4 *)(b + off));
    }
  }
  __device__ __forceinline__ void store(uint32_t *tl, int32_t bytes) const {
#pragma unroll
    for (int j = 0; j < kStageChunks; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      *(u32x4 *)((uint8_t *)tl + off) = w[j];
    }
  }
};

__device__ __forceinline__ const uint8_t *tile_base(const Job &j) {
  return j.d.w + (uint64_t)j.r0 * (j.d.n >> 5) * 34u;
}
__device__ __forceinline__ int32_t tile_bytes(const Job &j) {
  return j.rows * (j.d.n >> 5) * 34;
}

template <class Src>
__device__ __forceinline__ Job next_job(const Src &src, const Job &cur, int32_t t,
                                        int32_t m) {
  if (t < cur.d.tile_begin + tiles_of(cur.d)) return job_at(cur.desc, cur.d, t, m);
  const int32_t dn = src.find(t, cur.desc + 1);
  return job_at(dn, src.get(dn), t, m);
}

template <bool M1, bool ANY, class Src, int XC>
__device__ __forceinline__ bool tile_step(const Src &src, WStage &wuse,
                                          Prefetch<XC> &xp, Job &cur, Job &nxt,
                                          int32_t &t, int32_t end, int32_t stride,
                                          int32_t m, int32_t &xdesc,
                                          unsigned long long *best, uint32_t *tl,
                                          float *xs) {
  const bool has_next = t + stride < end;
  const int32_t t2 = t + 2 * stride;
  const bool has2 = t2 < end;
  Job j2 = nxt;
  if (has2) j2 = next_job(src, nxt, t2, m);
  const int32_t bpr = cur.d.n >> 5;
  const bool new_x = cur.path != kGeneric && cur.desc != xdesc;
  __syncthreads();  // the previous tile's readers of LDS are done
  if (cur.path == kStaged) wuse.store(tl, tile_bytes(cur));
  if (new_x) xp.store_x(xs, m, cur.d.n);
  __syncthreads();
  if (new_x) xdesc = cur.desc;
  if (has2 && j2.path == kStaged) wuse.load(tile_base(j2), tile_bytes(j2));
  if (has_next && nxt.path != kGeneric && nxt.desc != cur.desc)
    xp.load_x(nxt.d.x, m * nxt.d.n);
  const bool keys = cur.d.idx != nullptr;
  if (cur.path == kStaged) {
    const int nbl = nbl_of(cur.d.n);
    if (M1) {
      if (nbl == 1) staged_m1<1>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
      else if (nbl == 2) staged_m1<2>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
      else staged_m1<3>(tl, bpr, cur.rows, xs, cur.d.y, cur.r0, keys, best[0]);
    } else {
      if (nbl == 1) staged_mb<1>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
      else if (nbl == 2) staged_mb<2>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
      else staged_mb<3>(tl, bpr, cur.rows, m, cur.d.p, xs, cur.d.y, cur.r0, keys, best);
    }
  } else if (ANY) {
    Tile c;
    c.w = cur.d.w;
    c.bpr = bpr;
    c.wbytes = (uint64_t)cur.d.p * (uint64_t)bpr * 34u;
    c.xg = cur.d.x;
    c.xs = xs;
    c.y = cur.d.y;
    c.n = cur.d.n;
    c.p = cur.d.p;
    c.m = m;
    c.r0 = cur.r0;
    c.r1 = cur.r0 + cur.rows;
    run_direct<M1>(c, cur.path, best, keys);
  }
  if (keys && (!has_next || nxt.desc != cur.desc)) {
    argmax_finish(best, m, cur.d.slot, cur.d.idx, blockIdx.x, gridDim.x, tl);
#pragma unroll
    for (int r = 0; r < 8; r++) best[r] = 0ull;
  }
  if (!has_next) return true;
  t += stride;
  cur = nxt;
  nxt = j2;
  return false;
}

template <bool M1, bool ANY, class Src>
__device__ void run_tiles2(const Src &src, int32_t first, int32_t end,
                           int32_t stride, int32_t d_hint, int32_t m,
                           float *tl_lds, float *xs) {
  constexpr int XC = M1 ? 3 : 8;
  uint32_t *tl = (uint32_t *)tl_lds;
  if (first >= end) return;
  WStage wa, wb;
  Prefetch<XC> xp;
  int32_t t = first;
  const int32_t d0 = src.find(t, d_hint);
  Job cur = job_at(d0, src.get(d0), t, m);
  Job nxt = cur;
  if (t + stride < end) nxt = next_job(src, cur, t + stride, m);
  if (cur.path == kStaged) wa.load(tile_base(cur), tile_bytes(cur));
  if (cur.path != kGeneric) xp.load_x(cur.d.x, m * cur.d.n);
  if (t + stride < end && nxt.path == kStaged) wb.load(tile_base(nxt), tile_bytes(nxt));
  int32_t xdesc = -1;
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
  for (;;) {
    if (tile_step<M1, ANY>(src, wa, xp, cur, nxt, t, end, stride, m, xdesc, best, tl, xs))
      break;
    if (tile_step<M1, ANY>(src, wb, xp, cur, nxt, t, end, stride, m, xdesc, best, tl, xs))
      break;
  }
}

#ifndef Q8_PREFETCH_DEPTH
#define Q8_PREFETCH_DEPTH 1
#endif
#if Q8_PREFETCH_DEPTH == 2
#define Q8_RUN_TILES run_tiles2
#else
#define Q8_RUN_TILES run_tiles
#endif

// ---- kernels -----------------------------------------------------------------

// One matvec (descriptor passed by value), its tiles round-robin over the
// grid (gridDim.x <= tiles, so every workgroup arrives at the argmax): at
// any moment the grid streams one contiguous window of the weights.
template <bool M1, bool ANY>
__global__ void __launch_bounds__(kWG, Q8_MIN_WGS_PER_CU)
mv_kernel(StepDesc d, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  OneSrc src{d};
  Q8_RUN_TILES<M1, ANY>(src, blockIdx.x, tiles_of(d), gridDim.x, 0, m, lds,
                        lds + kTileMaxBytes / 4);
}

// The decode step: every tile of every descriptor of a device-side table
// (count entries in tile order), with no ordering between descriptors.
// Workgroups form groups; a group interleaves its contiguous tile range.
template <bool M1, bool ANY>
__global__ void __launch_bounds__(kWG, Q8_MIN_WGS_PER_CU)
step_kernel(const StepDesc *__restrict__ table, int32_t count,
            const WgGroup *__restrict__ groups, int32_t group_size, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  TableSrc src{table, count};
  const WgGroup g = groups[blockIdx.x / group_size];
  const int32_t j = (int32_t)blockIdx.x - g.first;
  Q8_RUN_TILES<M1, ANY>(src, g.t0 + j, g.t1, g.size, 0, m, lds,
                        lds + kTileMaxBytes / 4);
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
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int i = 0; i < 8; i++)
    if (i == (int)blockIdx.y) best[i] = key;
  __shared__ unsigned long long red[kWaves * 8];
  argmax_finish(best, m, slot, idx, blockIdx.y * gridDim.x + blockIdx.x,
                gridDim.x * gridDim.y, red);
}

// ---- host side ---------------------------------------------------------------

// Dynamic LDS of a launch whose matvecs have widths up to n_max.
size_t lds_bytes_for(int m, int n) {
  // the x region starts after the tile region
  const size_t x = path_of(m, n) == kGeneric ? 0 : (size_t)x_lds_floats(m, n);
  return kTileMaxBytes + x * sizeof(float);
}

int device_cus(int dev) {
  static int cache[64] = {0};
  int &c = cache[dev & 63];
  if (!c) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || cus <= 0)
      cus = 256;
    c = cus;
  }
  return c;
}

template <typename K>
int resident_wgs(K kernel, size_t lds, int dev) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kWG, lds) !=
          hipSuccess || per_cu <= 0)
    per_cu = 1;
  return per_cu * device_cus(dev);
}

// Occupancy-limited grid of a single-matvec kernel variant, cached per
// device, for the largest LDS a launch of that variant can ask for.
template <bool M1, bool ANY>
int mv_grid_cap(int dev) {
  static int cache[64] = {0};
  int &c = cache[dev & 63];
  if (!c) {
    const size_t lds = kTileMaxBytes + (M1 ? (size_t)kMaxLdsBlocks * 36 * 4
                                           : (size_t)kXMaxFloats / 32 * 36 * 4);
    c = resident_wgs(mv_kernel<M1, ANY>, lds, dev);
  }
  return c;
}

template <bool M1, bool ANY>
hipError_t launch_mv(const StepDesc &d, int m, hipStream_t s) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int32_t ntiles = tiles_of(d);
  const int cap = mv_grid_cap<M1, ANY>(dev);
  const int grid = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL((mv_kernel<M1, ANY>), dim3(grid), dim3(kWG),
                     lds_bytes_for(m, d.n), s, d, m);
  return hipGetLastError();
}

}  // namespace

int step_rows_per_tile(int n, int m) { return tile_rows_of(m, n); }

size_t step_lds_bytes(int m, int n) { return lds_bytes_for(m, n); }

bool step_all_staged(int m, int n) { return path_of(m, n) == kStaged; }

int step_grid(int device, int m, size_t lds, bool all_staged) {
  if (m == 1)
    return all_staged ? resident_wgs(step_kernel<true, false>, lds, device)
                      : resident_wgs(step_kernel<true, true>, lds, device);
  return all_staged ? resident_wgs(step_kernel<false, false>, lds, device)
                    : resident_wgs(step_kernel<false, true>, lds, device);
}

hipError_t launch_matvec(const uint8_t *w, const float *x, float *y, int m,
                         int n, int p, ArgmaxSlot *slot, int32_t *idx,
                         hipStream_t s) {
  if (p <= 0) return hipSuccess;
  StepDesc d;
  d.w = w;
  d.x = x;
  d.y = y;
  d.idx = idx;
  d.slot = slot;
  d.n = n;
  d.p = p;
  d.tile_begin = 0;
  d.rows_per_tile = tile_rows_of(m, n);
  // small matvecs: shorter tiles spread them over more workgroups
  while (d.rows_per_tile > kRowsPerPass &&
         (p + d.rows_per_tile - 1) / d.rows_per_tile < 512)
    d.rows_per_tile >>= 1;
  const bool staged = path_of(m, n) == kStaged;
  if (m == 1)
    return staged ? launch_mv<true, false>(d, m, s) : launch_mv<true, true>(d, m, s);
  return staged ? launch_mv<false, false>(d, m, s) : launch_mv<false, true>(d, m, s);
}

hipError_t launch_step(const StepDesc *descs, int count, const WgGroup *groups,
                       int group_size, int m, int grid, size_t lds,
                       bool all_staged, hipStream_t s) {
  if (m == 1) {
    if (all_staged)
      hipLaunchKernelGGL((step_kernel<true, false>), dim3(grid), dim3(kWG), lds,
                         s, descs, count, groups, group_size, m);
    else
      hipLaunchKernelGGL((step_kernel<true, true>), dim3(grid), dim3(kWG), lds,
                         s, descs, count, groups, group_size, m);
  } else {
    if (all_staged)
      hipLaunchKernelGGL((step_kernel<false, false>), dim3(grid), dim3(kWG), lds,
                         s, descs, count, groups, group_size, m);
    else
      hipLaunchKernelGGL((step_kernel<false, true>), dim3(grid), dim3(kWG), lds,
                         s, descs, count, groups, group_size, m);
  }
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

}  // namespace q8
