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

#include "q8dec_decode_dev.h"
#include "q8dec_internal.h"

namespace q8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// Four floats read at device scope (another XCD may have written them in
// this launch; a plain load could return a stale L2 copy), and four stored
// at device scope.
__device__ __forceinline__ void st_dev4(float *p, const f32x4 &v) {
#pragma unroll
  for (int e = 0; e < 4; e++) dec::st_dev(p + e, v[e]);
}

// A matvec output.  dev: stored at device scope (written through to where
// every XCD sees it), so that a workgroup of the same launch can read it with
// device-scope loads and no L2 write-back (the epilogue, see arrive_last).
__device__ __forceinline__ void store_y(float *p, float v, bool dev = false) {
  if (dev) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else gpw(p)[0] = v;
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

// A 64-bit value of lane l (l uniform).
__device__ __forceinline__ unsigned long long readlane64(unsigned long long v, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((unsigned long long)hi << 32) | lo;
}

// Unsigned max over each 16-lane row, left in the row's last lane (lanes
// shifted in from outside the row read 0, the empty key).
__device__ __forceinline__ unsigned long long row16_max(unsigned long long v) {
  v = umax64(v, dpp64<0x111>(v));  // row_shr:1
  v = umax64(v, dpp64<0x112>(v));  // row_shr:2
  v = umax64(v, dpp64<0x114>(v));  // row_shr:4
  v = umax64(v, dpp64<0x118>(v));  // row_shr:8
  return v;
}

// Maximum over the wave.
__device__ __forceinline__ unsigned long long wave_max64(unsigned long long v) {
  v = row16_max(v);
  return umax64(umax64(readlane64(v, 15), readlane64(v, 31)),
                umax64(readlane64(v, 47), readlane64(v, 63)));
}

// Adds a workgroup's keys to the slot.  lk[w][r] (LDS) holds wave w's key of
// activation row r < m (0: none); every wave writes its entries before the
// call, which every thread makes.  Workgroup `wg` of a grid of `nwg` joins
// team wg % kArgmaxTeams: it raises the team keys with atomic max and then
// counts itself in.  The team's last arrival counts the team into the top
// group; the top group's last arrival takes (and clears) every team's keys
// and writes idx[0..m-1] (and the slot's host copy, if any).  Arrival
// counts come from the groups' `expected`
// fields, or, when those are 0, from "every workgroup arrives once".
// Atomics are relaxed: each counter increment is issued only after the
// updates before it have completed (performed at the memory side), which
// orders them without L2 write-back or invalidation.  Four dependent round
// trips separate the last arrival from the result.
template <int MR>
__device__ void argmax_arrive(const unsigned long long (*lk)[MR], int m,
                              ArgmaxSlot *__restrict__ slot,
                              int32_t *__restrict__ idx, uint32_t wg,
                              uint32_t nwg) {
  __syncthreads();  // lk is complete
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const uint32_t T = kArgmaxTeams;
  uint32_t last = 0;
  int32_t *host = nullptr;
  if (lane == 0) {
    host = gp(&slot->host)[0];  // read early: it is needed at the very end
    const uint32_t j = wg % T;
    ArgmaxGroup *g = &slot->team[j];
    uint32_t size = gp(&g->expected)[0], nteams = gp(&slot->top.expected)[0];
    if (size == 0u) {
      size = (nwg - j + T - 1) / T;
      nteams = nwg < T ? nwg : T;
    }
    // The m maxima go out together as global atomics that return nothing,
    // and one wait for all of them (vmcnt covers stores and atomics: they
    // are then performed at the memory side) orders them before the counter.
    // (Atomics that return the old value were turned by the compiler into
    // one read of each result right after its atomic: m round trips.)
#pragma unroll
    for (int r = 0; r < MR; r++) {
      if (r < m) {
        unsigned long long v = lk[0][r];
        for (int w = 1; w < kWaves; w++) v = umax64(v, lk[w][r]);
        __hip_atomic_fetch_max(gpw(&g->keys[r]), v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the maxima are performed
    const uint32_t prev = __hip_atomic_fetch_add(gpw(&g->counter), 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == size - 1u) {
      __hip_atomic_store(gpw(&g->counter), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t p2 = __hip_atomic_fetch_add(gpw(&slot->top.counter), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = p2 == nteams - 1u;
    }
  }
  if (!__builtin_amdgcn_readfirstlane(last)) return;
  // Every team is complete: lane j takes team j's keys in one round trip.
  unsigned long long v[MR];
#pragma unroll
  for (int r = 0; r < MR; r++) {
    v[r] = 0ull;
    if (r < m && lane < (int)T)
      v[r] = __hip_atomic_exchange(gpw(&slot->team[lane].keys[r]), 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  }
  // One wait for every exchange, every row's index, then all the stores
  // together, as global stores: a wait between them would also wait for the
  // stores before it, the host copy's round trip included.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int32_t res[MR];
#pragma unroll
  for (int r = 0; r < MR; r++) {
    res[r] = 0;
    if (r < m) res[r] = key_index(wave_max64(v[r]));
  }
#pragma unroll
  for (int r = 0; r < MR; r++) asm volatile("" ::"v"(res[r]));
  asm volatile("" ::: "memory");
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MR; r++) {
      if (r < m) {
        gpw(idx)[r] = res[r];
        if (host)
          __hip_atomic_store(gpw(&host[r]), res[r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    __hip_atomic_store(gpw(&slot->top.counter), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- matvec geometry ---------------------------------------------------------

// How the tiles of a matvec are processed.
//  kStaged : m = 1.  The tile's rows are streamed with coalesced, 16-byte
//            aligned loads (whole rows are contiguous) into registers one
//            tile ahead, written to LDS, and each lane reads its blocks'
//            windows from LDS.  Needs a row pitch that is a multiple of 16
//            (n/32 % 8 == 0).
//  kMfma   : 1 < m <= 8 and n in {1024, 2048, 3072}: same staging (rows
//            padded in LDS); the products run on the matrix cores (see
//            mfma_tile).
//  kDirect : each lane loads its blocks' windows straight from global
//            memory (dword aligned, 34-byte lane stride); any row pitch.
//  kGeneric: as kDirect, but x is read from global memory (large m * n).
//  kWide   : 8 < m <= 32, n a multiple of 256 (see wide_tiles).
enum Path : int { kStaged = 0, kDirect = 1, kGeneric = 2, kMfma = 3, kWide = 4 };

constexpr int kTileMaxBytes = 26112;  // 8 rows of 3072 columns
constexpr int kStageChunks = (kTileMaxBytes + 16 * kWG - 1) / (16 * kWG);
constexpr int kXMaxFloats = 8192;     // m * n of x kept in LDS (32 KB)
constexpr int kMaxLdsBlocks = 96;     // n <= 3072 for the LDS paths

// Batched tiles: 16-row groups; each staged row is followed by kMfmaRowPad
// bytes of LDS so that the 16 rows of a group start in different banks.
constexpr int kMfmaRowPad = 16;
constexpr int kMfmaTileBytes = 53248;  // LDS of a batched tile, pads included
constexpr int kMfmaChunks = (kMfmaTileBytes + 16 * kWG - 1) / (16 * kWG);
constexpr int kMfmaMaxBlocks = kMaxLdsBlocks / kWaves;  // x blocks per wave
constexpr int kMaxM = 8;  // activation rows of the m <= 8 paths (wider: kWide)
constexpr int kI8xMaxBlocks = kMaxM * kMaxLdsBlocks;  // int8-activation steps
constexpr int kRedStride = 80;  // floats between a wave's partial-sum entries
// One set of the waves' partial sums of a 16-row group.  An odd group puts
// its set into the tile rows of the group before it instead (every wave has
// read them before that group's barrier), so consecutive groups still write
// different LDS and need no barrier between one's reads and the next's
// writes, and the tile's own barrier orders the last group's reads before
// the next tile is stored.
constexpr int kRedFloats = kWaves * 4 * kRedStride;

__host__ __device__ inline int path_of(int m, int n) {
  const int bpr = n >> 5;
  if (m > kMaxM) return kWide;  // callers ensure n % 256 == 0 (wide_shape_ok)
  if (bpr == 0 || bpr > kMaxLdsBlocks) return kGeneric;
  if (m == 1) return bpr % 8 == 0 ? kStaged : kDirect;
  if (bpr == 32 || bpr == 64 || bpr == 96) return kMfma;
  return m * n > kXMaxFloats ? kGeneric : kDirect;
}

__host__ __device__ inline int nbl_of(int n) { return ((n >> 5) + 31) >> 5; }
// matrix-core tiles are at least 32 blocks wide: 16 rows hold a set of partials
static_assert(16 * ((32 * 34 + kMfmaRowPad) / 4) >= kRedFloats, "partials fit a row group");

// Rows per tile: staged tiles fill up to kTileMaxBytes (at least one pass of
// 8 rows), batched tiles up to kMfmaTileBytes in 16-row groups; direct and
// generic tiles are two or four passes.
__host__ __device__ inline int tile_rows_of(int m, int n) {
  const int path = path_of(m, n);
  if (path == kWide) return 128;  // kWideRows
  if (path == kStaged) {
    const int r = kTileMaxBytes / ((n >> 5) * 34);
    return r >= 64 ? 64 : (r < 1 ? 1 : r);
  }
  if (path == kMfma) {
    const int g = kMfmaTileBytes / (16 * ((n >> 5) * 34 + kMfmaRowPad));
    return 16 * (g < 1 ? 1 : g);
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
  bool devy;        // y takes device-scope stores
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
        if (c.y) store_y(&c.y[r], acc, c.devy);
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
            if (c.y) store_y(&c.y[(int64_t)j * c.p + r], v, c.devy);
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
          if (c.y) store_y(&c.y[(int64_t)j * c.p + r], v, c.devy);
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
template <int NBL, bool DEVY>
__device__ __forceinline__ void staged_m1(const uint32_t *tl, int32_t bpr,
                                          int32_t rows, const float *xs,
                                          float *y, int32_t r0, bool keys,
                                          unsigned long long &best,
                                          float *stash = nullptr) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int32_t pitch = bpr * 34;
  // A staged row pitch is a multiple of 16, so a block's byte offset mod 4
  // follows from its index alone: 2 for odd blocks, 0 for even ones (and
  // k + 32 i has the parity of k).
  const uint32_t amod = (uint32_t)(k & 1) << 1;
  const uint32_t sel = quant_sel(amod);
  // With one block per lane (n <= 1024) the lane's 32 x values are the same
  // for every row: they are read from LDS once per tile.
  float xk[32];
  if (NBL == 1) load_x32(xs + 36 * min(k, bpr - 1), xk);
  // The row-owning lane's best row of the tile for the argmax: the first
  // value that is not NaN, then only strictly larger ones.  Its rows ascend,
  // so among equal values (-0 and +0 included) the lowest row stays, as the
  // keys order them; the key is formed once per tile.
  float bv = __builtin_nanf("");
  int32_t br = 0;
  for (int32_t rr0 = 2 * wave; rr0 < rows; rr0 += kRowsPerPass) {
    // rr may be `rows` (odd row count): that window lies in the x region of
    // LDS, and its sum is dropped
    const int32_t rr = rr0 + half;
    float acc = 0.f;
    // keeps the x reads inside the loop (hoisted, they would pin 32 * NBL
    // registers for the whole tile)
    if (NBL > 1) asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int32_t b = min(k + 32 * i, bpr - 1);
      const uint32_t *wp = tl + ((rr * pitch + 34 * b) >> 2);
      uint32_t d[9];
#pragma unroll
      for (int q = 0; q < 9; q++) d[q] = wp[q];
      float xb[32];
      if (NBL == 1) {
#pragma unroll
        for (int t = 0; t < 32; t++) xb[t] = xk[t];
      } else {
        load_x32(xs + 36 * b, xb);
      }
      const float v = scale_of(d, amod) * block_dot(d, sel, xb);
      acc += (k + 32 * i < bpr) ? v : 0.f;
    }
    acc = half_wave_sum(acc);
    const bool mine = k == 31 && rr < rows;
    if (mine && y) store_y(&y[r0 + rr], acc, DEVY);
    if (mine && stash) stash[rr] = acc;  // a paired tile's sums (LDS)
    const bool better = mine & ((acc > bv) | ((bv != bv) & (acc == acc)));  // no branches
    bv = better ? acc : bv;
    br = better ? rr : br;
  }
  if (keys && bv == bv) best = umax64(best, argmax_key(bv, (uint32_t)(r0 + br)));
}

// ---- int8-activation variant -----------------------------------------------
//
// The CPU's sdot kernel quantises the activations and multiplies integers
// (inferno.rs "IV.4: One command buffer per token", the prose after the
// q8_matvec listing in "Eight kernels", and "The correctness ladder").  Here
// x is quantised per 32-value block by the Q8_0 rule, in binary32: amax =
// max |x_j|, d = amax / 127, q_j = x_j * (1/d) rounded to nearest even; a
// block holding a NaN or an infinity gets d = NaN and zero codes.  Each
// block's product is then an exact integer sum of eight v_dot4_i32_i8, and
// only scale * d * sum is floating point.

// Codes of four consecutive x values (packed int8, lowest byte first) and
// the block's step d.  The 32 values of a block sit in 8 consecutive lanes
// (aligned to 8), which exchange their maxima with DPP.
__device__ __forceinline__ float q8x_chunk(const f32x4 v, uint32_t &codes) {
  float a = 0.f;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const float t = fabsf(v[k]);
    bad = bad || !(t <= 3.402823466e38f);  // NaN or infinity
    a = fmaxf(a, t);
  }
  float e = bad ? __builtin_inff() : a;
  e = fmaxf(e, dpp_shift<0xB1, 0xF>(e));   // quad_perm [1,0,3,2]
  e = fmaxf(e, dpp_shift<0x4E, 0xF>(e));   // quad_perm [2,3,0,1]
  e = fmaxf(e, dpp_shift<0x141, 0xF>(e));  // row_half_mirror: 8 lanes
  const bool block_bad = e == __builtin_inff();
  const float d = block_bad ? __builtin_nanf("") : e / 127.0f;
  const float inv = (block_bad || d == 0.f) ? 0.f : 1.0f / d;
  codes = 0u;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const int32_t q = block_bad ? 0 : (int32_t)rintf(v[k] * inv);
    codes |= ((uint32_t)q & 0xFFu) << (8 * k);
  }
  return d;
}

// m rows of x ([m][n] f32 in global memory) quantised into LDS: xq (packed
// codes, row i block b at dword 8 (i * n/32 + b)) and xd (the steps, block
// i * n/32 + b, or with BM block-major: b * kMaxM + i).  Loaded directly
// (the batched form, once per matvec).
// With BM, x's rows may lie xstride floats apart (a column slice of a wider
// x, whose blocks quantise as they do in the whole row).
// PADS (BM only): block b's steps at (b / 2) * kRedStride + 8 (b % 2) + i,
// the unused tail of a set of partial sums' entries (16 blocks of steps
// where a set has 16 entries, offset by 64 floats).
template <int NT, bool BM = false, bool PADS = false>
__device__ void quantize_x_lds(const float *x, int32_t m, int32_t n,
                               uint32_t *xq, float *xd, int32_t xstride = 0) {
  const int32_t chunks = (m * n) >> 2;  // a multiple of 8: no block is split
  const int32_t bpr = n >> 5;
  for (int32_t c0 = 0; c0 < chunks; c0 += NT) {
    const int32_t c = c0 + (int32_t)threadIdx.x;
    const int32_t cc = c < chunks ? c : chunks - 1;
    int32_t at = cc;  // the chunk's f32x4 index in x
    if (BM) {
      const int32_t r = cc / (n >> 2);
      at = (r * xstride >> 2) + (cc - r * (n >> 2));
    }
    const f32x4 v = gp((const f32x4 *)x)[at];
    uint32_t codes;
    const float d = q8x_chunk(v, codes);
    if (c < chunks) {
      xq[c] = codes;
      if ((c & 7) == 0) {
        const int32_t k = c >> 3, i = BM ? k / bpr : 0;
        const int32_t b = k - i * bpr;
        xd[!BM ? k : (PADS ? (b >> 1) * kRedStride + 8 * (b & 1) + i : b * kMaxM + i)] = d;
      }
    }
  }
}

// Rows [0, rows) of a staged tile against int8 activations, m = 1: as
// staged_m1, with the block product an integer dot.
template <int NBL>
__device__ __forceinline__ void staged_m1_i8(const uint32_t *tl, int32_t bpr,
                                             int32_t rows, const uint32_t *xq,
                                             const float *xd, float *y, int32_t r0,
                                             bool keys, unsigned long long &best) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int32_t pitch = bpr * 34;
  for (int32_t rr0 = 2 * wave; rr0 < rows; rr0 += kRowsPerPass) {
    const int32_t rr = rr0 + half;
    const int32_t rc = rr < rows ? rr : rows - 1;
    float acc = 0.f;
    // keeps each pass's LDS reads inside the pass (four workgroups per CU
    // need the kernel within 128 registers)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int32_t b = min(k + 32 * i, bpr - 1);
      const int32_t o = rc * pitch + 34 * b;
      const uint32_t *wp = tl + (o >> 2);
      uint32_t d[9];
#pragma unroll
      for (int q = 0; q < 9; q++) d[q] = wp[q];
      const uint32_t amod = (uint32_t)o & 2u, sel = quant_sel(amod);
      const uint32_t *xc = xq + 8 * b;
      int32_t isum = 0;
#pragma unroll
      for (int t = 0; t < 8; t++)
        isum = __builtin_amdgcn_sdot4((int)__builtin_amdgcn_perm(d[t + 1], d[t], sel),
                                      (int)xc[t], isum, false);
      const float v = (float)isum * (scale_of(d, amod) * xd[b]);
      acc += (k + 32 * i < bpr) ? v : 0.f;
    }
    acc = half_wave_sum(acc);
    if (k == 31 && rr < rows) {
      if (y) store_y(&y[r0 + rr], acc);
      if (keys) best = umax64(best, argmax_key(acc, (uint32_t)(r0 + rr)));
    }
  }
}

// Same for 1 < m <= 8: each block's quant dwords are realigned once and
// dotted with m rows of codes.
template <int NBL>
__device__ __forceinline__ void staged_mb_i8(const uint32_t *tl, int32_t bpr,
                                             int32_t rows, int32_t m, int32_t p,
                                             const uint32_t *xq, const float *xd,
                                             float *y, int32_t r0, bool keys,
                                             unsigned long long *best) {
  const int lane = threadIdx.x & 63, k = lane & 31, half = lane >> 5;
  const int wave = threadIdx.x >> 6;
  const int32_t pitch = bpr * 34;
  for (int32_t rr0 = 2 * wave; rr0 < rows; rr0 += kRowsPerPass) {
    const int32_t rr = rr0 + half;
    const int32_t rc = rr < rows ? rr : rows - 1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NBL; i++) {
      const int32_t b = min(k + 32 * i, bpr - 1);
      const int32_t o = rc * pitch + 34 * b;
      const uint32_t *wp = tl + (o >> 2);
      uint32_t d[9];
#pragma unroll
      for (int q = 0; q < 9; q++) d[q] = wp[q];
      const uint32_t amod = (uint32_t)o & 2u, sel = quant_sel(amod);
      uint32_t qw[8];
#pragma unroll
      for (int t = 0; t < 8; t++) qw[t] = __builtin_amdgcn_perm(d[t + 1], d[t], sel);
      const bool live = k + 32 * i < bpr;
      const float s = scale_of(d, amod);
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (j < m) {
          const uint32_t *xc = xq + 8 * (j * bpr + b);
          int32_t isum = 0;
#pragma unroll
          for (int t = 0; t < 8; t++)
            isum = __builtin_amdgcn_sdot4((int)qw[t], (int)xc[t], isum, false);
          const float v = fmaf((float)isum, s * xd[j * bpr + b], acc[j]);
          acc[j] = live ? v : acc[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
      if (j < m) {
        const float v = half_wave_sum(acc[j]);
        if (k == 31 && rr < rows) {
          if (y) store_y(&y[(int64_t)j * p + r0 + rr], v);
          if (keys) best[j] = umax64(best[j], argmax_key(v, (uint32_t)(r0 + rr)));
        }
      }
    }
  }
}

// ---- batched path: matrix cores -----------------------------------------------
//
// For 1 < m <= 8 a 16-row group of a staged tile against one block is one
// v_mfma_f32_16x16x32_bf16, with k running over the block's 32 quants:
//  * operand A is x: column i < 8 holds x row i rounded to bf16 ("hi"),
//    column i + 8 the bf16 of what that rounding left ("lo"), so hi + lo
//    carries x to about 2^-17 relative; rows i >= m are zero;
//  * operand B holds the 16 weight rows' quants as bf16 (exact for int8);
//  * D[i][j] = sum over the block of x_i * q_j exactly rounded products,
//    accumulated in f32; the block's scale for row j multiplies it once
//    (the dequantise-in-the-dot order of the q8_matvec listing in inferno.rs
//    "IV.4: One command buffer per token", section "Eight kernels") and the
//    result adds into an f32 accumulator.
// Lane l of a wave holds A[l % 16][8 (l / 16) .. + 7], B[8 (l / 16) .. + 7]
// [l % 16] and D[4 (l / 16) + r][l % 16] for r < 4, so each lane scales its
// four D values by the scale of weight row l % 16.  The four waves of a
// workgroup split each row's blocks into four contiguous slices and keep their
// slice of x in registers for the whole matvec; their 16 x 16 partials meet
// in LDS, where y[i][row] = sum over waves of column i plus column i + 8.

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// A 16-row group's outputs of the int8 matrix-core tile from the four waves'
// partials acc, through LDS as mfma_tile's (there y[xr][row] also adds the
// column xr + 8 of x's low parts, which the int8 form does not have).
__device__ __forceinline__ void mfma_group_out(const f32x4 &acc, float *rb,
                                               int32_t rg, int32_t rows, int32_t m,
                                               int32_t p, float *y, int32_t r0, bool keys,
                                               unsigned long long &kb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int r = 0; r < 4; r++) rb[(wave * 4 + r) * kRedStride + lane] = acc[r];
  __syncthreads();
  if (threadIdx.x < 128) {
    const int xr = threadIdx.x >> 4, jj = threadIdx.x & 15;
    const int hi = (xr & 3) * kRedStride + 16 * (xr >> 2) + jj;  // column xr
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) v += rb[w * 4 * kRedStride + hi];
    const int32_t rr = rg + jj;
    if (xr < m && rr < rows) {
      if (y) store_y(&y[(int64_t)xr * p + r0 + rr], v);
      if (keys) kb = umax64(kb, argmax_key(v, (uint32_t)(r0 + rr)));
    }
  }
}

// Two int8 quants (bytes lo, lo + 1 of q) as a pair of bf16 (exact): the f32
// of a small integer has zero low halves, so the high halves are the bf16.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t q, int lo) {
  const float f0 = (float)(int8_t)(q >> (8 * lo));
  const float f1 = (float)(int8_t)(q >> (8 * lo + 8));
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, f1),
                               __builtin_bit_cast(uint32_t, f0), 0x07060302u);
}

__device__ __forceinline__ bf16x8 quants_bf16(uint32_t qa, uint32_t qb) {
  u32x4 r;
  r.x = bf16_pair(qa, 0);
  r.y = bf16_pair(qa, 2);
  r.z = bf16_pair(qb, 0);
  r.w = bf16_pair(qb, 2);
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// This lane's operand A for the blocks of its wave's slice of one matvec:
// x row (lane % 16) & 7, hi or lo part, elements 8 (lane / 16) .. + 7 of each
// block; NBW = n / 128 blocks per wave.  Lanes i and i + 8 of a 16-lane row
// need the same eight floats: each loads four and a DPP rotation by 8 within
// the row swaps the halves.  xstride: floats from one x row to the next (n,
// or the whole matrix's width for a column slice).
template <int NBW, int MB>
__device__ __forceinline__ void load_xa(u32x4 (&xa)[MB],
                                        const float *x, int32_t m, int32_t xstride) {
  static_assert(NBW <= MB, "the slice fits the registers");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, xr = i & 7, g = lane >> 4;
  const bool lo = i >= 8, live = xr < m;
  const __attribute__((address_space(1))) f32x4 *src =
      (const __attribute__((address_space(1))) f32x4 *)gp(
          x + (int64_t)(live ? xr : 0) * xstride + 32 * wave * NBW + 8 * g + 4 * lo);
  f32x4 v[NBW];
#pragma unroll
  for (int t = 0; t < NBW; t++) v[t] = src[8 * t];
#pragma unroll
  for (int t = 0; t < NBW; t++) {
    f32x4 w;
#pragma unroll
    for (int c = 0; c < 4; c++) w[c] = dpp_shift<0x128, 0xF>(v[t][c]);  // row_ror:8
    float e[8];
#pragma unroll
    for (int c = 0; c < 4; c++) {
      e[c] = lo ? w[c] : v[t][c];
      e[c + 4] = lo ? v[t][c] : w[c];
    }
    uint32_t h[8];
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const float hi = (float)(__bf16)e[c];
      h[c] = lo ? bf16_bits(e[c] - hi) : bf16_bits(e[c]);
    }
    u32x4 r;
    r.x = h[0] | (h[1] << 16);
    r.y = h[2] | (h[3] << 16);
    r.z = h[4] | (h[5] << 16);
    r.w = h[6] | (h[7] << 16);
    xa[t] = live ? r : u32x4{0u, 0u, 0u, 0u};
  }
}

// Rows [0, rows) of a batched tile in LDS (row pitch 34 * bpr + kMfmaRowPad
// bytes, bpr = 4 * NBW): y[i][r0 + row] for i < m.  `red` is kRedFloats of LDS.  Keys of
// x row threadIdx.x / 16 (threads below 128) go to `kb`.
template <int NBW, int MB>
__device__ __forceinline__ void mfma_tile(const uint32_t *tl, int32_t bpr,
                                          int32_t rows, int32_t m, int32_t p,
                                          const u32x4 (&xa)[MB],
                                          float *red, float *y, int32_t r0,
                                          bool keys, unsigned long long &kb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int32_t lpd = (bpr * 34 + kMfmaRowPad) >> 2;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  int buf = 0;
  for (int32_t rg = 0; rg < rows; rg += 16) {
    const int32_t row = min(rg + j, rows - 1);
    // the slice starts at an even block, so at a dword boundary
    const uint32_t *rp = tl + row * lpd + ((34 * wave * NBW) >> 2);
    f32x4 acc = zero;
#pragma unroll
    for (int t = 0; t < NBW; t += 2) {
      {
        // blocks t (byte 0 of wp, quants from byte 2) and t + 1 (byte 34,
        // quants from byte 36) of the slice
        const uint32_t *wp = rp + 17 * (t >> 1);
        const uint32_t *wq = wp + 2 * g;
        const uint32_t e0 = wq[0], e1 = wq[1], e2 = wq[2];
        const uint32_t o0 = wq[9], o1 = wq[10];
        const uint32_t s01 = wp[0], s23 = wp[8];
        const bf16x8 qe = quants_bf16(__builtin_amdgcn_perm(e1, e0, 0x05040302u),
                                      __builtin_amdgcn_perm(e2, e1, 0x05040302u));
        const bf16x8 qo = quants_bf16(o0, o1);
        const f32x4 de = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, xa[t]), qe, zero, 0, 0, 0);
        const f32x4 dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, xa[t + 1]), qo, zero, 0, 0, 0);
        const float se = (float)__builtin_bit_cast(_Float16, (uint16_t)(s01 & 0xFFFFu));
        const float so = (float)__builtin_bit_cast(_Float16, (uint16_t)(s23 >> 16));
#pragma unroll
        for (int r = 0; r < 4; r++) {
          acc[r] = fmaf(se, de[r], acc[r]);
          acc[r] = fmaf(so, dd[r], acc[r]);
        }
      }
    }
    // partials: entry r of lane l at kRedStride * r + l, so a wave's
    // writes (fixed r) and its reads below (four r, sixteen lanes each)
    // both fall in 64 different banks; column i of row jj is entry i % 4
    // of lane 16 (i / 4) + jj
    float *rb = buf ? (float *)(tl + (rg - 16) * lpd) : red;
#pragma unroll
    for (int r = 0; r < 4; r++) rb[(wave * 4 + r) * kRedStride + lane] = acc[r];
    __syncthreads();
    if (threadIdx.x < 128) {
      const int xr = threadIdx.x >> 4, jj = threadIdx.x & 15;
      const int hi = (xr & 3) * kRedStride + 16 * (xr >> 2) + jj;  // column xr
      const int lo = hi + 32;                                      // column xr + 8
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; w++)
        v += rb[w * 4 * kRedStride + hi] + rb[w * 4 * kRedStride + lo];
      const int32_t rr = rg + jj;
      if (xr < m && rr < rows) {
        if (y) store_y(&y[(int64_t)xr * p + r0 + rr], v);
        if (keys) kb = umax64(kb, argmax_key(v, (uint32_t)(r0 + rr)));
      }
    }
    // the next group's set is elsewhere (kRedFloats); the barrier after its
    // writes orders this group's reads before the one after reuses this set
    buf ^= 1;
  }
}

// Rows [0, rows) of a batched tile against int8 activations (1 < m <= 8,
// n = 32 NBW * kWaves): a 16-row group against one block is one
// v_mfma_i32_16x16x32_i8, operand A the x rows' codes (rows >= m zero),
// operand B the 16 weight rows' quants as they are stored (no conversion),
// D[i][j] the exact integer block sum of x row i and weight row j.  Each
// block's sum is then scaled as the VALU form scales it, by the weight
// row's scale times x row i's step (xd, block-major: xd[b * kMaxM + i]),
// and added to the f32 accumulator of its x row; the waves' partials meet
// in LDS as mfma_tile's do.  The lane layout is mfma_tile's (operands of
// 8 bytes instead of 8 bf16).
template <int NBW, int MB, bool PADS = false>
__device__ __forceinline__ void mfma_tile_i8(const uint32_t *tl, int32_t bpr,
                                             int32_t rows, int32_t m, int32_t p,
                                             const u32x2 (&xi)[MB], const float *xd,
                                             float *red, float *y, int32_t r0,
                                             bool keys, unsigned long long &kb) {
  static_assert(NBW <= MB && NBW % 2 == 0, "a wave's blocks: pairs within its registers");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int32_t lpd = (bpr * 34 + kMfmaRowPad) >> 2;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const i32x4 izero = {0, 0, 0, 0};
  // steps of x rows 4 g .. 4 g + 3 (rows 8 .. 15, which A holds as zeros,
  // read rows 0 .. 7's: their sums are 0 and never leave the tile)
  // (PADS: the steps as quantize_x_lds places them in the partials' padding)
  const float *xdw =
      xd + (PADS ? ((wave * NBW) >> 1) * kRedStride : (wave * NBW) * kMaxM) + 4 * (g & 1);
  int buf = 0;
  for (int32_t rg = 0; rg < rows; rg += 16) {
    const int32_t row = min(rg + j, rows - 1);
    const uint32_t *rp = tl + row * lpd + ((34 * wave * NBW) >> 2);
    f32x4 acc = zero;
#pragma unroll
    for (int t = 0; t < NBW; t += 2) {
      // blocks t (quants from byte 2 of wp) and t + 1 (from byte 36)
      const uint32_t *wp = rp + 17 * (t >> 1);
      const uint32_t *wq = wp + 2 * g;
      const uint32_t e0 = wq[0], e1 = wq[1], e2 = wq[2];
      const uint32_t o0 = wq[9], o1 = wq[10];
      const uint32_t s01 = wp[0], s23 = wp[8];
      const int64_t qe = (int64_t)(((uint64_t)__builtin_amdgcn_perm(e2, e1, 0x05040302u) << 32) |
                                   __builtin_amdgcn_perm(e1, e0, 0x05040302u));
      const int64_t qo = (int64_t)(((uint64_t)o1 << 32) | o0);
      const i32x4 de = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          (int64_t)__builtin_bit_cast(uint64_t, xi[t]), qe, izero, 0, 0, 0);
      const i32x4 dd = __builtin_amdgcn_mfma_i32_16x16x32_i8(
          (int64_t)__builtin_bit_cast(uint64_t, xi[t + 1]), qo, izero, 0, 0, 0);
      const float se = (float)__builtin_bit_cast(_Float16, (uint16_t)(s01 & 0xFFFFu));
      const float so = (float)__builtin_bit_cast(_Float16, (uint16_t)(s23 >> 16));
      const float *xdt = xdw + (PADS ? (t >> 1) * kRedStride : t * kMaxM);
      const f32x4 xe = *(const f32x4 *)xdt;
      const f32x4 xo = *(const f32x4 *)(xdt + (PADS ? 8 : kMaxM));
#pragma unroll
      for (int r = 0; r < 4; r++) {
        acc[r] = fmaf((float)de[r], se * xe[r], acc[r]);
        acc[r] = fmaf((float)dd[r], so * xo[r], acc[r]);
      }
    }
    mfma_group_out(acc, buf ? (float *)(tl + (rg - 16) * lpd) : red, rg, rows, m, p, y, r0,
                   keys, kb);
    buf ^= 1;
  }
}

// Each wave's operand A of the int8 tile: lane l takes x row l % 16 (zero
// from row m on), block wave * NBW + t, codes 8 (l / 16) .. + 7, from the
// codes quantize_x_lds left in LDS (row i block b at dword 8 (i bpr + b)).
template <int NBW, int MB>
__device__ __forceinline__ void load_xi(u32x2 (&xi)[MB], const uint32_t *xq, int32_t m,
                                        int32_t bpr) {
  static_assert(NBW <= MB, "a wave's blocks fit its registers");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const u32x2 z = {0u, 0u};
#pragma unroll
  for (int t = 0; t < NBW; t++)
    xi[t] = i < m ? *(const u32x2 *)(xq + 8 * (i * bpr + wave * NBW + t) + 2 * g) : z;
}

// Registers that carry the next tile's weights (and x, when the next tile
// belongs to another matvec) while the current tile is computed.  The
// weights are spread over the first NL threads (load_w, store_w; the other
// loaders use all kWG).
template <int XC, int CH, int NL = kWG>
struct Prefetch {
  static_assert(NL % 64 == 0 && NL <= kWG, "whole waves load");
  u32x4 w[CH];
  f32x4 x[XC];

  // `bytes` (a multiple of 16, >= 16) contiguous bytes at base (16-aligned).
  // Every chunk is loaded (offsets past the end repeat the last chunk), so
  // the loads are straight-line code the compiler can count.
  __device__ __forceinline__ void load_w(const uint8_t *base, int32_t bytes) {
    if (NL < kWG && (int)threadIdx.x >= NL) return;  // wave-uniform
    const __attribute__((address_space(1))) uint8_t *b = gp(base);
#pragma unroll
    for (int j = 0; j < CH; j++) {
      int32_t off = (j * NL + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      w[j] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4 *)(b + off));
    }
  }
  // `bytes` bytes at a then `bytes` bytes at b (a paired tile: the same
  // rows of two matrices), packed as load_w packs 2 * bytes contiguous ones.
  __device__ __forceinline__ void load_w_pair(const uint8_t *a, const uint8_t *b,
                                              int32_t bytes) {
    if (NL < kWG && (int)threadIdx.x >= NL) return;
    const __attribute__((address_space(1))) uint8_t *pa = gp(a), *pb = gp(b);
#pragma unroll
    for (int j = 0; j < CH; j++) {
      int32_t off = (j * NL + (int32_t)threadIdx.x) * 16;
      off = off < 2 * bytes - 16 ? off : 2 * bytes - 16;
      const __attribute__((address_space(1))) uint8_t *src =
          off < bytes ? pa + off : pb + (off - bytes);
      w[j] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)src);
    }
  }
  __device__ __forceinline__ void store_w(uint32_t *tl, int32_t bytes) const {
    if (NL < kWG && (int)threadIdx.x >= NL) return;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      int32_t off = (j * NL + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;  // repeats write equal data
      *(u32x4 *)((uint8_t *)tl + off) = w[j];
    }
  }
  // `bytes` bytes of whole rows of `rb` bytes each (a multiple of 16) that
  // lie `pitch` bytes apart in memory (a column slice of a wider matrix),
  // packed in the registers as load_w packs contiguous rows.
  __device__ __forceinline__ void load_w_strided(const uint8_t *base, int32_t bytes,
                                                 int32_t rb, int32_t pitch) {  // NL = kWG only
    const __attribute__((address_space(1))) uint8_t *b = gp(base);
    const int32_t cpr = rb >> 4;  // chunks per row
    // chunk c of row c / cpr: c < 2^12 and c / cpr is at least 1 / (2 cpr)
    // from an integer, far above the rounding of the product
    const float rcp = 1.0f / (float)cpr;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      const int32_t c = off >> 4;
      const int32_t row = (int32_t)(((float)c + 0.5f) * rcp);
      w[j] = __builtin_nontemporal_load(
          (const __attribute__((address_space(1))) u32x4 *)(b + (int64_t)row * pitch +
                                                            16 * (c - row * cpr)));
    }
  }
  // Same, with kMfmaRowPad bytes after every row of `pitch` bytes (a
  // multiple of 16, so no chunk straddles two rows).
  __device__ __forceinline__ void store_w_rows(uint32_t *tl, int32_t bytes,
                                               int32_t pitch) const {  // NL = kWG only
    const int32_t cpr = pitch >> 4;  // chunks per row
    // chunk c of row c / cpr: c < 2^12 and c / cpr is at least 1 / (2 cpr)
    // from an integer, far above the rounding of the product
    const float rcp = 1.0f / (float)cpr;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      int32_t off = (j * kWG + (int32_t)threadIdx.x) * 16;
      off = off < bytes - 16 ? off : bytes - 16;
      const int32_t row = (int32_t)(((float)(off >> 4) + 0.5f) * rcp);
      *(u32x4 *)((uint8_t *)tl + off + row * kMfmaRowPad) = w[j];
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
  // Quantised into LDS (int8-activation variant): packed codes xq and steps
  // xd, laid out as quantize_x_lds does.  Chunks of one block sit in 8
  // consecutive lanes, and chunk counts are multiples of 8, so every lane
  // of a block takes part in its DPP maximum.
  __device__ __forceinline__ void store_xq(uint32_t *xq, float *xd, int32_t m,
                                           int32_t n) const {
    const int32_t chunks = (m * n) >> 2;
#pragma unroll
    for (int j = 0; j < XC; j++) {
      if (j * kWG < chunks) {
        const int32_t c = j * kWG + (int32_t)threadIdx.x;
        uint32_t codes;
        const float d = q8x_chunk(x[j], codes);
        if (c < chunks) {
          xq[c] = codes;
          if ((c & 7) == 0) xd[c >> 3] = d;
        }
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
        // one row (m = 1) needs no division
        const int32_t i = m == 1 ? 0 : c / row_chunks, e = (c - i * row_chunks) * 4;
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

// One matvec cut into column slices (split-K, m = 1): slice i covers
// blocks [i * sb, min((i + 1) * sb, bpr)) of every row, owns tiles
// [i * tps, (i + 1) * tps) (the same row tiles in every slice) and writes its
// partial sums to part + i * p.  Its descriptor is derived, not stored.
struct SliceSrc {
  StepDesc base;   // the whole matvec; rows_per_tile is a slice's
  float *part;
  int32_t slices, sb, tps, pitch16;
  __device__ __forceinline__ int32_t find(int32_t t, int32_t) const { return t / tps; }
  __device__ __forceinline__ StepDesc get(int32_t i) const {
    StepDesc d = base;
    const int32_t b0 = i * sb, bpr = base.n >> 5;
    const int32_t nb = bpr - b0 < sb ? bpr - b0 : sb;
    d.w = base.w + (int64_t)b0 * 34;
    d.x = base.x + (int64_t)b0 * 32;
    d.n = nb * 32;
    d.y = part + (int64_t)i * base.p;
    d.idx = nullptr;
    d.slot = nullptr;
    d.tile_begin = i * tps;
    d.tile_end = d.tile_begin + tps;
    d.flags = pitch16 << kDescPitchShift;
    return d;
  }
};

struct TableSrc {
  const StepDesc *tab;
  int32_t count;
  // Last descriptor at or after `lo` with tile_begin <= t.  A workgroup
  // moves to the next matvec or the one after it almost always, so a short
  // forward scan answers before the binary search (dependent loads delay
  // the next tile's prefetch).
  __device__ __forceinline__ int32_t find(int32_t t, int32_t lo) const {
#pragma unroll
    for (int k = 0; k < 2; k++)
      if (lo + 1 < count && tab[lo + 1].tile_begin <= t) lo++;
    if (lo + 1 >= count || tab[lo + 1].tile_begin > t) return lo;
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

// A launch's prologue (see Prologue): the launch's x, computed by every
// workgroup into the padded LDS layout of its x region while its first tile
// loads, and stored to memory by one workgroup (`keep`).  It replaces a
// last-workgroup epilogue on the launch before, whose chain (completion
// wait, arrival counters, device-scope loads) followed the last tile.  Its
// loads (pro_load, the norm weight included) are issued before the first
// tile's: loads complete in issue order, so issued after the tile's bytes
// they would wait for them.
constexpr int kProChunks = kProMaxN / (4 * kWG);  // float4 chunks per thread
struct ProRegs {
  f32x4 a[kProChunks], b[kProChunks], c[kProChunks], w[kProChunks];
};

__device__ __forceinline__ void pro_load(const Prologue &p, ProRegs &r) {
  const int32_t chunks = p.n >> 2;
  const bool norm = p.op == kProAddNorm || p.op == kProNorm;
  const bool add = p.op != kProNorm;
  auto ld = [](const float *q, int32_t c) { return gp((const f32x4 *)q)[c]; };
#pragma unroll
  for (int k = 0; k < kProChunks; k++) {
    const int32_t c = (int32_t)threadIdx.x + k * kWG;
    r.a[k] = r.b[k] = r.c[k] = r.w[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < chunks) {
      r.a[k] = ld(p.a, c);
      if (add) r.b[k] = ld(p.b, c);
      if (norm) {
        if (add && p.c) r.c[k] = ld(p.c, c);
        r.w[k] = gp((const f32x4 *)p.w)[c];
      }
    }
  }
}

// The prologue's arithmetic on the values pro_load fetched.  red: 4 floats
// of LDS not otherwise in use.
// COH: workgroup 0's stores are device-scope (workgroups on other XCDs read
// them in later phases of the launch).
template <bool COH = false>
__device__ __forceinline__ void pro_finish(const Prologue &p, ProRegs &r, float *xs,
                                           float *red, bool keep) {
  const int32_t chunks = p.n >> 2;
  const bool norm = p.op == kProAddNorm || p.op == kProNorm;
  const bool add = p.op == kProAddNorm;
  float inv = 0.f;
  if (norm) {  // the residual sum in the order the adds run: (a + b) + c
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kProChunks; k++) {
      if (add) {
        r.a[k] = r.a[k] + r.b[k];
        if (p.c) r.a[k] = r.a[k] + r.c[k];
      }
#pragma unroll
      for (int e = 0; e < 4; e++) ss += r.a[k][e] * r.a[k][e];
    }
    ss = dec::block_sum_lds(ss, red);  // (the tile's loads in flight are not waited for)
    inv = 1.0f / sqrtf(ss / (float)p.n + p.eps);
  }
#pragma unroll
  for (int k = 0; k < kProChunks; k++) {
    const int32_t c = (int32_t)threadIdx.x + k * kWG;
    if (c < chunks) {
      f32x4 o;
      if (norm) {
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = r.a[k][e] * inv * r.w[k][e];
        if (keep && p.resid) {
          if (COH) st_dev4(p.resid + 4 * c, r.a[k]);
          else gpw((f32x4 *)p.resid)[c] = r.a[k];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; e++) o[e] = r.a[k][e] / (1.0f + expf(-r.a[k][e])) * r.b[k][e];
      }
      const int32_t i = 4 * c;
      *(f32x4 *)&xs[36 * (i >> 5) + (i & 31)] = o;
      if (keep) {
        if (COH) st_dev4(p.out + 4 * c, o);
        else gpw((f32x4 *)p.out)[c] = o;
      }
    }
  }
}

// Wave priority from the share of a workgroup's tiles still to come (left
// of total): 3 until the last three eighths, then 2, 1 and 0 for each
// further eighth.  The SIMD's arbiter prefers older waves, so of the
// workgroups sharing a CU the first dispatched streams its tiles fastest
// and the last finishes well after it (measured on MI355X with equal tile
// counts: 76 µs against 104 µs in one 197-matvec launch); priority to the
// workgroups with more tiles left evens out their progress and shortens
// the tail of launches with a few tiles per workgroup (the eighths were
// measured against quarters, halves, sixteenths and tiles: fused lm_head
// 29.5 µs against 30.3, 31.0, 29.9, 29.4; m = 8 step 152.9 µs against
// 153.4, 156.3, 155.1, 159.4).  s_setprio takes an
// immediate, hence the branches (uniform: scalar).
// Workgroups with fewer tiles keep the default priority: for launches of
// one or two tiles per workgroup (the chain graph's matvecs, the decode
// step's nodes) the priority was measured slower (197-node chain 711 →
// 747 µs).
constexpr int32_t kPrioMinTiles = 4;
__device__ __forceinline__ void set_progress_prio(int32_t left, int32_t total) {
  const int32_t b = min(3, left * 8 / (total + 1));
  if (b >= 3) __builtin_amdgcn_s_setprio(3);
  else if (b == 2) __builtin_amdgcn_s_setprio(2);
  else if (b == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Tiles first, first + stride, ... (< end) of the launch, in order.  Each
// tile's weights (and x, when the tile opens another matvec) are loaded into
// registers while the previous tile is computed.  Tiles of one matvec are
// contiguous, so a workgroup meets each matvec in one run of tiles; the run
// adds its argmax keys, if any, as one arrival.  M1: the launch has m = 1;
// ANY: some matvec of the launch takes the direct or generic path; PRIO:
// wave priority by progress (set_progress_prio), for the launches where it
// was measured faster on MI355X — standalone matvecs (fused lm_head 31.6 →
// 29.6 µs, with int8 activations 30.2 → 28.8 µs; not batched int8, where
// it is neutral) and the batched matrix-core step (m = 8: 170 → 153 µs);
// the m = 1 and int8-activation steps run slower with it (+1–3 %).
// NBLS: 0, or the blocks per lane (1, 2, 3) of every matvec of the launch,
// known at compile time (a standalone staged matvec), so the kernel holds
// one copy of the row loop instead of one per width and output mode.
// LDS: the staged tile, then (batched) the partial sums, then the padded x.
// COH (the persistent decode step, with DEC): what the launch hands from one
// phase to the next (the prologue's stores) is stored at device scope, and
// `wait` (the grid barrier; false when it failed) runs after this
// workgroup's first tile's weight bytes are requested and before anything
// the launch produced is read, so the barrier's latency and the first
// tile's overlap.  A workgroup without tiles only waits.  Its reads are
// plain loads: each buffer they read is written once in the launch, before
// the barrier that precedes the read, so no cache can hold an older copy
// (see decode_kernel).
struct NoWait {
  __device__ bool operator()() const { return true; }
};
template <bool M1, bool ANY, bool I8X, bool PRIO, int NBLS, bool DEC, class Src,
          bool STRIDED = false, bool COH = false, class Wait = NoWait,
          int MTB = kMfmaTileBytes, int MMB = kMfmaMaxBlocks>
__device__ void run_tiles(const Src &src, int32_t first, int32_t end,
                          int32_t stride, int32_t d_hint, int32_t m,
                          float *lds, const Prologue *pro = nullptr, Wait wait = Wait(),
                          const PairOut *pair = nullptr) {
  static_assert(!COH || (DEC && M1 && !ANY && !I8X && !STRIDED),
                "the persistent decode step: staged m = 1 tiles of the decode variant");
  static_assert(!(I8X && ANY), "int8 activations: staged shapes only");
  constexpr int XC = M1 ? 3 : (ANY ? 8 : 1);  // float4 chunks of x per thread
  // MTB, MMB: the batched tile's LDS bytes and each wave's x blocks
  constexpr int CH = M1 ? kStageChunks : (MTB + 16 * kWG - 1) / (16 * kWG);
  uint32_t *tl = (uint32_t *)lds;
  float *red = lds + (M1 ? kTileMaxBytes : MTB) / 4;
  float *xs = M1 ? red : red + kRedFloats;
  // int8 activations: the steps, then the packed codes (m = 1: after the
  // tile; batched: after the partial sums; the matrix-core tiles hold their
  // codes in registers and need no packed region)
  // (column slices: the steps of a slice's 32 blocks fit the last 16 floats
  // of the 16 entries of the partial sums, which no reduction touches)
  constexpr bool XPAD = I8X && STRIDED && !M1;
  static_assert(!XPAD || MMB * kWaves <= 2 * kWaves * 4, "a slice's steps fit the padding");
  static_assert(kRedStride - 64 >= 16, "two blocks of steps an entry");
  float *xd = M1 ? red : (XPAD ? red + 64 : red + kRedFloats);
  uint32_t *xq = (uint32_t *)(xd + kI8xMaxBlocks);
  // which path a tile takes; without ANY every m = 1 tile takes the staged
  // one; batched int8 tiles of the matrix-core widths take the matrix cores
  auto staged = [&](const Job &j) {
    return (I8X && (M1 || j.path != kMfma)) || (M1 && (!ANY || j.path == kStaged));
  };
  auto mfma = [&](const Job &j) {
    return !M1 && (I8X ? j.path == kMfma : (!ANY || j.path == kMfma));
  };
  // x prefetched into registers and staged in LDS with the tile
  auto x_in_lds = [&](const Job &j) {
    return M1 ? (!ANY || j.path != kGeneric) : (ANY && j.path == kDirect);
  };
  int32_t t = first;
  if (t >= end) {
    wait();
    return;
  }
  // The persistent step leaves the last wave's registers free of weight
  // loads: that wave arrives at and polls the grid barrier, and vector loads
  // return in issue order, so a poll behind the next phase's tile would
  // learn of the release only once the tile had arrived.
  constexpr int NL = COH ? kWG - 64 : kWG;
  constexpr int CHL = COH ? (kTileMaxBytes + 16 * NL - 1) / (16 * NL) : CH;
  Prefetch<XC, CHL, NL> pf;
  // The job of tile tn, a later tile than `from`'s: the same matvec, or one
  // found in the table.
  auto job_after = [&](const Job &from, int32_t tn) {
    if (tn < from.d.tile_end) return job_at(from.desc, from.d, tn, m);
    const int32_t dn = src.find(tn, from.desc + 1);
    return job_at(dn, src.get(dn), tn, m);
  };
  int32_t di = src.find(t, d_hint);
  Job cur = job_at(di, src.get(di), t, m);
  bool more = t + stride < end;
  Job nxt = more ? job_after(cur, t + stride) : cur;
  ProRegs prr;
  // a paired tile's row sums (DEC only): up to kPairMaxRows rows of each matrix
  float *pair_sums = nullptr;
  if constexpr (DEC) {
    __shared__ float pair_lds[2 * kPairMaxRows];
    pair_sums = pair_lds;
  }
  // the prologue's descriptor, read before the tiles' loads (and, in the
  // persistent step, before the barrier): its fields address the loads
  Prologue pr{};
  PairOut po{};  // the launch's paired matrix and outputs (DEC), read before any tile
  if constexpr (DEC) {
    if (pro) pr = *pro;
    if (pair) po = *pair;
  }
  if constexpr (DEC && !COH) {
    if (pro) pro_load(pr, prr);  // before the tile's loads: see pro_load
  }
  // a tile's weight bytes: whole rows, or (STRIDED) rows of a column slice
  auto load_tile = [&](const Job &j) {
    const int32_t rb = (j.d.n >> 5) * 34;
    if (DEC && (j.d.flags & kDescPairedSilu))
      pf.load_w_pair(j.d.w + (uint64_t)j.r0 * rb, po.w2 + (uint64_t)j.r0 * rb, j.rows * rb);
    else if (STRIDED)
      pf.load_w_strided(j.d.w + (uint64_t)j.r0 * desc_pitch16(j.d.flags) * 16u, j.rows * rb, rb,
                        desc_pitch16(j.d.flags) * 16);
    else
      pf.load_w(j.d.w + (uint64_t)j.r0 * rb, j.rows * rb);
  };
  if (staged(cur) || mfma(cur)) load_tile(cur);
  if (!wait()) return;  // the weights are in flight; what follows may read this launch's values
  if constexpr (DEC && COH) {
    if (pro) pro_load(pr, prr);
  }
  // the x staged in LDS (and the batched path's operand A): matvecs that
  // share x (the same pointer and width) are staged once
  const float *xptr = nullptr, *xaptr = nullptr;
  int32_t xn = 0, xan = 0;
  if constexpr (DEC) {
    if (pro) {  // the launch's x is pro->out, computed here while the first tile loads
      pro_finish<COH>(pr, prr, xs, lds, blockIdx.x == 0);  // the tile buffer is still free
      xptr = pr.out;
      xn = pr.n;
    }
  }
  if (x_in_lds(cur) && (cur.d.x != xptr || cur.d.n != xn))
    pf.load_x(cur.d.x, m * cur.d.n);
  unsigned long long best[8] = {0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull, 0ull};
  unsigned long long kb = 0ull;  // batched path: key of x row threadIdx.x / 16
  u32x4 xa[MMB];                 // batched path: this lane's operand A
  u32x2 xi[MMB];                 // batched int8 path: the same, x's codes
  const int32_t total = (end - 1 - first) / stride + 1;  // this workgroup's tiles
  (void)total;
  for (;;) {
    const int32_t tn = t + stride;
    const int32_t bpr = cur.d.n >> 5;
    if constexpr (PRIO)
      if (total >= kPrioMinTiles) set_progress_prio((end - 1 - t) / stride, total);
    const bool x_changed = cur.d.x != xptr || cur.d.n != xn;
    const bool new_x = x_in_lds(cur) && x_changed;
    __syncthreads();  // the previous tile's readers of LDS are done
    // batched int8 on the matrix cores: a new x's codes go through the tile
    // buffer (before this tile is staged there) into each wave's operand A;
    // its steps stay in LDS, block-major
    const bool quant_xi = I8X && !M1 && mfma(cur) && x_changed;
    if constexpr (I8X && !M1) {
      if (quant_xi) {
        // a column slice's x rows lie the whole matrix's width apart
        const int32_t xstride =
            STRIDED ? desc_pitch16(cur.d.flags) * 16 / 34 * 32 : cur.d.n;
        quantize_x_lds<kWG, true, XPAD>(cur.d.x, m, cur.d.n, tl, xd, xstride);
        __syncthreads();
        if constexpr (MMB >= 24) {
          if (bpr == 32) load_xi<8>(xi, tl, m, bpr);
          else if (bpr == 64) load_xi<16>(xi, tl, m, bpr);
          else load_xi<24>(xi, tl, m, bpr);
        } else {  // (every batched matvec of the launch 1024 wide)
          load_xi<8>(xi, tl, m, bpr);
        }
        __syncthreads();  // every wave holds its codes: the tile may overwrite them
      }
    }
    // a paired tile holds its rows of both matrices, one after the other
    const bool pair = DEC && (cur.d.flags & kDescPairedSilu);
    const int32_t trows = pair ? 2 * cur.rows : cur.rows;
    if (staged(cur)) pf.store_w(tl, trows * bpr * 34);
    else if (mfma(cur)) pf.store_w_rows(tl, cur.rows * bpr * 34, bpr * 34);
    if (new_x) {
      if (I8X) pf.store_xq(xq, xd, m, cur.d.n);
      else pf.store_x(xs, m, cur.d.n);
    }
    // batched (VALU tiles): straight from memory
    const bool quant_x = I8X && !M1 && !XPAD && !mfma(cur) && x_changed;
    if (quant_x) quantize_x_lds<kWG>(cur.d.x, m, cur.d.n, xq, xd);
    __syncthreads();
    if (new_x || quant_x || quant_xi) {
      xptr = cur.d.x;
      xn = cur.d.n;
    }
    // a new matvec's operand A is loaded before the next tile's bytes are
    // requested, so waiting for it does not wait for them
    if (!I8X && mfma(cur) && (cur.d.x != xaptr || cur.d.n != xan)) {
      // a column slice's x rows lie the whole matrix's width apart
      const int32_t xstride =
          STRIDED ? desc_pitch16(cur.d.flags) * 16 / 34 * 32 : cur.d.n;
      if constexpr (MMB >= 24) {
        if (bpr == 32) load_xa<8>(xa, cur.d.x, m, xstride);
        else if (bpr == 64) load_xa<16>(xa, cur.d.x, m, xstride);
        else load_xa<24>(xa, cur.d.x, m, xstride);
      } else {  // (every batched matvec of the launch 1024 wide)
        load_xa<8>(xa, cur.d.x, m, xstride);
      }
      xaptr = cur.d.x;
      xan = cur.d.n;
    }
    if (more) {  // next tile's bytes go out before this tile is computed
      // x first: a few scattered lines, slower to arrive than the tile's
      // streamed bytes, so its latency overlaps theirs rather than following
      if (x_in_lds(nxt) && (nxt.d.x != xptr || nxt.d.n != xn))
        pf.load_x(nxt.d.x, m * nxt.d.n);
      if (staged(nxt) || mfma(nxt)) load_tile(nxt);
    }
    // The job two tiles ahead.  A new matvec's descriptor is read from the
    // table here, so its scalar loads complete while this tile is computed:
    // read at the top of the next round, they would hold its first barrier
    // (which waits for every outstanding scalar load) and with it the next
    // tile's loads.
    const int32_t tn2 = tn + stride;
    const bool more2 = more && tn2 < end;
    const Job nxt2 = more2 ? job_after(nxt, tn2) : nxt;
    const bool keys = cur.d.idx != nullptr;
    const bool devy = DEC && (cur.d.flags & kDescDeviceOut);
    float *const yout = pair ? nullptr : cur.d.y;
    if (I8X) {
      const int nbl = NBLS ? NBLS : nbl_of(cur.d.n);
      if (M1) {
        if (nbl == 1) staged_m1_i8<1>(tl, bpr, cur.rows, xq, xd, cur.d.y, cur.r0, keys, best[0]);
        else if (nbl == 2) staged_m1_i8<2>(tl, bpr, cur.rows, xq, xd, cur.d.y, cur.r0, keys, best[0]);
        else staged_m1_i8<3>(tl, bpr, cur.rows, xq, xd, cur.d.y, cur.r0, keys, best[0]);
      } else if (mfma(cur)) {
        if constexpr (I8X && !M1 && MMB >= 24) {
          if (bpr == 32)
            mfma_tile_i8<8>(tl, bpr, cur.rows, m, cur.d.p, xi, xd, red, cur.d.y, cur.r0, keys, kb);
          else if (bpr == 64)
            mfma_tile_i8<16>(tl, bpr, cur.rows, m, cur.d.p, xi, xd, red, cur.d.y, cur.r0, keys, kb);
          else
            mfma_tile_i8<24>(tl, bpr, cur.rows, m, cur.d.p, xi, xd, red, cur.d.y, cur.r0, keys, kb);
        } else if constexpr (I8X && !M1) {
          mfma_tile_i8<8, MMB, XPAD>(tl, bpr, cur.rows, m, cur.d.p, xi, xd, red, cur.d.y, cur.r0,
                                     keys, kb);
        }
      } else if constexpr (!STRIDED) {  // (the sliced step's tiles all take the matrix cores)
        if (nbl == 1) staged_mb_i8<1>(tl, bpr, cur.rows, m, cur.d.p, xq, xd, cur.d.y, cur.r0, keys, best);
        else if (nbl == 2) staged_mb_i8<2>(tl, bpr, cur.rows, m, cur.d.p, xq, xd, cur.d.y, cur.r0, keys, best);
        else staged_mb_i8<3>(tl, bpr, cur.rows, m, cur.d.p, xq, xd, cur.d.y, cur.r0, keys, best);
      }
    } else if (staged(cur)) {
      const int nbl = NBLS ? NBLS : nbl_of(cur.d.n);
      float *const stash = pair ? pair_sums : nullptr;
      if (devy) {  // outputs read by the launch's epilogue (decode step levels)
        if (nbl == 1) staged_m1<1, true>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
        else if (nbl == 2) staged_m1<2, true>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
        else staged_m1<3, true>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
      } else {
        if (nbl == 1) staged_m1<1, false>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
        else if (nbl == 2) staged_m1<2, false>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
        else staged_m1<3, false>(tl, bpr, trows, xs, yout, cur.r0, keys, best[0], stash);
      }
      if constexpr (DEC) {
        if (pair) {  // silu_hadamard of the tile's rows, from both matrices' sums
          __syncthreads();
          const int32_t i = (int32_t)threadIdx.x;
          if (i < cur.rows) {
            const float gv = pair_sums[i], uv = pair_sums[cur.rows + i];
            const float hv = gv / (1.0f + expf(-gv)) * uv;
            store_y(&cur.d.y[cur.r0 + i], gv, devy);
            store_y(&po.y2[cur.r0 + i], uv, devy);
            store_y(&po.h[cur.r0 + i], hv, devy);
          }
        }
      }
    } else if (mfma(cur)) {
      if constexpr (MMB >= 24) {
        if (bpr == 32)
          mfma_tile<8>(tl, bpr, cur.rows, m, cur.d.p, xa, red, cur.d.y, cur.r0, keys, kb);
        else if (bpr == 64)
          mfma_tile<16>(tl, bpr, cur.rows, m, cur.d.p, xa, red, cur.d.y, cur.r0, keys, kb);
        else
          mfma_tile<24>(tl, bpr, cur.rows, m, cur.d.p, xa, red, cur.d.y, cur.r0, keys, kb);
      } else {
        mfma_tile<8>(tl, bpr, cur.rows, m, cur.d.p, xa, red, cur.d.y, cur.r0, keys, kb);
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
      c.devy = devy;
      run_direct<M1>(c, cur.path, best, keys);
    }
    if (keys && (!more || nxt.desc != cur.desc)) {
      // each wave's keys (the batched path holds x row r's in 16-lane row
      // r & 3 of wave r / 4) go to the start of the tile buffer once every
      // wave is done reading it (a static LDS array measured slower)
      __syncthreads();
      unsigned long long(*lk)[8] = (unsigned long long(*)[8])lds;
      const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
      if (mfma(cur)) {
        const unsigned long long rm = row16_max(kb);
#pragma unroll
        for (int r = 0; r < 8; r++) {
          if (r < m) {
            const unsigned long long k =
                (r >> 2) == wave ? readlane64(rm, 16 * (r & 3) + 15) : 0ull;
            if (lane == 0) lk[wave][r] = k;
          }
        }
        kb = 0ull;
      } else {
#pragma unroll
        for (int r = 0; r < 8; r++) {
          if (r < m) {
            const unsigned long long k = wave_max64(best[r]);
            if (lane == 0) lk[wave][r] = k;
          }
          best[r] = 0ull;
        }
      }
      argmax_arrive(lk, m, cur.d.slot, cur.d.idx, blockIdx.x, gridDim.x);
    }
    if (!more) break;
    t = tn;
    cur = nxt;
    nxt = nxt2;
    more = more2;
  }
}


// ---- wide batches: 8 < m <= 32 -------------------------------------------------
//
// Up to 32 activation rows share one sweep of the weights (the Algenta page's
// batched decode arm, where the rows of a batch share one weight sweep;
// rvllm's linear_small loops the rows inside its weight loop).  At this width
// the products are a dense contraction, so they run on the matrix cores, but
// x (32 rows x n, hi and lo bf16) no longer fits in registers, so it is
// staged in LDS a K-chunk at a time beside the weights:
//  * a tile is 128 weight rows (each wave two 16-row groups) over the whole
//    row, walked in chunks of 8 blocks (256 columns);
//  * per chunk the tile's 128 x 272 weight bytes go to LDS (coalesced
//    16-byte loads, rows padded to 288 bytes) and the m x 256 floats of x
//    become operand columns: column group c holds x rows 8c .. 8c + 7 as bf16
//    "hi" (columns 0..7) and the bf16 of the rounding rest "lo" (8..15), the
//    split of the m <= 8 path;
//  * per block, each wave builds the quant operand of its two row groups
//    once, reads each column group's operand once and issues up to eight
//    v_mfma_f32_16x16x32_bf16, each scaled once by the block's scale;
//  * the next chunk's bytes are loaded into registers while this one is
//    computed.
// At the end y[xr][row] = hi column + lo column (a lane and the lane 32
// above it).  Requires n a multiple of 256.

constexpr int kWideRows = 128;
constexpr int kWideKB = 8;                                // blocks per chunk
constexpr int kWideWPitch = kWideKB * 34 + 16;            // staged weight row, bytes
constexpr int kWideXPitch = kWideKB * 32 * 2 + 16;        // operand column, bytes
constexpr int kWideWBytes = kWideRows * kWideWPitch;      // 36,864
constexpr int kWideXBytes = 4 * 16 * kWideXPitch;         // 33,792
constexpr int kWideKeys = kWaves * 32 * 8;                // argmax keys, bytes
constexpr int kWideLds = kWideWBytes + kWideXBytes + kWideKeys;
constexpr int kWideWChunks = (kWideRows * 17 + kWG - 1) / kWG;  // 16-byte loads / thread
constexpr int kWideXChunks = 32 * 64 / kWG;                      // float4 loads / thread

struct WideItem {
  int32_t desc;  // descriptor index, -1: none
  int32_t r0, rows, kc;
  StepDesc d;
};

// Registers carrying one chunk from memory to LDS.
struct WidePrefetch {
  u32x4 w[kWideWChunks];
  f32x4 x[kWideXChunks];

  __device__ __forceinline__ void load(const WideItem &it, int32_t m) {
    const int32_t pitch = (it.d.n >> 5) * 34;
    const uint8_t *wb = it.d.w + (int64_t)it.r0 * pitch + 272 * it.kc;
#pragma unroll
    for (int i = 0; i < kWideWChunks; i++) {
      const int idx = (int)threadIdx.x + kWG * i;
      const int row = idx / 17, q = idx % 17;
      w[i] = u32x4{0u, 0u, 0u, 0u};
      if (row < it.rows)
        w[i] = __builtin_nontemporal_load(
            (const u32x4 *)(wb + (int64_t)row * pitch + 16 * q));
    }
#pragma unroll
    for (int i = 0; i < kWideXChunks; i++) {
      const int idx = (int)threadIdx.x + kWG * i;
      const int xr = idx >> 6, q = idx & 63;
      x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (xr < m)
        x[i] = *(const f32x4 *)(it.d.x + (int64_t)xr * it.d.n + 256 * it.kc + 4 * q);
    }
  }

  __device__ __forceinline__ void store(uint8_t *wl, uint8_t *xl) const {
#pragma unroll
    for (int i = 0; i < kWideWChunks; i++) {
      const int idx = (int)threadIdx.x + kWG * i;
      const int row = idx / 17, q = idx % 17;
      if (row < kWideRows) *(u32x4 *)(wl + row * kWideWPitch + 16 * q) = w[i];
    }
#pragma unroll
    for (int i = 0; i < kWideXChunks; i++) {
      const int idx = (int)threadIdx.x + kWG * i;
      const int xr = idx >> 6, q = idx & 63;
      uint32_t h[4], l[4];
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const float hi = (float)(__bf16)x[i][c];
        h[c] = bf16_bits(x[i][c]);
        l[c] = bf16_bits(x[i][c] - hi);
      }
      uint8_t *col = xl + (xr >> 3) * 16 * kWideXPitch + (xr & 7) * kWideXPitch + 8 * q;
      *(uint2 *)col = uint2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      *(uint2 *)(col + 8 * kWideXPitch) = uint2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    }
  }
};

// The work items of one workgroup: tiles first, first + stride, ... (< end),
// each in bpr / 8 chunks.
template <class Src>
__device__ __forceinline__ WideItem wide_item(const Src &src, int32_t t, int32_t end,
                                              int32_t kc, int32_t hint) {
  WideItem it;
  it.desc = -1;
  if (t >= end) return it;
  it.desc = src.find(t, hint);
  it.d = src.get(it.desc);
  it.r0 = (t - it.d.tile_begin) * kWideRows;
  it.rows = min(kWideRows, it.d.p - it.r0);
  it.kc = kc;
  return it;
}

// PRIO: wave priority by progress (set_progress_prio); measured on MI355X
// it shortens the persistent step (m = 32: 337 → 333 µs) and slows the
// standalone matvec slightly, so only the step launch takes it.
template <bool PRIO, class Src>
__device__ void wide_tiles(const Src &src, int32_t first, int32_t end, int32_t stride,
                           int32_t m, float *lds) {
  uint8_t *wl = (uint8_t *)lds;
  uint8_t *xl = wl + kWideWBytes;
  unsigned long long(*lk)[32] = (unsigned long long(*)[32])(xl + kWideXBytes);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int ncg = (m + 7) >> 3;  // live column groups
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  int32_t t = first;
  WideItem cur = wide_item(src, t, end, 0, 0);
  if (cur.desc < 0) return;
  WidePrefetch pf;
  pf.load(cur, m);
  f32x4 acc[2][4];
  unsigned long long best[4][4];
#pragma unroll
  for (int c = 0; c < 4; c++)
#pragma unroll
    for (int r = 0; r < 4; r++) best[c][r] = 0ull;
  for (;;) {
    if (cur.kc == 0) {
      if constexpr (PRIO) set_progress_prio((end - 1 - t) / stride, (end - 1 - first) / stride + 1);
#pragma unroll
      for (int rg = 0; rg < 2; rg++)
#pragma unroll
        for (int c = 0; c < 4; c++) acc[rg][c] = zero;
    }
    // the next chunk: this tile's, or the next tile's first
    const int32_t nchunks = (cur.d.n >> 5) / kWideKB;
    WideItem nxt = cur;
    if (cur.kc + 1 < nchunks) {
      nxt.kc = cur.kc + 1;
    } else {
      const int32_t tn = t + stride;
      nxt = wide_item(src, tn, end, 0, cur.desc);
    }
    __syncthreads();  // the previous chunk's readers are done
    pf.store(wl, xl);
    __syncthreads();
    if (nxt.desc >= 0) pf.load(nxt, m);

#pragma unroll
    for (int b = 0; b < kWideKB; b++) {
      // quant operands and scales of the wave's two row groups (row j)
      bf16x8 qb[2];
      float sc[2];
#pragma unroll
      for (int rg = 0; rg < 2; rg++) {
        // row pitch and 34 * (even b) are multiples of 4: an even block's
        // scale opens a dword and its quants start 2 bytes in; an odd
        // block's scale closes a dword and its quants are dword-aligned
        const uint8_t *rp = wl + (32 * wave + 16 * rg + j) * kWideWPitch + 34 * b;
        uint32_t qa, qc;
        if ((b & 1) == 0) {
          const uint32_t *wq = (const uint32_t *)(rp + 8 * g);
          const uint32_t e0 = wq[0], e1 = wq[1], e2 = wq[2];
          qa = __builtin_amdgcn_perm(e1, e0, 0x05040302u);
          qc = __builtin_amdgcn_perm(e2, e1, 0x05040302u);
          sc[rg] = (float)__builtin_bit_cast(
              _Float16, (uint16_t)(((const uint32_t *)rp)[0] & 0xFFFFu));
        } else {
          const uint32_t *wq = (const uint32_t *)(rp + 2 + 8 * g);
          qa = wq[0];
          qc = wq[1];
          sc[rg] = (float)__builtin_bit_cast(
              _Float16, (uint16_t)(((const uint32_t *)(rp - 2))[0] >> 16));
        }
        qb[rg] = quants_bf16(qa, qc);
      }
#pragma unroll
      for (int c = 0; c < 4; c++) {
        if (c < ncg) {
          const u32x4 xa = *(const u32x4 *)(xl + c * 16 * kWideXPitch + j * kWideXPitch +
                                            2 * (32 * b + 8 * g));
#pragma unroll
          for (int rg = 0; rg < 2; rg++) {
            const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xa), qb[rg], zero, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; r++) acc[rg][c][r] = fmaf(sc[rg], d[r], acc[rg][c][r]);
          }
        }
      }
    }

    if (cur.kc + 1 == nchunks) {  // the tile is complete: outputs and keys
      const bool keys = cur.d.idx != nullptr;
#pragma unroll
      for (int rg = 0; rg < 2; rg++) {
        const int32_t row = 32 * wave + 16 * rg + j;
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const float v = acc[rg][c][r] + __shfl_xor(acc[rg][c][r], 32, 64);
            const int xr = 8 * c + 4 * (g & 1) + r;
            if (g < 2 && c < ncg && xr < m && row < cur.rows) {
              if (cur.d.y) store_y(&cur.d.y[(int64_t)xr * cur.d.p + cur.r0 + row], v);
              if (keys) best[c][r] = umax64(best[c][r], argmax_key(v, (uint32_t)(cur.r0 + row)));
            }
          }
        }
      }
      if (keys && (nxt.desc < 0 || nxt.desc != cur.desc)) {
        // per x row: the maximum over the 16 lanes of each row, then over waves
        __syncthreads();  // lk (after the x chunk) is free
#pragma unroll
        for (int c = 0; c < 4; c++) {
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const unsigned long long k = row16_max(best[c][r]);
            const int xr = 8 * c + 4 * (g & 1) + r;
            if ((lane & 15) == 15 && g < 2 && xr < 32) lk[wave][xr] = xr < m ? k : 0ull;
            best[c][r] = 0ull;
          }
        }
        argmax_arrive(lk, m, cur.d.slot, cur.d.idx, blockIdx.x, gridDim.x);
      }
      t += stride;
    }
    if (nxt.desc < 0) break;
    cur = nxt;
  }
}


// ---- kernels -----------------------------------------------------------------

// One matvec (descriptor passed by value), its tiles round-robin over the
// grid (gridDim.x <= tiles, so every workgroup arrives at the argmax): at
// any moment the grid streams one contiguous window of the weights.
template <bool M1, bool ANY, bool I8X, int NBLS>
__global__ void __launch_bounds__(kWG, M1 ? 1 : 2)
mv_kernel(StepDesc d, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  OneSrc src{d};
  // tiles round-robin over the grid; within each 32 workgroups, runs of
  // four consecutive tiles on one XCD (as the step's groups)
  const int32_t b = (int32_t)blockIdx.x, b0 = b & ~31;
  const int32_t first = b0 + 32 <= (int32_t)gridDim.x ? b0 + group_slot(b & 31, 0, 32) : b;
  run_tiles<M1, ANY, I8X, M1 || !I8X, NBLS, false>(src, first, d.tile_end, gridDim.x, 0, m,
                                                     lds);
}

// One matvec at m = 1 cut into column slices (SliceSrc), each slice's tiles
// staged like mv_kernel's; the partial sums go to the slices' vectors and
// reduce_slices adds them.
template <int NBLS>
__global__ void __launch_bounds__(kWG, 1) mv_split_kernel(SliceSrc src) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int32_t b = (int32_t)blockIdx.x, b0 = b & ~31;
  const int32_t first = b0 + 32 <= (int32_t)gridDim.x ? b0 + group_slot(b & 31, 0, 32) : b;
  run_tiles<true, false, false, true, NBLS, false, SliceSrc, true>(
      src, first, src.slices * src.tps, gridDim.x, 0, 1, lds);
}

// y[e] = part[e] + part[p + e] + ... (slices in order, one row), and the
// argmax of y when idx is set (every workgroup arrives once).
__global__ void __launch_bounds__(kWG)
reduce_slices(const float *__restrict__ part, int32_t slices, int32_t p, float *__restrict__ y,
              ArgmaxSlot *__restrict__ slot, int32_t *__restrict__ idx) {
  unsigned long long key = 0ull;
  for (int32_t e = blockIdx.x * kWG + threadIdx.x; e < p; e += gridDim.x * kWG) {
    float v = gp(part)[e];
    for (int32_t i = 1; i < slices; i++) v += gp(part)[(int64_t)i * p + e];
    if (y) gpw(y)[e] = v;
    key = umax64(key, argmax_key(v, (uint32_t)e));
  }
  if (!idx) return;
  __shared__ unsigned long long lk[kWaves][1];
  key = wave_max64(key);
  if ((threadIdx.x & 63) == 0) lk[threadIdx.x >> 6][0] = key;
  argmax_arrive(lk, 1, slot, idx, blockIdx.x, gridDim.x);
}

// The persistent step: every tile of every descriptor of a device-side
// table (count entries in tile order), with no ordering between
// descriptors.  Workgroups form groups; a group interleaves its contiguous
// tile range.  DEC (m = 1 with binary32 activations only): the whole decode
// step's variant, with the prologue (pro, or NULL) and the epilogue (epi, or
// NULL: element-wise work that the last workgroup to finish runs once every
// tile is written); the other launches do not carry that code.
template <bool M1, bool ANY, bool I8X, bool DEC>
__global__ void __launch_bounds__(kWG, M1 ? 1 : 2)
step_kernel(const StepDesc *__restrict__ table, int32_t count,
            const WgGroup *__restrict__ groups, int32_t group_size, int32_t m,
            const Epilogue *__restrict__ epi, const Prologue *__restrict__ pro,
            const PairOut *__restrict__ pair) {
  static_assert(!DEC || (M1 && !I8X), "the decode variant is m = 1, binary32");
  extern __shared__ __attribute__((aligned(16))) float lds[];
  TableSrc src{table, count};
  const WgGroup g = groups[blockIdx.x / group_size];
  const int32_t j = (int32_t)blockIdx.x - g.first;
  run_tiles<M1, ANY, I8X, !M1 && !I8X, 0, DEC>(src, g.t0 + group_slot(j, g.first, g.size),
                                               g.t1, g.size, g.d0, m, lds, pro, NoWait(),
                                               pair);
  if constexpr (DEC) {
    if (epi) {
      __syncthreads();  // every wave is done with the tile buffer
      dec::run_epilogue(epi, blockIdx.x, gridDim.x, lds);
    }
  }
}

// ---- the persistent decode step --------------------------------------------

__device__ __forceinline__ uint32_t ld_dev_u32(uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_u32(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A wait at the grid barrier gives up after this many ticks of the 100 MHz
// clock (200 ms; a whole decode step takes about 1 ms).
constexpr uint64_t kBarrierSpinTicks = 20000000ull;
// The thread that arrives at and polls the barrier: the first of the last
// wave, which requests no weights (run_tiles with COH).
constexpr uint32_t kBarrierThread = kWG - 64;

// This workgroup's arrival at the grid barrier that releases generation
// `target`.  Every wave first waits until its stores are complete (the
// values it hands on travel with device-scope stores), then kBarrierThread counts
// the workgroup into its team (workgroup b in team b % 32, its counter in
// its own line); the team's last arrival counts the team in, and the last
// team's arrival writes `target` into every team's release line.  The
// counters are never reset: after generation t is released team j's reads
// size_j * t and the top counter nteams * t (modulo 2^32), so an arrival
// knows it is the last one from the value its increment returns, and no
// store has to be ordered before another.  Relaxed agent-scope atomics.
__device__ __forceinline__ void grid_arrive(GridBarrier *b, uint32_t target) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x >= kBarrierThread) {  // the last wave
    uint32_t release = 0u;
    if (threadIdx.x == kBarrierThread) {
      const uint32_t G = gridDim.x, T = kGridTeams, j = blockIdx.x % T;
      const uint32_t size = (G - j + T - 1) / T, nteams = G < T ? G : T;
      const uint32_t prev = __hip_atomic_fetch_add(&b->team[j][0], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      if (prev + 1u == size * target) {
        const uint32_t p2 = __hip_atomic_fetch_add(&b->top[0], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
        release = p2 + 1u == nteams * target ? 1u : 0u;
      }
    }
    // the release lines are written by one store instruction of 32 lanes:
    // one lane storing them in turn took about 20 ns a line (the last team
    // saw its release 0.6 us after the first on MI355X)
    release = (uint32_t)__builtin_amdgcn_readlane((int)release, 0);
    const uint32_t k = threadIdx.x - kBarrierThread;
    if (release && k < (uint32_t)kGridTeams) st_dev_u32(&b->gen[k][0], target);
  }
}

// Waits (kBarrierThread polls its team's release line) until `target` is
// released.  False in every thread once the barrier has failed: this wait
// ran past kBarrierSpinTicks (it then marks the failure and stores -2 as
// the step's token) or another workgroup's did.  flag: one word of LDS.
__device__ __forceinline__ bool grid_wait(GridBarrier *b, uint32_t target, uint32_t *flag) {
  if (threadIdx.x == kBarrierThread) {
    uint32_t ok = 1u;
    uint32_t *line = &b->gen[blockIdx.x % kGridTeams][0];
    const uint64_t start = __builtin_amdgcn_s_memrealtime();
    for (;;) {
      if ((int32_t)(ld_dev_u32(line) - target) >= 0) break;
      if (ld_dev_u32(&b->error[0])) {
        ok = 0u;
        break;
      }
      if (__builtin_amdgcn_s_memrealtime() - start > kBarrierSpinTicks) {
        st_dev_u32(&b->error[0], 1u);
        ok = 0u;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) {
      int32_t *idx = gp(&b->idx)[0], *host = gp(&b->host)[0];
      if (idx) __hip_atomic_store(idx, -2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (host) __hip_atomic_store(host, -2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    *flag = ok;
  }
  // LDS-only barriers: the weight loads the other waves issued before the
  // wait are not waited for here (the code after the wait issues its own
  // loads first)
  dec::lds_barrier();
  const bool ok = *flag != 0u;
  dec::lds_barrier();  // the flag is rewritten by the next wait
  return ok;
}

// The batched step in column slices: every descriptor 1024 wide with its
// matrix's row pitch (a column slice, or a 1024-wide matrix whole), so each
// wave keeps 8 blocks of x (a third of the registers of 3072-wide rows) and
// a tile is two 16-row groups (35 KB of LDS, 40 KB with the partial sums,
// in whose padding the int8 form keeps x's steps): four workgroups a CU.
constexpr int kSliceRows = 32;
constexpr int kMaxSlices = 3;  // 3072 / kSliceWidth
constexpr int kSliceTileBytes = kSliceRows * ((kSliceWidth >> 5) * 34 + kMfmaRowPad);
// I8X: int8 activations (the matrix-core int8 tile, x quantised per slice:
// a slice starts at a block boundary, so its blocks' codes and steps are
// those of the whole row).
template <bool I8X>
__global__ void __launch_bounds__(kWG, 4)
sliced_step_kernel(const StepDesc *__restrict__ table, int32_t count,
                   const WgGroup *__restrict__ groups, int32_t group_size, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  TableSrc src{table, count};
  const WgGroup g = groups[blockIdx.x / group_size];
  const int32_t j = (int32_t)blockIdx.x - g.first;
  run_tiles<false, false, I8X, true, 0, false, TableSrc, true, false, NoWait, kSliceTileBytes,
            (kSliceWidth >> 5) / kWaves>(src, g.t0 + group_slot(j, g.first, g.size), g.t1,
                                         g.size, g.d0, m, lds);
}

// y = the sum of a sliced matvec's partial outputs, in slice order
// (blockIdx.y: the matvec).
// Four outputs a thread where the lengths and addresses allow it, with every
// slice's load in flight at once.
__global__ void __launch_bounds__(kWG)
slice_sum_kernel(const SliceSum *__restrict__ sums, int32_t count) {
  const SliceSum s = sums[blockIdx.y];
  const bool vec = (s.len & 3) == 0 && ((uintptr_t)s.y & 15) == 0 && ((uintptr_t)s.part & 15) == 0;
  if (vec) {  // (uniform)
    const f32x4 *pv = (const f32x4 *)s.part;
    f32x4 *yv = (f32x4 *)s.y;
    const int32_t n4 = s.len >> 2;
    for (int32_t e = (int32_t)(blockIdx.x * kWG + threadIdx.x); e < n4;
         e += (int32_t)(gridDim.x * kWG)) {
      f32x4 t[kMaxSlices];
#pragma unroll
      for (int q = 0; q < kMaxSlices; q++)
        if (q < s.k) t[q] = pv[(int64_t)q * n4 + e];
      f32x4 v = t[0];
#pragma unroll
      for (int q = 1; q < kMaxSlices; q++)
        if (q < s.k) v = v + t[q];
      yv[e] = v;
    }
    return;
  }
  for (int32_t e = (int32_t)(blockIdx.x * kWG + threadIdx.x); e < s.len;
       e += (int32_t)(gridDim.x * kWG)) {
    float v = s.part[e];
    for (int32_t q = 1; q < s.k; q++) v += s.part[(int64_t)q * s.len + e];
    s.y[e] = v;
  }
}

// The whole decode step in one launch (G query heads per key/value head):
// the phases of a device-side table in order, every workgroup meeting the
// others at the grid barrier between two phases.  A matvec phase runs the
// decode step kernel's tiles (outputs stored at device scope); an attention
// phase gives workgroup b the attention blocks b, b + grid, ...; a
// workgroup with nothing to do in a phase only meets the barrier.  Between
// its arrival and its wait a workgroup requests its next phase's first
// weight tile (a matvec phase) or its cached key and value rows (an
// attention phase), which do not depend on the phase before.
// The values one phase hands to the next are written to buffers that the
// launch writes once (each layer has its own, 256-byte aligned), stored at
// device scope, so they are in memory before their writer arrives at the
// barrier.  Their readers use plain loads: the caches were invalidated when
// the launch started and no workgroup has read those lines since, so the
// first read of a line by an XCD misses its L2 and fetches the stored
// value, and the XCD's other workgroups then hit in its L2.  (Device-scope
// loads instead go to memory for every workgroup: 512 workgroups reading
// the same 4-24 KB vector took 1-3 us per phase on MI355X.)  The attention
// partials, reused by every layer, are still read at device scope.
// Two workgroups per CU: the compiler then keeps every value in registers
// (224 VGPRs); asked for three or four it spills 56-261 of them.
template <int G>
__global__ void __launch_bounds__(kWG, 2)
decode_kernel(const DecPhase *__restrict__ phases, int32_t nphases,
              GridBarrier *__restrict__ bar) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ uint32_t flag;
  if (threadIdx.x == 0)  // read before this workgroup's first arrival, so no
                         // barrier of this launch has been released yet
    flag = ld_dev_u32(&bar->gen[blockIdx.x % kGridTeams][0]);
  __syncthreads();
  const uint32_t base = flag;
  __syncthreads();
  bool ok = true;
  for (int32_t i = 0; i < nphases && ok; i++) {
    if (i > 0) grid_arrive(bar, base + (uint32_t)i);
    const DecPhase ph = phases[i];
    auto wait = [&]() -> bool {
      if (i > 0 && ok) ok = grid_wait(bar, base + (uint32_t)i, &flag);
      return ok;
    };
    if (ph.kind == kPhaseMatvec) {
      const int32_t b = (int32_t)blockIdx.x;
      if (b < ph.grid) {
        TableSrc src{ph.table, ph.count};
        const WgGroup g = ph.groups[b / ph.group_size];
        const int32_t j = b - g.first;
        run_tiles<true, false, false, false, 0, true, TableSrc, false, true>(
            src, g.t0 + group_slot(j, g.first, g.size), g.t1, g.size, g.d0, 1, lds, ph.pro,
            wait, ph.pair);
      } else {
        wait();
      }
    } else {
      const AttnArgs a = *ph.attn;
      dec::AttnLds<G> &S = *(dec::AttnLds<G> *)lds;
      bool waited = false;
      auto wait_once = [&] {
        if (!waited) {
          waited = true;
          wait();
        }
      };
      for (int32_t blk = (int32_t)blockIdx.x; blk < a.n_kv * a.chunks && ok;
           blk += (int32_t)gridDim.x) {
        dec::attention_block<G, true>(a, blk, S, wait_once);
        __syncthreads();  // S serves the next block
      }
      wait_once();
    }
    __syncthreads();  // the phase's readers of LDS are done
  }
}

// Wide batches (8 < m <= 32): one matvec (tiles round-robin over the grid),
// or every tile of a descriptor table in workgroup groups, as the kernels
// above.
__global__ void __launch_bounds__(kWG, 2) wide_mv_kernel(StepDesc d, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  OneSrc src{d};
  wide_tiles<false>(src, blockIdx.x, tiles_of(d), gridDim.x, m, lds);
}

__global__ void __launch_bounds__(kWG, 2)
wide_step_kernel(const StepDesc *__restrict__ table, int32_t count,
                 const WgGroup *__restrict__ groups, int32_t group_size, int32_t m) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  TableSrc src{table, count};
  const WgGroup g = groups[blockIdx.x / group_size];
  const int32_t j = (int32_t)blockIdx.x - g.first;
  wide_tiles<true>(src, g.t0 + group_slot(j, g.first, g.size), g.t1, g.size, m, lds);
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
  __shared__ unsigned long long lk[kWaves][32];
  key = wave_max64(key);
  if ((threadIdx.x & 63) == 0)
    for (int r = 0; r < m; r++) lk[threadIdx.x >> 6][r] = r == (int)blockIdx.y ? key : 0ull;
  argmax_arrive(lk, m, slot, idx, blockIdx.y * gridDim.x + blockIdx.x,
                gridDim.x * gridDim.y);
}

// ---- host side ---------------------------------------------------------------

// Dynamic LDS of a launch whose matvecs have widths up to n_max.
// int8 activations: tile, steps, packed codes (m * n bytes).
// Batched (m > 1): the batched tile and its partial sums, the steps, and
// the packed codes for widths off the matrix cores (whose tiles keep x's
// codes in registers).
size_t lds_bytes_i8x(int m, int n) {
  if (m == 1) return kTileMaxBytes + (size_t)kI8xMaxBlocks * 4 + (size_t)n;
  return kMfmaTileBytes + (size_t)(kRedFloats + kI8xMaxBlocks) * 4 +
         (path_of(m, n) == kMfma ? 0 : (size_t)m * n);
}

// Rows per tile of the int8-activation variant: staged tiles, except the
// batched matrix-core widths (whole 16-row groups, as the f32 batched path).
int i8x_tile_rows(int m, int n) {
  return m > 1 && path_of(m, n) == kMfma ? tile_rows_of(m, n) : tile_rows_of(1, n);
}

size_t lds_bytes_for(int m, int n) {
  const int path = path_of(m, n);
  if (path == kWide) return kWideLds;
  if (m == 1) {  // the x region starts after the tile region
    const size_t x = path == kGeneric ? 0 : (size_t)x_lds_floats(m, n);
    return kTileMaxBytes + x * sizeof(float);
  }
  // tile, partial sums, then x for the direct path
  const size_t x = path == kDirect ? (size_t)x_lds_floats(m, n) : 0;
  return kMfmaTileBytes + (kRedFloats + x) * sizeof(float);
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
template <bool M1, bool ANY, bool I8X, int NBLS>
int mv_grid_cap(int dev) {
  static int cache[64] = {0};
  int &c = cache[dev & 63];
  if (!c) {
    const size_t lds = I8X ? lds_bytes_i8x(M1 ? 1 : kMaxM, kMaxLdsBlocks * 32)
                       : M1 ? kTileMaxBytes + (size_t)kMaxLdsBlocks * 36 * 4
                            : kMfmaTileBytes + (size_t)kRedFloats * 4 +
                                  (ANY ? (size_t)kXMaxFloats / 32 * 36 * 4 : 0);
    c = resident_wgs(mv_kernel<M1, ANY, I8X, NBLS>, lds, dev);
  }
  return c;
}

int wide_grid_cap(int dev) {
  static int cache[64] = {0};
  int &c = cache[dev & 63];
  if (!c) c = resident_wgs(wide_mv_kernel, kWideLds, dev);
  return c;
}

template <bool M1, bool ANY, bool I8X, int NBLS = 0>
hipError_t launch_mv(StepDesc d, int m, hipStream_t s) {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int cap = mv_grid_cap<M1, ANY, I8X, NBLS>(dev);
  // Every workgroup takes whole rounds of tiles, so the last round may be
  // part-empty.  Among tile heights from the largest down to three quarters
  // of it, take the one whose busiest workgroup costs least, counting a
  // tile as its rows plus four rows' worth of fixed work (barriers, LDS
  // staging).  Batched tiles stay whole 16-row groups.  (Whole rounds of
  // two tile heights, 21 and 22 rows for the lm_head, measured 1.5 us
  // slower: more tiles, and a part-empty last round also frees bandwidth
  // for the workgroups still running.)
  if (path_of(m, d.n) != kMfma && tiles_of(d) > cap) {
    int32_t best_rows = d.rows_per_tile;
    int64_t best_cost = INT64_MAX;
    for (int32_t r = d.rows_per_tile; r >= (3 * d.rows_per_tile + 3) / 4; r--) {
      const int64_t tiles = ((int64_t)d.p + r - 1) / r;
      const int64_t cost = (tiles + cap - 1) / cap * (r + 4);
      if (cost < best_cost) best_cost = cost, best_rows = r;
    }
    d.rows_per_tile = best_rows;
  }
  const int32_t ntiles = tiles_of(d);
  d.tile_end = ntiles;
  const int grid = ntiles < cap ? ntiles : cap;
  hipLaunchKernelGGL((mv_kernel<M1, ANY, I8X, NBLS>), dim3(grid), dim3(kWG),
                     I8X ? lds_bytes_i8x(m, d.n) : lds_bytes_for(m, d.n), s, d, m);
  return hipGetLastError();
}

}  // namespace

int step_rows_per_tile(int n, int m, bool i8x) {
  return i8x ? i8x_tile_rows(m, n) : tile_rows_of(m, n);
}

size_t step_lds_bytes(int m, int n, bool i8x) {
  return i8x ? lds_bytes_i8x(m, n) : lds_bytes_for(m, n);
}

bool step_all_staged(int m, int n, bool i8x) {
  if (i8x) return i8x_shape_ok(n);
  if (m > kMaxM) return true;  // one kernel for every wide matvec
  return path_of(m, n) == (m == 1 ? kStaged : kMfma);
}

bool wide_shape_ok(int n) { return n > 0 && n % 256 == 0; }

bool i8x_shape_ok(int n) { return path_of(1, n) == kStaged; }

int step_grid(int device, int m, size_t lds, bool all_staged, bool i8x, bool dec) {
  if (m > kMaxM) return resident_wgs(wide_step_kernel, lds, device);
  if (i8x)
    return m == 1 ? resident_wgs(step_kernel<true, false, true, false>, lds, device)
                  : resident_wgs(step_kernel<false, false, true, false>, lds, device);
  if (m == 1 && dec)
    return all_staged ? resident_wgs(step_kernel<true, false, false, true>, lds, device)
                      : resident_wgs(step_kernel<true, true, false, true>, lds, device);
  if (m == 1)
    return all_staged ? resident_wgs(step_kernel<true, false, false, false>, lds, device)
                      : resident_wgs(step_kernel<true, true, false, false>, lds, device);
  return all_staged ? resident_wgs(step_kernel<false, false, false, false>, lds, device)
                    : resident_wgs(step_kernel<false, true, false, false>, lds, device);
}

hipError_t launch_matvec(const uint8_t *w, const float *x, float *y, int m,
                         int n, int p, ArgmaxSlot *slot, int32_t *idx,
                         hipStream_t s, bool i8x) {
  if (p <= 0) return hipSuccess;
  StepDesc d{};  // flags 0: plain stores, tiles of equal height
  d.w = w;
  d.x = x;
  d.y = y;
  d.idx = idx;
  d.slot = slot;
  d.n = n;
  d.p = p;
  d.tile_begin = 0;
  d.rows_per_tile = i8x ? i8x_tile_rows(m, n) : tile_rows_of(m, n);
  d.tile_end = tiles_of(d);
  if (m > kMaxM) {  // wide batch: 128-row tiles round-robin over the grid
    const int32_t ntiles = tiles_of(d);
    int dev = 0;
    (void)hipGetDevice(&dev);
    const int cap = wide_grid_cap(dev);
    const int grid = ntiles < cap ? ntiles : cap;
    hipLaunchKernelGGL(wide_mv_kernel, dim3(grid), dim3(kWG), kWideLds, s, d, m);
    return hipGetLastError();
  }
  const int path = i8x && (m == 1 || path_of(m, n) != kMfma) ? (int)kStaged : path_of(m, n);
  // small matvecs: shorter tiles spread them over more workgroups (batched
  // tiles stay whole 16-row groups)
  if (path == kMfma) {
    while (d.rows_per_tile > 16 && (p + d.rows_per_tile - 1) / d.rows_per_tile < 512)
      d.rows_per_tile = d.rows_per_tile % 32 == 0 ? d.rows_per_tile >> 1 : 16;
  } else {
    while (d.rows_per_tile > kRowsPerPass &&
           (p + d.rows_per_tile - 1) / d.rows_per_tile < 512)
      d.rows_per_tile >>= 1;
  }
  // one matvec at m = 1 on the staged path: the kernel for its width
  const int nbl = nbl_of(n);
  if (i8x) {
    if (m > 1) return launch_mv<false, false, true>(d, m, s);
    return nbl == 1 ? launch_mv<true, false, true, 1>(d, m, s)
           : nbl == 2 ? launch_mv<true, false, true, 2>(d, m, s)
                      : launch_mv<true, false, true, 3>(d, m, s);
  }
  const bool staged = path == kStaged || path == kMfma;
  if (m == 1) {
    if (!staged) return launch_mv<true, true, false>(d, m, s);
    return nbl == 1 ? launch_mv<true, false, false, 1>(d, m, s)
           : nbl == 2 ? launch_mv<true, false, false, 2>(d, m, s)
                      : launch_mv<true, false, false, 3>(d, m, s);
  }
  return staged ? launch_mv<false, false, false>(d, m, s)
                : launch_mv<false, true, false>(d, m, s);
}

hipError_t launch_step(const StepDesc *descs, int count, const WgGroup *groups,
                       int group_size, int m, int grid, size_t lds,
                       bool all_staged, hipStream_t s, bool i8x, const Epilogue *epi,
                       const Prologue *pro, bool dec, const PairOut *pair) {
  // prologues, epilogues and paired tiles: the decode variant (m = 1,
  // binary32), and a prologue or a pair only where every tile is staged
  if ((epi || pro || pair) && !dec) return hipErrorInvalidValue;
  if (pair && !all_staged) return hipErrorInvalidValue;
  if (dec && (m != 1 || i8x)) return hipErrorInvalidValue;
  if (pro && !all_staged) return hipErrorInvalidValue;
#define Q8_STEP(M1, ANY, I8X, DEC)                                                          \
  hipLaunchKernelGGL((step_kernel<M1, ANY, I8X, DEC>), dim3(grid), dim3(kWG), lds, s, descs, \
                     count, groups, group_size, m, epi, pro, pair)
  if (m > kMaxM) {
    if (i8x) return hipErrorInvalidValue;
    hipLaunchKernelGGL(wide_step_kernel, dim3(grid), dim3(kWG), lds, s, descs, count, groups,
                       group_size, m);
  } else if (i8x) {
    if (m == 1) Q8_STEP(true, false, true, false);
    else Q8_STEP(false, false, true, false);
  } else if (dec) {
    if (all_staged) Q8_STEP(true, false, false, true);
    else Q8_STEP(true, true, false, true);
  } else if (m == 1) {
    if (all_staged) Q8_STEP(true, false, false, false);
    else Q8_STEP(true, true, false, false);
  } else {
    if (all_staged) Q8_STEP(false, false, false, false);
    else Q8_STEP(false, true, false, false);
  }
#undef Q8_STEP
  return hipGetLastError();
}

int sliced_rows_per_tile() { return kSliceRows; }

// The tile and its partial sums (int8 activations: and x's steps, block-major).
size_t sliced_lds_bytes(bool i8x) {
  (void)i8x;  // the int8 form's steps live in the partial sums' padding
  return kSliceTileBytes + (size_t)kRedFloats * sizeof(float);
}

int sliced_step_grid(int dev, bool i8x) {
  static int cache[2][64] = {{0}};
  int &c = cache[i8x ? 1 : 0][dev & 63];
  if (!c)
    c = i8x ? resident_wgs(sliced_step_kernel<true>, sliced_lds_bytes(true), dev)
            : resident_wgs(sliced_step_kernel<false>, sliced_lds_bytes(false), dev);
  return c;
}

hipError_t launch_sliced_step(const StepDesc *descs, int count, const WgGroup *groups,
                              int group_size, int m, int grid, size_t lds, bool i8x,
                              hipStream_t s) {
  if (m < 2 || m > kMaxM) return hipErrorInvalidValue;
  if (i8x)
    hipLaunchKernelGGL(sliced_step_kernel<true>, dim3(grid), dim3(kWG), lds, s, descs, count,
                       groups, group_size, m);
  else
    hipLaunchKernelGGL(sliced_step_kernel<false>, dim3(grid), dim3(kWG), lds, s, descs, count,
                       groups, group_size, m);
  return hipGetLastError();
}

hipError_t launch_slice_sum(const SliceSum *sums, int count, int max_len, hipStream_t s) {
  if (count < 1 || max_len < 1) return hipErrorInvalidValue;
  int gx = (max_len + kWG * 4 - 1) / (kWG * 4);  // 4 outputs a thread
  gx = gx < 1 ? 1 : (gx > 64 ? 64 : gx);
  hipLaunchKernelGGL(slice_sum_kernel, dim3(gx, count), dim3(kWG), 0, s, sums, count);
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

bool split_shape_ok(int m, int n) {
  return m == 1 && n > kMaxLdsBlocks * 32 && n % 256 == 0;
}

int split_slices(int n, int32_t *sb) {
  const int32_t bpr = n >> 5;
  int32_t s = (bpr + kMaxLdsBlocks - 1) / kMaxLdsBlocks;  // slices of at most 96 blocks
  int32_t b = (bpr + s - 1) / s;
  b = (b + 7) & ~7;  // a multiple of 8 blocks: 16-byte aligned slices, staged widths
  s = (bpr + b - 1) / b;
  if (sb) *sb = b;
  return s;
}

int split_plan(int m, int n, int p, int32_t *sb) {
  if (p < 1 || !split_shape_ok(m, n)) return 0;
  return split_slices(n, sb);
}

namespace {
template <int NBLS>
int split_grid_cap(int dev) {
  static int cache[64] = {0};
  int &c = cache[dev & 63];
  if (!c)
    c = resident_wgs(mv_split_kernel<NBLS>,
                     kTileMaxBytes + (size_t)kMaxLdsBlocks * 36 * sizeof(float), dev);
  return c;
}
}  // namespace

hipError_t launch_matvec_split(const uint8_t *w, const float *x, float *y, int n, int p,
                               float *part, ArgmaxSlot *slot, int32_t *idx, hipStream_t s) {
  int32_t sb = 0;
  const int32_t slices = split_plan(1, n, p, &sb);
  if (slices < 2) return hipErrorInvalidValue;
  SliceSrc src{};
  src.base.w = w;
  src.base.x = x;
  src.base.n = n;
  src.base.p = p;
  src.part = part;
  src.slices = slices;
  src.sb = sb;
  src.pitch16 = (n >> 5) * 34 / 16;
  // rows per tile of a full-width slice, halved (down to one pass) while the
  // launch has fewer than 512 tiles
  int32_t rows = tile_rows_of(1, sb * 32);
  while (rows > kRowsPerPass && slices * ((p + rows - 1) / rows) < 512) rows >>= 1;
  src.base.rows_per_tile = rows;
  src.tps = (p + rows - 1) / rows;
  const int32_t tiles = slices * src.tps;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int nbl = nbl_of(sb * 32);
  const int cap = nbl == 1 ? split_grid_cap<1>(dev) : nbl == 2 ? split_grid_cap<2>(dev)
                                                                : split_grid_cap<3>(dev);
  const int grid = tiles < cap ? tiles : cap;
  const size_t lds = lds_bytes_for(1, sb * 32);
  if (nbl == 1) hipLaunchKernelGGL(mv_split_kernel<1>, dim3(grid), dim3(kWG), lds, s, src);
  else if (nbl == 2) hipLaunchKernelGGL(mv_split_kernel<2>, dim3(grid), dim3(kWG), lds, s, src);
  else hipLaunchKernelGGL(mv_split_kernel<3>, dim3(grid), dim3(kWG), lds, s, src);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the sums: about 8 outputs per thread, at most 512 workgroups
  int64_t per = ((int64_t)p + kWG * 8 - 1) / (kWG * 8);
  const int gx = (int)(per < 1 ? 1 : (per > 512 ? 512 : per));
  hipLaunchKernelGGL(reduce_slices, dim3(gx), dim3(kWG), 0, s, part, slices, p, y, slot, idx);
  return hipGetLastError();
}

namespace {
template <int G>
int decode_grid_of(int dev, size_t lds) {
  return resident_wgs(decode_kernel<G>, lds, dev);
}
}  // namespace

size_t attention_lds_bytes(int G) {
  switch (G) {
    case 1: return sizeof(dec::AttnLds<1>);
    case 2: return sizeof(dec::AttnLds<2>);
    case 3: return sizeof(dec::AttnLds<3>);
    default: return sizeof(dec::AttnLds<4>);
  }
}

int decode_persistent_grid(int dev, int G, size_t lds) {
  switch (G) {
    case 1: return decode_grid_of<1>(dev, lds);
    case 2: return decode_grid_of<2>(dev, lds);
    case 3: return decode_grid_of<3>(dev, lds);
    case 4: return decode_grid_of<4>(dev, lds);
    default: return 0;
  }
}

hipError_t launch_decode_persistent(const DecPhase *phases, int nphases, GridBarrier *bar,
                                    int grid, size_t lds, int G, hipStream_t s) {
  const dim3 g((unsigned)grid), b(kWG);
  switch (G) {
    case 1: hipLaunchKernelGGL(decode_kernel<1>, g, b, lds, s, phases, nphases, bar); break;
    case 2: hipLaunchKernelGGL(decode_kernel<2>, g, b, lds, s, phases, nphases, bar); break;
    case 3: hipLaunchKernelGGL(decode_kernel<3>, g, b, lds, s, phases, nphases, bar); break;
    case 4: hipLaunchKernelGGL(decode_kernel<4>, g, b, lds, s, phases, nphases, bar); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

const void *probe_kernel() { return (const void *)&argmax_rows; }

}  // namespace q8
