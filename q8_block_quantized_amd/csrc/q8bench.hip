// Measurement helper of the benchmark (not part of the decode path): a plain
// read of a device buffer with coalesced 16-byte loads, the ceiling HBM
// offers a pure read stream, against which the matvec kernels' bandwidth is
// read.  Declared in include/q8bench.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/q8bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// The buffer is cut into tiles of 256 * L 16-byte chunks (L = loads in
// flight per thread); workgroup b reads tiles b, b + G, b + 2G, ... (G the
// grid), thread t chunk t + 256 j of a tile for j < L, so each load
// instruction of a wave covers 1 KB of contiguous bytes and a tile is one
// contiguous run.  The loaded words are folded into one, stored only when
// it equals a value random data almost never gives, so the loads are kept
// and nothing else is written.
template <int L>
__global__ void __launch_bounds__(kThreads)
read_stream(const u32x4 *__restrict__ src, uint64_t chunks, uint32_t *__restrict__ sink) {
  constexpr uint64_t kTile = (uint64_t)kThreads * L;
  const uint64_t tiles = (chunks + kTile - 1) / kTile;
  uint32_t acc = 0u;
  for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint64_t base = t * kTile + threadIdx.x;
    u32x4 v[L];
    if (base + (L - 1) * (uint64_t)kThreads < chunks) {
#pragma unroll
      for (int j = 0; j < L; j++) v[j] = __builtin_nontemporal_load(src + base + j * kThreads);
    } else {
#pragma unroll
      for (int j = 0; j < L; j++) {
        const uint64_t c = base + j * kThreads;
        v[j] = c < chunks ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < L; j++) acc += v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  if (acc == 0x9E3779B9u) sink[(uint64_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int q8bench_read_stream(const void *buf, uint64_t bytes, uint32_t *sink,
                                   int32_t grid, int32_t loads, void *stream) {
  if (!buf || !sink) return 1;
  if (grid < 1 || grid > (1 << 20) || bytes % 16 != 0 || ((uintptr_t)buf & 15)) return 2;
  const hipStream_t s = (hipStream_t)stream;
  const u32x4 *src = (const u32x4 *)buf;
  const dim3 g((unsigned)grid), b(kThreads);
  switch (loads) {
    case 4: hipLaunchKernelGGL(read_stream<4>, g, b, 0, s, src, bytes / 16, sink); break;
    case 8: hipLaunchKernelGGL(read_stream<8>, g, b, 0, s, src, bytes / 16, sink); break;
    case 16: hipLaunchKernelGGL(read_stream<16>, g, b, 0, s, src, bytes / 16, sink); break;
    default: return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 7;
}
