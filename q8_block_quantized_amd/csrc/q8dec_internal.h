// Internal interface between the C ABI (q8dec_api.hip) and the gfx950
// kernels (q8dec_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

// Cross-workgroup argmax workspace for one launch: one 64-bit key per
// activation row and an arrival counter.  Zero between launches: the last
// workgroup of every launch reads the keys and clears them and the counter.
struct ArgmaxSlot {
  unsigned long long keys[8];
  unsigned int counter;
  unsigned int pad[15];
};
static_assert(sizeof(ArgmaxSlot) == 128, "slot layout");

// One matvec of a persistent step, as stored in device memory.
struct StepDesc {
  const uint8_t *w;
  const float *x;
  float *y;
  int32_t *idx;
  ArgmaxSlot *slot;
  int32_t n, p;
  int32_t tile_begin;  // first global tile index of this matvec
  int32_t rows_per_tile;
};

// Launches y = W x (m rows) with an optional fused argmax.  slot/idx are
// both NULL for a plain matvec.  y may be NULL only when idx is set.
hipError_t launch_matvec(const uint8_t *w, const float *x, float *y, int m,
                         int n, int p, ArgmaxSlot *slot, int32_t *idx,
                         hipStream_t s);

// Launches idx[i] = argmax(logits[i][:p]) for i < m.
hipError_t launch_argmax(const float *logits, int m, int p, ArgmaxSlot *slot,
                         int32_t *idx, hipStream_t s);

// Persistent step: one launch over `ntiles` tiles described by `descs`
// (device memory, `count` entries, sorted by tile_begin).
hipError_t launch_step(const StepDesc *descs, int count, int ntiles, int m,
                       int grid, hipStream_t s);

// Rows per tile the persistent step uses for a matvec of width n and m rows.
int step_rows_per_tile(int n, int m);

// Workgroups the persistent step launches on this device.
int step_grid(int device);

// Host stub of one kernel, used to check that the code object loads.
const void *probe_kernel();

}  // namespace q8
