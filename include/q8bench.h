/*
 * q8bench.h - measurement helper of the benchmark, built as libq8bench.so
 * beside libq8dec.so.  Not part of the decode path.
 */
#ifndef Q8BENCH_H
#define Q8BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of the device buffer `buf` (16-byte aligned, bytes a
 * multiple of 16) once, with coalesced 16-byte loads: the buffer is cut into
 * contiguous tiles of 256 * loads chunks of 16 bytes, dealt round-robin to
 * `grid` workgroups of 256 threads, each thread keeping `loads` (4, 8 or 16)
 * loads in flight.  Nothing is written but (with probability about 2^-32
 * per thread) one word of `sink`, a device buffer of grid * 256 uint32.
 * The HBM read ceiling the matvec kernels are set against (rvllm "Adding
 * Metal to my Rust LLM engine", "The matmul pain story": what a weight read
 * at memory speed takes).  Stream-ordered and asynchronous on `stream` (a
 * hipStream_t as void*).  Returns 0, 1 for a NULL pointer, 2 for a bad size,
 * alignment, grid (1 <= grid <= 2^20) or loads, 7 for a launch error. */
int q8bench_read_stream(const void *buf, uint64_t bytes, uint32_t *sink, int32_t grid,
                        int32_t loads, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8BENCH_H */
