// Internal interface between the C ABI (q8dec_api.hip) and the gfx950
// kernels (q8dec_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace q8 {

// One arrival group of the cross-workgroup argmax: a 64-bit key per
// activation row, an arrival counter and the number of arrivals it waits
// for (0: every workgroup of the grid arrives once, and the kernel works the
// count out itself).  The keys and the counter sit in different 128-byte
// lines, so atomics on one do not queue behind atomics on the other.
struct ArgmaxGroup {
  unsigned long long keys[32];
  unsigned int counter;
  unsigned int expected;
  unsigned int pad1[30];
};
static_assert(sizeof(ArgmaxGroup) == 384, "group layout");
static_assert(offsetof(ArgmaxGroup, counter) == 256, "counter line");

// Argmax teams.  One value for every translation unit: the slot's size and
// the offset of its `host` pointer follow from it, so the code that
// allocates a slot and the kernels that index it must agree.  The last
// arrival collects the team keys with one lane per team of a single
// 64-lane wave (argmax_arrive), so at most 64 teams can be collected and
// cleared.
constexpr int kArgmaxTeams = 32;
static_assert(kArgmaxTeams >= 1 && kArgmaxTeams <= 64,
              "the final exchange reads one team per lane of one wave");

// Argmax workspace of one matvec.  An arriving workgroup g joins team
// g % kArgmaxTeams; the last arrival of a team forwards the team's keys to
// the top group, and the last team writes the indices.  Keys and counters
// are zero between launches: the arrival that completes a group reads and
// clears them.  When `host` is set, the indices are also stored there with
// system-scope stores, so they reach host memory without a copy.
struct ArgmaxSlot {
  ArgmaxGroup top;
  ArgmaxGroup team[kArgmaxTeams];
  int32_t *host;  // device address of pinned host memory that also receives
                  // the indices, or NULL
  unsigned long long pad[7];
};

// One matvec of a launch, as the kernels see it.

struct StepDesc {
  const uint8_t *w;
  const float *x;
  float *y;
  int32_t *idx;           // fused argmax: the index output, or NULL
  ArgmaxSlot *slot;       // fused argmax: its arrival slot
  int32_t n, p;
  int32_t tile_begin;     // first tile of this matvec in the launch
  int32_t rows_per_tile;  // (paired: rows of each matrix)
  int32_t flags;          // kDescDeviceOut, kDescPairedSilu; split-K pitch
  int32_t tile_end;       // one past its last tile: tile_begin + ceil(p / rows_per_tile)
};
// y is stored with device-scope stores, so that the launch's epilogue (m = 1)
// can read it (see Epilogue); otherwise y takes plain stores.
constexpr int32_t kDescDeviceOut = 1;
// A descriptor may cover a column slice of a wider matrix (split-K): w then
// points at the slice's first block of row 0, n is the slice's width, and
// flags bits 8..23 hold the matrix's row pitch in 16-byte units.
constexpr int kDescPitchShift = 8;
__host__ __device__ inline int32_t desc_pitch16(int32_t flags) {
  return (flags >> kDescPitchShift) & 0xFFFF;
}
static_assert(sizeof(StepDesc) == 64, "descriptor layout");
// Paired (the decode step's gate and up projections, prologue form): a tile
// holds rows r0 .. r0 + rows of w and the same rows of the launch's
// PairOut::w2, both n wide over the same x; the tile's workgroup stores
// y[r] = w[r]·x, y2[r] = w2[r]·x and h[r] = silu_hadamard = y[r] / (1 +
// e^-y[r]) · y2[r].  At most one paired descriptor per launch; no argmax.
constexpr int32_t kDescPairedSilu = 2;
constexpr int kPairMaxRows = 32;  // a paired tile's rows of each matrix (plans give <= 32)
struct PairOut {
  const uint8_t *w2;  // the second matrix
  float *y2;          // its outputs
  float *h;           // silu(y) * y2
  int64_t pad;
};
static_assert(sizeof(PairOut) == 32, "pair layout");

// Workgroups g in [first, first + size) of a persistent step share the
// contiguous tile range [t0, t1), interleaved: workgroup first + j takes
// tiles t0 + j, t0 + j + size, ...  d0: the descriptor holding tile t0 (a
// start for the workgroups' descriptor search).
struct WgGroup {
  int32_t t0, t1, first, size;
  int32_t d0, pad[3];
};
static_assert(sizeof(WgGroup) == 32, "group layout");

// The first tile offset (within its group's range) of the group's j-th
// workgroup.  Workgroups are dispatched to the 8 XCDs in turn (workgroup b
// runs on XCD b % 8), so when the group is a whole number of XCD rounds the
// offsets are dealt so that consecutive tiles run on one XCD: their outputs
// share 128-byte lines, which one L2 then writes back whole.
__host__ __device__ inline int32_t group_slot(int32_t j, int32_t first, int32_t size) {
  if ((first & 7) || (size & 7)) return j;
  return (j & 7) * (size >> 3) + (j >> 3);
}

// Launches y = W x (m rows) with an optional fused argmax.  slot/idx are
// both NULL for a plain matvec.  y may be NULL only when idx is set.  i8x:
// the int8-activation variant (x quantised per 32-block; i8x_shape_ok(n)).
hipError_t launch_matvec(const uint8_t *w, const float *x, float *y, int m,
                         int n, int p, ArgmaxSlot *slot, int32_t *idx,
                         hipStream_t s, bool i8x = false);

// Widths the int8-activation variant takes: the staged ones (n/32 a
// multiple of 8, n <= 3072).
bool i8x_shape_ok(int n);

// Split-K for one activation row of a matrix wider than the staged path
// takes (n > 3072, n a multiple of 256): the columns are cut into
// split_slices(n) slices of sb blocks (a multiple of 8, at most 96; the
// last one narrower), each slice's tiles staged, each slice's partial sums
// written to part + i * p (part: split_slices(n) * p floats of device
// memory), then added in slice order into y (when set) and, when idx is set,
// the argmax taken over the sums.  Two launches on s.
bool split_shape_ok(int m, int n);
int split_slices(int n, int32_t *sb);
// split_plan(m, n, p, &sb): the slice count of a split launch (>= 2, with
// sb), or 0 for an unsplit one.  Only wide matrices split: a staged width
// with few output rows (the rvllm page's K-split of a 960 x 320 matrix, "The
// matmul pain story") was cut into slices too and measured 1.8-2.2x slower
// on MI355X, since its unsplit launch is bound by one tile's latency, not by
// idle compute units, and the split adds the summing launch.
int split_plan(int m, int n, int p, int32_t *sb);
hipError_t launch_matvec_split(const uint8_t *w, const float *x, float *y, int n, int p,
                               float *part, ArgmaxSlot *slot, int32_t *idx, hipStream_t s);

// Widths a wide batch (8 < m <= 32) takes: n a positive multiple of 256.
bool wide_shape_ok(int n);

// Launches idx[i] = argmax(logits[i][:p]) for i < m.
hipError_t launch_argmax(const float *logits, int m, int p, ArgmaxSlot *slot,
                         int32_t *idx, hipStream_t s);

// Persistent step: one launch of `grid` workgroups over the tiles of the
// `descs` table (device memory, `count` entries in tile order); workgroup g
// belongs to groups[g / group_size] (device memory).  `lds` bytes of dynamic
// LDS: step_lds_bytes of the widest matvec.
// `epi` (device memory, or NULL): work the last workgroup to finish runs
// once every tile of the launch is written (see Epilogue).
struct Epilogue;
struct Prologue;
// `dec`: the decode step's kernel variant (prologues and epilogues; m = 1,
// binary32 activations), kept apart so the other launches do not carry its
// code.
hipError_t launch_step(const StepDesc *descs, int count, const WgGroup *groups,
                       int group_size, int m, int grid, size_t lds,
                       bool all_staged, hipStream_t s, bool i8x = false,
                       const Epilogue *epi = nullptr, const Prologue *pro = nullptr,
                       bool dec = false, const PairOut *pair = nullptr);

// True when a matvec of width n with m rows takes the staged path (the step
// can then use the kernel variant without the other paths).
bool step_all_staged(int m, int n, bool i8x = false);

// Rows per tile the persistent step uses for a matvec of width n, m rows.
int step_rows_per_tile(int n, int m, bool i8x = false);

// Dynamic LDS the step needs for a matvec of width n with m rows.
size_t step_lds_bytes(int m, int n, bool i8x = false);

// Workgroups of the step kernel resident at once on `device` (the grid).
int step_grid(int device, int m, size_t lds, bool all_staged, bool i8x = false,
              bool dec = false);

// The batched persistent step in column slices (1 < m <= 8, every width
// 1024, 2048 or 3072): a matvec wider than 1024 runs as n / 1024 column
// slices of 1024, each a descriptor of its own (flags: the matrix's pitch;
// its x rows the matrix's width apart) whose y is a partial output, and a
// second launch adds the slices' partials in slice order.  Every slice is
// then as narrow as the 1024-wide matvecs, whose tiles need a third of the
// x registers and LDS, so three workgroups fit a CU instead of two.  The
// int8-activation step (i8x) is sliced the same way.
struct SliceSum {
  float *y;           // m * p outputs
  const float *part;  // k partial outputs of m * p floats, slice after slice
  int32_t k, len;     // slices, m * p
};
constexpr int kSliceWidth = 1024;
int sliced_rows_per_tile();
size_t sliced_lds_bytes(bool i8x = false);
int sliced_step_grid(int device, bool i8x = false);
hipError_t launch_sliced_step(const StepDesc *descs, int count, const WgGroup *groups,
                              int group_size, int m, int grid, size_t lds, bool i8x,
                              hipStream_t s);
hipError_t launch_slice_sum(const SliceSum *sums, int count, int max_len, hipStream_t s);

// Everything a persistent step launch needs, worked out on the host.
struct StepPlan {
  std::vector<StepDesc> descs;  // slot pointers filled in by the caller
  std::vector<WgGroup> groups;
  std::vector<std::vector<uint32_t>> expected;  // per argmax desc, per team
  size_t lds = 0;
  int grid = 0;
  int group_size = 1;
  bool all_staged = true;
  bool i8x = false;
};

// Workgroups per group of the persistent step.  m = 1: groups of 32 to 64
// streaming neighbouring tiles were fastest on MI355X (a sweep of 1..4096),
// 64 since the wave-priority and prologue changes (m = 1 step 101.0 µs
// against 102.6 µs with 32, interleaved A/B).  Batched: a workgroup reloads
// its slice of x at every new matvec, so each keeps a contiguous range of
// its own (kStepGroupSizeBatched).
constexpr int kStepGroupSize = 64;
constexpr int kStepMinTiles = 512;  // fewer: staged m = 1 tiles get shorter
constexpr int kStepMinRows = 8;                   // only heights above one pass halve
// m > 1: every workgroup its own contiguous tile range (groups of 1; with
// the wave priority by progress, 1 measured fastest of 1–512 for m = 4, 8,
// 16, 32 and int8 activations: m = 8 148 µs against 153 µs at 2)
constexpr int kStepGroupSizeBatched = 1;
// Extra weight of an argmax matvec's tiles in the step's byte balancing
// (percent): the arrival chain after the last tile (about 3 us at m = 1,
// 6 us at m = 8) measured best hidden at 3 % and 6 % (of 0, 3, 6, 10).
constexpr int kArgmaxWeightPct = 3;
constexpr int kArgmaxWeightPctBatched = 6;

// Host stub of one kernel, used to check that the code object loads.
const void *probe_kernel();

// ---- the rest of the decode step (norms, attention, SwiGLU) -------------

// Element-wise work a persistent step launch finishes with, run by the last
// workgroup to arrive (every workgroup arrives once, after its tiles):
//   kEpiAddNorm: x += r over n values (r may be NULL: no add), then
//                out = x / sqrt(mean(x^2) + eps) * g   (rms_norm_row);
//   kEpiSiluMul: out = g / (1 + e^-g) * r over n values (silu_hadamard,
//                g the gate, r the up projection).
// `arrive` is a zeroed ArgmaxSlot used only for its counters.
enum EpiOp : int32_t { kEpiNone = 0, kEpiAddNorm = 1, kEpiSiluMul = 2 };
struct Epilogue {
  int32_t op, n;
  float eps;
  int32_t pad0;
  float *x;
  const float *r;
  const float *g;
  float *out;
  ArgmaxSlot *arrive;
  int64_t pad1;
};
static_assert(sizeof(Epilogue) == 64, "epilogue layout");

// Element-wise work a persistent step launch starts with (m = 1, every tile
// staged, n <= kProMaxN): every workgroup computes the launch's x into its
// staged x while its first tile loads, and the launch's matvecs read
// x = out; workgroup 0 also stores out (and resid) in memory.
//   kProSiluMul: out = a / (1 + e^-a) * b           (silu_hadamard: a the
//                gate, b the up projection);
//   kProAddNorm: s = (a + b) + c (c may be NULL), out = s / sqrt(mean(s^2)
//                + eps) * w (rms_norm_row of the residual stream), resid
//                (or NULL) receives s.
//   kProNorm:    s = a, out = s / sqrt(mean(s^2) + eps) * w, resid (or NULL)
//                receives s (the persistent step's first layer: x = x_in).
enum ProOp : int32_t { kProNone = 0, kProSiluMul = 1, kProAddNorm = 2, kProNorm = 3 };
struct Prologue {
  int32_t op, n;
  float eps;
  int32_t pad;
  const float *a, *b, *c, *w;
  float *out, *resid;
};
static_assert(sizeof(Prologue) == 64, "prologue layout");
constexpr int kProMaxN = 3072;

constexpr int kNormMaxDim = 4096;   // widest row a norm workgroup takes
constexpr int kSiluMaxN = 65536;    // widest SwiGLU epilogue
constexpr int kAttnHeadDim = 128;   // the attention kernel's head width
constexpr int kAttnChunk = 64;      // cached rows per attention workgroup
constexpr int kAttnPart = 132;      // floats per (head, chunk) partial: m, l, pad, acc[128]
constexpr int kAttnMaxGroup = 4;    // query heads per key/value head

// attention_decode for one token (with the QK-norm, the RoPE of q and k and
// the append of k, v at row *pos folded in).  Grid n_kv * chunks workgroups,
// chunks = attn_chunks(cache_rows); workgroup (g, c) takes cached rows
// [64c, 64c + 64) of key/value head g and writes a partial softmax; the last
// workgroup of head g to finish merges them into out.
struct AttnArgs {
  const float *q, *k, *v;        // projections: [n_heads*128], [n_kv*128] x 2
  const float *q_norm, *k_norm;  // [128]
  float *kc, *vc;                // [cache_rows][n_kv*128]
  const int32_t *pos;            // device int32
  const float *rope;             // [64][2] cos, sin of pos * freq (step_start)
  const float *freq;             // [64] the RoPE frequencies (the persistent step
                                 // takes cos, sin of pos * freq itself), or NULL
  float *out;                    // [n_heads*128]
  float *part;                   // [n_heads][chunks][kAttnPart]
  ArgmaxSlot *arrive;            // [n_kv], zeroed (counters only)
  int32_t n_heads, n_kv, cache_rows, chunks;
  float eps;
};
int attn_chunks(int cache_rows);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);

// The step's first node: rope[2i], rope[2i + 1] = cos, sin of *pos * freq[i]
// for i < 64, and when x_in is set x = x_in, xn = rms_norm_row(x_in) * w
// (dim <= kNormMaxDim).
hipError_t launch_step_start(const float *x_in, const float *w, float *xn, float *x,
                             int dim, float eps, const int32_t *pos, const float *freq,
                             float *rope, hipStream_t s);

// ---- the persistent decode step ------------------------------------------
//
// One launch runs every phase of the step (per layer: q/k/v, attention, o,
// gate/up, down; then the lm_head and its argmax), workgroups meeting at a
// grid-wide barrier between phases.  Every workgroup must be resident at
// once (the grid is the kernel's resident capacity); a wait that runs past
// its limit (another workgroup never arrived) marks the barrier failed,
// stores -2 as the token and ends the workgroup, so no launch can hang.
constexpr int32_t kPhaseMatvec = 0, kPhaseAttention = 1;
struct DecPhase {
  int32_t kind;        // kPhaseMatvec or kPhaseAttention
  int32_t count;       // matvec: descriptors of the table
  int32_t group_size;  // matvec: its plan's groups of workgroups
  int32_t grid;        // matvec: workgroups with tiles (the rest only meet the barrier)
  const StepDesc *table;
  const WgGroup *groups;
  const Prologue *pro;   // or NULL
  const AttnArgs *attn;  // attention
  const PairOut *pair;   // matvec: the paired descriptor's, or NULL
  int64_t pad;
};
static_assert(sizeof(DecPhase) == 64, "phase layout");

// Grid barrier state, zeroed once (the graph's workspace): team j's arrival
// counter and released generation each in their own 128-byte line.  The
// counters only grow, so a barrier belongs to one grid size.
struct GridBarrier {
  uint32_t team[32][32];  // team j counts at [j][0]
  uint32_t top[32];
  uint32_t gen[32][32];   // the generation released to team j, at [j][0]
  uint32_t error[32];     // [0]: nonzero once a wait ran past its limit
  int32_t *idx;           // the step's token (device), -2 on failure
  int32_t *host;          // its pinned host copy, or NULL
  uint64_t pad[14];
};
constexpr int kGridTeams = 32;

// Resident workgroups of the persistent decode kernel (G query heads per
// key/value head, `lds` bytes of dynamic LDS) on `dev`.
int decode_persistent_grid(int dev, int G, size_t lds);
// LDS of one attention block with G query heads per key/value head.
size_t attention_lds_bytes(int G);
hipError_t launch_decode_persistent(const DecPhase *phases, int nphases, GridBarrier *bar,
                                    int grid, size_t lds, int G, hipStream_t s);

// freq[i] = 1 / theta^(i / 64) for i < 64, the power rounded to binary32
// from binary64 and the quotient in binary32 (the RoPE frequencies).
hipError_t launch_rope_freq(float theta, float *freq, hipStream_t s);

}  // namespace q8

struct q8_matvec_desc;
namespace q8 {
// Plans a persistent step (q8dec_api.hip) with groups of `group_size`.
// grid_cap > 0: the launch's grid (the persistent decode step's) instead of
// the step kernel's resident capacity.  paired_mask bit i: descriptor i is
// paired (kDescPairedSilu, m = 1 staged only): its tiles hold rows of two
// matrices, so they are half as tall and weigh twice the bytes; the caller
// fills w2, y2 and h and sets the flag.
// sliced: a launch of sliced_step_kernel (every descriptor 1024 wide, 1 < m
// <= 8; the caller sets each descriptor's pitch flags).
int plan_step(const q8_matvec_desc *descs, int32_t count, int32_t m, int dev,
              int group_size, StepPlan &plan, bool i8x = false, bool dec = false,
              int grid_cap = 0, uint32_t paired_mask = 0, bool sliced = false);
}  // namespace q8
