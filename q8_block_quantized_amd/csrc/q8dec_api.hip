// C ABI of libq8dec (declared in include/q8dec.h): argument validation,
// per-device set-up, launches and the decode-step graph.
//
// Error convention (after the Metal decode pages: the inferno.rs decoder
// hands back "not handled" instead of failing, and the Algenta "Metal LLM
// decode" page refuses with named status codes before any GPU work and maps
// unknown codes to an out-of-range name): every entry point checks all of its
// arguments first and returns a Q8_ERR_* code without touching the GPU when
// one is wrong.  A device that fails its set-up stays failed (the inferno.rs
// decoder slot remembers a failed start and never retries it).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <vector>

#include "../../include/q8dec.h"
#include "q8dec_internal.h"

namespace {

thread_local int g_last_hip = 0;

// Records a HIP failure for q8_last_hip_error and clears the runtime's
// sticky last-error state, so that the failure is reported once, here, and
// not again by the caller's next unrelated HIP call.
int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  (void)hipGetLastError();
  return Q8_ERR_HIP;
}

// ---- per-device state --------------------------------------------------

constexpr int kMaxDevices = 64;

// The standalone calls keep one workspace per stream they run on: an
// ArgmaxSlot for the argmax entry points, and the split-K partial sums of
// the matvecs wider than the staged path (grown as needed).  Calls on
// different streams never share one; calls on one stream are ordered by it.
// At most kMaxStreamSlots streams per device.
constexpr int kMaxStreamSlots = 256;
struct StreamSlot {
  hipStream_t stream;
  q8::ArgmaxSlot *slot;
  float *part = nullptr;
  size_t part_floats = 0;
};

struct DeviceState {
  int status = -1;                  // -1 unchecked, else a Q8 status
  std::vector<StreamSlot> slots;    // argmax workspaces by stream (null stream first)
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

// Workspace of q8_matvec_argmax_noalloc: one argmax slot (team keys and
// arrival counters for up to Q8_MAX_M activation rows), in the code
// object's own device memory, so that entry point allocates nothing.  Each
// device holds its own copy until the process ends; its address on a
// device comes from hipGetSymbolAddress at that device's set-up
// (g_scratch), never from the name in host code.  It is zero when the code
// object loads, and every launch that uses it leaves it zero again (the
// last arrival clears the keys and counters it used; `expected` and `host`
// are never written, so they stay 0 and NULL).
constexpr size_t kScratchBytes = sizeof(q8::ArgmaxSlot);
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void *g_scratch[kMaxDevices];  // per device, under g_mu

// An argmax workspace, zeroed in the order of `stream` (the stream whose
// argmax calls will use it), or, for the null stream's, before returning.
int alloc_slot(q8::ArgmaxSlot **out, hipStream_t stream, bool on_stream) {
  void *p = nullptr;
  hipError_t e = hipMalloc(&p, sizeof(q8::ArgmaxSlot));
  if (e != hipSuccess) return hip_fail(e);
  if (on_stream) {
    e = hipMemsetAsync(p, 0, sizeof(q8::ArgmaxSlot), stream);
  } else {
    e = hipMemset(p, 0, sizeof(q8::ArgmaxSlot));
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  if (e != hipSuccess) {
    (void)hipFree(p);
    return hip_fail(e);
  }
  *out = (q8::ArgmaxSlot *)p;
  return Q8_OK;
}

// The current device, checked once (gfx950, kernels loadable); allocates
// nothing.  Caller holds g_mu.
int check_device_locked(int dev) {
  DeviceState &st = g_dev[dev];
  if (st.status >= 0) return st.status;
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e);
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    st.status = Q8_ERR_ARCH;
    return st.status;
  }
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, q8::probe_kernel());
  if (e != hipSuccess) {
    hip_fail(e);
    st.status = Q8_ERR_CODE_OBJECT;
    return st.status;
  }
  // this device's copy of the no-allocation workspace (dev is current)
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    st.status = Q8_ERR_CODE_OBJECT;
    return st.status;
  }
  g_scratch[dev] = ptr;
  st.status = Q8_OK;
  return Q8_OK;
}

int current_device(int *dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return Q8_ERR_NO_DEVICE;
  }
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e);
  if (*dev < 0 || *dev >= kMaxDevices) return Q8_ERR_NO_DEVICE;
  return Q8_OK;
}

// Selects nothing: checks the current device and sets it up once (the
// null stream's argmax workspace included).
int ensure_device(int *dev_out) {
  int dev = 0;
  int st = current_device(&dev);
  if (st) return st;
  if (dev_out) *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_mu);
  if ((st = check_device_locked(dev))) return st;
  DeviceState &ds = g_dev[dev];
  if (ds.slots.empty()) {
    q8::ArgmaxSlot *slot = nullptr;
    if ((st = alloc_slot(&slot, nullptr, false))) return st;
    ds.slots.push_back(StreamSlot{nullptr, slot});
  }
  return Q8_OK;
}

// Checks the current device without allocating anything.
int check_device(int *dev_out) {
  int dev = 0;
  int st = current_device(&dev);
  if (st) return st;
  if (dev_out) *dev_out = dev;
  std::lock_guard<std::mutex> lock(g_mu);
  return check_device_locked(dev);
}

// The argmax workspace of `stream` on device dev (after ensure_device),
// allocated on the stream's first argmax call and cleared in its order.
// That first call must not be made while the stream is capturing
// (Q8_ERR_GRAPH): the clearing is not something to record into a graph.
int stream_slot(int dev, hipStream_t stream, q8::ArgmaxSlot **out) {
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState &ds = g_dev[dev];
  for (const StreamSlot &s : ds.slots)
    if (s.stream == stream) {
      *out = s.slot;
      return Q8_OK;
    }
  if ((int)ds.slots.size() >= kMaxStreamSlots) return Q8_ERR_COUNT;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e);
  if (cap != hipStreamCaptureStatusNone) return Q8_ERR_GRAPH;
  q8::ArgmaxSlot *slot = nullptr;
  int st = alloc_slot(&slot, stream, true);
  if (st) return st;
  ds.slots.push_back(StreamSlot{stream, slot});
  *out = slot;
  return Q8_OK;
}

// The split-K partial-sum buffer of `stream` on device dev (after
// stream_slot), at least `floats` long.  Growing it waits for the stream's
// work (the old buffer may still be read), and is refused with Q8_ERR_GRAPH
// while the stream is capturing.  Every partial is written before it is
// read, so the buffer needs no clearing.
int stream_part(int dev, hipStream_t stream, size_t floats, float **out) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (StreamSlot &s : g_dev[dev].slots) {
    if (s.stream != stream) continue;
    if (s.part_floats < floats) {
      hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
      hipError_t e = hipStreamIsCapturing(stream, &cap);
      if (e != hipSuccess) return hip_fail(e);
      if (cap != hipStreamCaptureStatusNone) return Q8_ERR_GRAPH;
      if (s.part) {
        if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e);
        (void)hipFree(s.part);
        s.part = nullptr;
        s.part_floats = 0;
      }
      void *p = nullptr;
      if ((e = hipMalloc(&p, floats * sizeof(float))) != hipSuccess) return hip_fail(e);
      s.part = (float *)p;
      s.part_floats = floats;
    }
    *out = s.part;
    return Q8_OK;
  }
  return Q8_ERR_HIP;  // stream_slot was not called for this stream
}

// One activation row of a matrix wider than the staged path: split-K over
// the stream's partial-sum buffer (y and/or the argmax).
int matvec_split(const void *w, const float *x, float *y, int32_t *idx, int32_t n,
                 int32_t p, hipStream_t stream) {
  int dev = 0;
  int st = ensure_device(&dev);
  if (st) return st;
  q8::ArgmaxSlot *slot = nullptr;
  if ((st = stream_slot(dev, stream, &slot))) return st;
  float *part = nullptr;
  if ((st = stream_part(dev, stream, (size_t)q8::split_plan(1, n, p, nullptr) * (size_t)p, &part)))
    return st;
  hipError_t e = q8::launch_matvec_split((const uint8_t *)w, x, y, n, p, part,
                                         idx ? slot : nullptr, idx, stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

// ---- argument checks (no HIP calls) -----------------------------------

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Shape and pointer rules shared by every matvec entry point.
int check_matvec(const void *w, const float *x, const float *y,
                 const int32_t *idx, int32_t m, int32_t n, int32_t p,
                 bool need_y) {
  if (m < 1 || m > Q8_MAX_M) return Q8_ERR_SHAPE;
  if (n < 0 || n > Q8_MAX_N || (n % Q8_BLOCK) != 0) return Q8_ERR_SHAPE;
  if (m > Q8_MAX_M_NARROW && !q8::wide_shape_ok(n)) return Q8_ERR_SHAPE;
  if (p < 0) return Q8_ERR_SHAPE;
  if (idx && p < 1) return Q8_ERR_SHAPE;
  const bool wbytes = n > 0 && p > 0;
  if ((wbytes && !w) || (n > 0 && !x)) return Q8_ERR_NULL;
  if (need_y && p > 0 && !y) return Q8_ERR_NULL;
  if ((w && !aligned(w, 16)) || (x && !aligned(x, 16))) return Q8_ERR_ALIGN;
  if ((y && !aligned(y, 4)) || (idx && !aligned(idx, 4))) return Q8_ERR_ALIGN;
  return Q8_OK;
}

// ---- step graph ----------------------------------------------------------

constexpr uint32_t kGraphMagic = 0x51384447u;  // "Q8DG"

}  // namespace

// One persistent kernel launch of a step: the descriptor table and
// workgroup ranges of its descriptors (device memory) and its shape.
// Decode graphs add attention and norm nodes (kind), or hold the one
// launch of the persistent decode step (kDecodeNode).
constexpr int kStepNode = 0, kAttnNode = 1, kNormNode = 2, kDecodeNode = 3;
// the batched step in column slices (sliced_step_kernel), then its sums
constexpr int kSlicedNode = 4, kSliceSumNode = 5;
struct SegmentLaunch {
  const q8::StepDesc *table;
  const q8::WgGroup *groups;
  int32_t count, group_size, grid;
  size_t lds;
  bool all_staged;
  int kind = kStepNode;
  const q8::Epilogue *epi = nullptr;
  const q8::Prologue *pro = nullptr;
  const q8::PairOut *pair = nullptr;  // a paired launch's second matrix and outputs
  bool dec = false;  // the decode step's kernel variant
  q8::AttnArgs attn{};
  const float *nx = nullptr, *nw = nullptr;
  float *nout = nullptr, *ncopy = nullptr;
  int32_t ndim = 0;
  float neps = 0.f;
  const int32_t *npos = nullptr;  // kNormNode: the position, the RoPE frequencies
  const float *nfreq = nullptr;   // and the cos/sin table it writes
  float *rope_out = nullptr;
  const q8::DecPhase *phases = nullptr;  // kDecodeNode: the phase table,
  int32_t nphases = 0;                   // the barrier and the query heads
  q8::GridBarrier *bar = nullptr;        // per key/value head
  int32_t heads_per_kv = 0;
  const q8::SliceSum *sums = nullptr;    // kSliceSumNode: the sliced matvecs,
  int32_t nsums = 0, sum_len = 0;        // their count and largest m * p
};

hipError_t run_segment(const SegmentLaunch &L, int m, bool i8x, hipStream_t s) {
  if (L.kind == kAttnNode) return q8::launch_attention(L.attn, s);
  if (L.kind == kSlicedNode)
    return q8::launch_sliced_step(L.table, L.count, L.groups, L.group_size, m, L.grid, L.lds,
                                  i8x, s);
  if (L.kind == kSliceSumNode) return q8::launch_slice_sum(L.sums, L.nsums, L.sum_len, s);
  if (L.kind == kDecodeNode)
    return q8::launch_decode_persistent(L.phases, L.nphases, L.bar, L.grid, L.lds,
                                        L.heads_per_kv, s);
  if (L.kind == kNormNode)
    return q8::launch_step_start(L.nx, L.nw, L.nout, L.ncopy, L.ndim, L.neps, L.npos,
                                 L.nfreq, L.rope_out, s);
  return q8::launch_step(L.table, L.count, L.groups, L.group_size, m, L.grid, L.lds,
                         L.all_staged, s, i8x, L.epi, L.pro, L.dec, L.pair);
}

struct q8_step_graph {
  uint32_t magic;
  int device;
  int mode;
  int32_t kernel_nodes;
  int32_t memcpy_nodes;
  hipGraph_t graph;
  hipGraphExec_t exec;
  void *workspace;  // argmax slots, then each segment's table and ranges
  void *act;        // decode graphs: activation buffers of the step's own
  int32_t m;
  bool i8x;
  // persistent modes: the recorded kernel launches in order, for
  // q8_step_graph_launch_kernel
  std::vector<SegmentLaunch> launches;
};

namespace {

std::set<const q8_step_graph *> g_graphs;  // live handles, guarded by g_mu

bool live_graph(const q8_step_graph *g) {
  std::lock_guard<std::mutex> lock(g_mu);
  return g && g_graphs.count(g) && g->magic == kGraphMagic;
}

void release_graph(q8_step_graph *g) {
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  if (g->workspace) (void)hipFree(g->workspace);
  if (g->act) (void)hipFree(g->act);
  g->magic = 0;
  delete g;
}

int count_nodes(q8_step_graph *g) {
  size_t num = 0;
  hipError_t e = hipGraphGetNodes(g->graph, nullptr, &num);
  if (e != hipSuccess) return hip_fail(e);
  std::vector<hipGraphNode_t> nodes(num);
  if (num) {
    e = hipGraphGetNodes(g->graph, nodes.data(), &num);
    if (e != hipSuccess) return hip_fail(e);
  }
  g->kernel_nodes = 0;
  g->memcpy_nodes = 0;
  for (size_t i = 0; i < num; i++) {
    hipGraphNodeType t;
    e = hipGraphNodeGetType(nodes[i], &t);
    if (e != hipSuccess) return hip_fail(e);
    if (t == hipGraphNodeTypeKernel) g->kernel_nodes++;
    if (t == hipGraphNodeTypeMemcpy) g->memcpy_nodes++;
  }
  return Q8_OK;
}

}  // namespace

namespace q8 {

// Plans a persistent step: tiles per descriptor (in descriptor order), the
// dynamic LDS (staged tile and the widest x), the grid (the
// resident workgroups, at most one per tile), groups of `group_size`
// workgroups with contiguous tile ranges of about equal weight bytes, and
// for every argmax descriptor the arrivals each argmax team waits for.
int plan_step(const q8_matvec_desc *descs, int32_t count, int32_t m, int dev,
              int group_size, StepPlan &plan, bool i8x, bool dec, int grid_cap,
              uint32_t paired_mask, bool sliced) {
  auto paired = [&](int32_t i) { return i < 32 && ((paired_mask >> i) & 1u); };
  if (paired_mask && (m != 1 || i8x || count > 32)) return Q8_ERR_SHAPE;
  if (sliced && (m < 2 || m > Q8_MAX_M_NARROW || dec || paired_mask))
    return Q8_ERR_SHAPE;
  plan.descs.assign(count, StepDesc());
  plan.all_staged = true;
  plan.i8x = i8x;
  int64_t tiles = 0;
  size_t widest = 0;
  for (int32_t i = 0; i < count; i++) {
    const q8_matvec_desc &d = descs[i];
    StepDesc &t = plan.descs[i];
    std::memset(&t, 0, sizeof(t));
    t.w = (const uint8_t *)d.w;
    t.x = d.x;
    t.y = d.y;
    t.idx = d.idx;
    t.n = d.n;
    t.p = d.p;
    if (sliced && d.n != kSliceWidth) return Q8_ERR_SHAPE;
    t.rows_per_tile = sliced ? sliced_rows_per_tile() : step_rows_per_tile(d.n, m, i8x);
    if (paired(i)) {
      if (!step_all_staged(1, d.n, false)) return Q8_ERR_SHAPE;
      t.rows_per_tile = t.rows_per_tile / 2 > 0 ? t.rows_per_tile / 2 : 1;
    }
    t.tile_begin = (int32_t)tiles;
    tiles += (d.p + t.rows_per_tile - 1) / t.rows_per_tile;
    if (tiles > 0x7FFFFFFF) return Q8_ERR_SHAPE;
    t.tile_end = (int32_t)tiles;
    const size_t l = sliced ? sliced_lds_bytes(i8x) : step_lds_bytes(m, d.n, i8x);
    if (l > widest) widest = l;
    plan.all_staged = plan.all_staged && (sliced || step_all_staged(m, d.n, i8x));
  }
  if (tiles < 1) return Q8_ERR_SHAPE;  // nothing to run
  if (grid_cap > 0 && m == 1 && !i8x && plan.all_staged) {
    // The persistent decode step's phases: the least tile height h that
    // leaves at most one tile per workgroup of the grid (each phase then
    // costs one tile's latency), or the staged maximum where that is lower.
    int64_t rows = 0, hmax = 1;
    for (int32_t i = 0; i < count; i++) {
      rows += descs[i].p;
      hmax = plan.descs[i].rows_per_tile > hmax ? plan.descs[i].rows_per_tile : hmax;
    }
    int64_t h = (rows + grid_cap - 1) / grid_cap;
    if (h < 1) h = 1;
    for (;; h++) {
      int64_t nt = 0;
      for (int32_t i = 0; i < count; i++) {
        const int64_t r = h < plan.descs[i].rows_per_tile ? h : plan.descs[i].rows_per_tile;
        nt += (descs[i].p + r - 1) / r;
      }
      if (nt <= grid_cap || h >= hmax) break;
    }
    tiles = 0;
    for (int32_t i = 0; i < count; i++) {
      StepDesc &t = plan.descs[i];
      if (h < t.rows_per_tile) t.rows_per_tile = (int32_t)h;
      t.tile_begin = (int32_t)tiles;
      tiles += (t.p + t.rows_per_tile - 1) / t.rows_per_tile;
      t.tile_end = (int32_t)tiles;
    }
  } else if (m == 1 && !i8x && plan.all_staged) {
    // A launch of few tiles (the decode step's levels) spreads them over more
    // workgroups: staged m = 1 tile heights above one pass (8 rows) halve
    // until there are at least kStepMinTiles (as standalone matvecs do).
    while (tiles < kStepMinTiles) {
      bool changed = false;
      tiles = 0;
      for (int32_t i = 0; i < count; i++) {
        StepDesc &t = plan.descs[i];
        if (t.rows_per_tile > (paired(i) ? kStepMinRows / 2 : kStepMinRows)) {
          t.rows_per_tile >>= 1;
          changed = true;
        }
        t.tile_begin = (int32_t)tiles;
        tiles += (t.p + t.rows_per_tile - 1) / t.rows_per_tile;
        t.tile_end = (int32_t)tiles;
      }
      if (!changed) break;
    }
  }
  const int32_t ntiles = (int32_t)tiles;
  plan.lds = widest;
  if (i8x && !plan.all_staged) return Q8_ERR_SHAPE;
  int grid = grid_cap > 0 ? grid_cap
             : sliced   ? sliced_step_grid(dev, i8x)
                        : step_grid(dev, m, plan.lds, plan.all_staged, i8x, dec);
  if (grid > ntiles) grid = ntiles;
  if (grid < 1) grid = 1;
  if (group_size < 1) group_size = 1;
  if (group_size > grid) group_size = grid;
  plan.grid = grid;
  plan.group_size = group_size;
  // prefix sums of tile weight bytes.  An argmax matvec's tiles count
  // kArgmaxWeightPct % more (kArgmaxWeightPctBatched for m > 1): the
  // workgroups holding them end with the arrival chain after their last
  // tile, so they get that much less to stream and the chain overlaps the
  // others' last tiles.
  std::vector<int64_t> pre((size_t)ntiles + 1, 0);
  const int64_t argmax_pct = 100 + (m > 1 ? kArgmaxWeightPctBatched : kArgmaxWeightPct);
  for (int32_t i = 0, t = 0; i < count; i++) {
    const StepDesc &d = plan.descs[i];
    const int64_t pitch = (int64_t)(d.n / 32) * 34 * (paired(i) ? 2 : 1);
    const int64_t pct = d.idx ? argmax_pct : 100;
    for (int32_t r0 = 0; r0 < d.p; r0 += d.rows_per_tile, t++) {
      const int32_t rows = d.p - r0 < d.rows_per_tile ? d.p - r0 : d.rows_per_tile;
      pre[t + 1] = pre[t] + rows * pitch * pct / 100 + 1;  // +1: zero-width tiles still count
    }
  }
  const int ngroups = (grid + group_size - 1) / group_size;
  plan.groups.resize(ngroups);
  int32_t prev_end = 0;
  for (int a = 0; a < ngroups; a++) {
    WgGroup &gr = plan.groups[a];
    gr.first = a * group_size;
    gr.size = grid - gr.first < group_size ? grid - gr.first : group_size;
    gr.t0 = prev_end;
    const int64_t target =
        (int64_t)((__int128)pre[ntiles] * (gr.first + gr.size) / grid);
    int32_t e = a == ngroups - 1
                    ? ntiles
                    : (int32_t)(std::lower_bound(pre.begin(), pre.end(), target) -
                                pre.begin());
    if (e < gr.t0) e = gr.t0;
    gr.t1 = e;
    prev_end = e;
    // the last descriptor starting at or before t0 (empty ones skipped)
    gr.d0 = 0;
    for (int32_t i = 0; i < count; i++)
      if (plan.descs[i].tile_begin <= gr.t0) gr.d0 = i;
  }
  // arrivals of each argmax descriptor, by team
  plan.expected.clear();
  for (int32_t i = 0; i < count; i++) {
    const StepDesc &d = plan.descs[i];
    if (!d.idx) continue;
    std::vector<uint32_t> team(kArgmaxTeams, 0);
    const int32_t tb = d.tile_begin, te = tb + (d.p + d.rows_per_tile - 1) / d.rows_per_tile;
    for (const WgGroup &gr : plan.groups) {
      const int32_t u = gr.t0 > tb ? gr.t0 : tb, v = gr.t1 < te ? gr.t1 : te;
      if (u >= v) continue;
      for (int32_t j = 0; j < gr.size; j++) {
        int32_t t = gr.t0 + group_slot(j, gr.first, gr.size);
        if (t < u) t += (u - t + gr.size - 1) / gr.size * gr.size;
        if (t < v) team[(gr.first + j) % kArgmaxTeams]++;
      }
    }
    plan.expected.push_back(team);
  }
  return Q8_OK;
}

}  // namespace q8

namespace {

}  // namespace

extern "C" {

const char *q8_status_name(int status) {
  switch (status) {
    case Q8_OK: return "q8_ok";
    case Q8_ERR_NULL: return "q8_err_null";
    case Q8_ERR_SHAPE: return "q8_err_shape";
    case Q8_ERR_ALIGN: return "q8_err_align";
    case Q8_ERR_NO_DEVICE: return "q8_err_no_device";
    case Q8_ERR_ARCH: return "q8_err_arch";
    case Q8_ERR_CODE_OBJECT: return "q8_err_code_object";
    case Q8_ERR_HIP: return "q8_err_hip";
    case Q8_ERR_GRAPH: return "q8_err_graph";
    case Q8_ERR_BAD_HANDLE: return "q8_err_bad_handle";
    case Q8_ERR_COUNT: return "q8_err_count";
    case Q8_ERR_MODE: return "q8_err_mode";
    case Q8_ERR_LEVELS: return "q8_err_levels";
    default: return "q8_code_out_of_range";
  }
}

int q8_last_hip_error(void) { return g_last_hip; }

int q8_device_count(int32_t *count) {
  if (!count) return Q8_ERR_NULL;
  int c = 0;
  if (hipGetDeviceCount(&c) != hipSuccess) {
    (void)hipGetLastError();
    c = 0;
  }
  *count = c;
  return Q8_OK;
}

int q8_init(void) { return ensure_device(nullptr); }

int q8_matvec(const void *w, const float *x, float *y, int32_t n, int32_t p,
              void *stream) {
  int st = check_matvec(w, x, y, nullptr, 1, n, p, true);
  if (st) return st;
  if (q8::split_plan(1, n, p, nullptr) > 1)
    return matvec_split(w, x, y, nullptr, n, p, (hipStream_t)stream);
  if ((st = ensure_device(nullptr))) return st;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y, 1, n, p, nullptr,
                                   nullptr, (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_matvec_batched(const void *w, const float *x, float *y, int32_t m,
                      int32_t n, int32_t p, void *stream) {
  int st = check_matvec(w, x, y, nullptr, m, n, p, true);
  if (st) return st;
  if (q8::split_plan(m, n, p, nullptr) > 1)
    return matvec_split(w, x, y, nullptr, n, p, (hipStream_t)stream);
  if ((st = ensure_device(nullptr))) return st;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y, m, n, p, nullptr,
                                   nullptr, (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_argmax(const float *logits, int32_t m, int32_t p, int32_t *idx,
              void *stream) {
  if (m < 1 || m > Q8_MAX_M || p < 1) return Q8_ERR_SHAPE;
  if (!logits || !idx) return Q8_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(idx, 4)) return Q8_ERR_ALIGN;
  int dev = 0;
  int st = ensure_device(&dev);
  if (st) return st;
  q8::ArgmaxSlot *slot = nullptr;
  if ((st = stream_slot(dev, (hipStream_t)stream, &slot))) return st;
  hipError_t e = q8::launch_argmax(logits, m, p, slot, idx, (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_matvec_argmax(const void *w, const float *x, float *y_or_null,
                     int32_t *idx, int32_t m, int32_t n, int32_t p,
                     void *stream) {
  if (!idx) return Q8_ERR_NULL;
  int st = check_matvec(w, x, y_or_null, idx, m, n, p, false);
  if (st) return st;
  if (q8::split_plan(m, n, p, nullptr) > 1)
    return matvec_split(w, x, y_or_null, idx, n, p, (hipStream_t)stream);
  int dev = 0;
  if ((st = ensure_device(&dev))) return st;
  q8::ArgmaxSlot *slot = nullptr;
  if ((st = stream_slot(dev, (hipStream_t)stream, &slot))) return st;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y_or_null, m, n, p,
                                   slot, idx, (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_matvec_argmax_noalloc(const void *w, const float *x, float *y_or_null,
                             int32_t *idx, int32_t m, int32_t n, int32_t p,
                             void *stream) {
  if (!idx) return Q8_ERR_NULL;
  // m <= Q8_MAX_M is also the scratch's limit: one key per row per group
  int st = check_matvec(w, x, y_or_null, idx, m, n, p, false);
  if (st) return st;
  static_assert(sizeof(q8::ArgmaxSlot) <= kScratchBytes, "one slot fits the scratch");
  int dev = 0;
  if ((st = check_device(&dev))) return st;
  q8::ArgmaxSlot *slot = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    slot = (q8::ArgmaxSlot *)g_scratch[dev];
  }
  if (!slot) return Q8_ERR_CODE_OBJECT;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y_or_null, m, n, p, slot, idx,
                                   (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_matvec_i8x(const void *w, const float *x, float *y, int32_t m, int32_t n,
                  int32_t p, void *stream) {
  int st = check_matvec(w, x, y, nullptr, m, n, p, true);
  if (st) return st;
  if (m > Q8_MAX_M_NARROW || (n > 0 && !q8::i8x_shape_ok(n))) return Q8_ERR_SHAPE;
  if ((st = ensure_device(nullptr))) return st;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y, m, n, p, nullptr,
                                   nullptr, (hipStream_t)stream, n > 0);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_matvec_argmax_i8x(const void *w, const float *x, float *y_or_null,
                         int32_t *idx, int32_t m, int32_t n, int32_t p,
                         void *stream) {
  if (!idx) return Q8_ERR_NULL;
  int st = check_matvec(w, x, y_or_null, idx, m, n, p, false);
  if (st) return st;
  if (m > Q8_MAX_M_NARROW || (n > 0 && !q8::i8x_shape_ok(n))) return Q8_ERR_SHAPE;
  int dev = 0;
  if ((st = ensure_device(&dev))) return st;
  q8::ArgmaxSlot *slot = nullptr;
  if ((st = stream_slot(dev, (hipStream_t)stream, &slot))) return st;
  hipError_t e = q8::launch_matvec((const uint8_t *)w, x, y_or_null, m, n, p,
                                   slot, idx, (hipStream_t)stream, n > 0);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

namespace {

// Records what `record` enqueues into g's graph on a capture stream,
// instantiates it and registers the handle in *out; releases g on failure.
extern "C++" {
template <class F>
int capture_graph(q8_step_graph *g, q8_step_graph **out, F record) {
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) {
    release_graph(g);
    return hip_fail(e);
  }
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  hipError_t le = hipSuccess;
  if (e == hipSuccess) {
    le = record(cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    g->graph = graph;
  }
  (void)hipStreamDestroy(cs);
  if (le != hipSuccess || e != hipSuccess || !g->graph) {
    hip_fail(le != hipSuccess ? le : e);
    release_graph(g);
    return Q8_ERR_GRAPH;
  }
  e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hip_fail(e);
    release_graph(g);
    return Q8_ERR_GRAPH;
  }
  int st = count_nodes(g);
  if (st) {
    release_graph(g);
    return st;
  }
  {
    std::lock_guard<std::mutex> lock(g_mu);
    g_graphs.insert(g);
  }
  *out = g;
  return Q8_OK;
}
}  // extern "C++"

// Device memory freed on scope exit unless released.
struct DevBuf {
  void *p = nullptr;
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  void *release() {
    void *r = p;
    p = nullptr;
    return r;
  }
};

// Builds every form of step graph.  levels (Q8_GRAPH_LEVELS only) gives each
// descriptor's dependency level; each run of equal levels becomes one
// persistent kernel node, the nodes in level order.
int build_graph(const q8_matvec_desc *descs, const int32_t *levels, int32_t count,
                int32_t m, int32_t *host_idx, int32_t mode, q8_step_graph **out) {
  if (!out) return Q8_ERR_NULL;
  *out = nullptr;  // on every failure the caller holds no handle
  if (!descs) return Q8_ERR_NULL;
  if (count < 1 || count > Q8_MAX_DESCS) return Q8_ERR_COUNT;
  if (mode != Q8_GRAPH_CHAIN && mode != Q8_GRAPH_PERSISTENT &&
      mode != Q8_GRAPH_PERSISTENT_I8X && mode != Q8_GRAPH_LEVELS)
    return Q8_ERR_MODE;
  if (m < 1 || m > Q8_MAX_M) return Q8_ERR_SHAPE;
  if (mode == Q8_GRAPH_LEVELS) {
    if (!levels) return Q8_ERR_NULL;
    for (int32_t i = 0; i < count; i++)
      if (levels[i] < 0 || (i && levels[i] < levels[i - 1])) return Q8_ERR_LEVELS;
  }
  const bool i8x = mode == Q8_GRAPH_PERSISTENT_I8X;
  const bool persistent = mode != Q8_GRAPH_CHAIN;
  int nargmax = 0;
  for (int32_t i = 0; i < count; i++) {
    const q8_matvec_desc &d = descs[i];
    int st = check_matvec(d.w, d.x, d.y, d.idx, m, d.n, d.p, d.idx == nullptr);
    if (st) return st;
    if (i8x && (m > Q8_MAX_M_NARROW || !q8::i8x_shape_ok(d.n))) return Q8_ERR_SHAPE;
    if (d.idx) nargmax++;
  }
  if (nargmax > Q8_MAX_ARGMAX_DESCS) return Q8_ERR_COUNT;
  if (host_idx && !aligned(host_idx, 4)) return Q8_ERR_ALIGN;
  int dev = 0;
  int st = ensure_device(&dev);
  if (st) return st;
  // the kernels store the indices straight into the pinned host buffer
  int32_t *host_dev = nullptr;
  if (host_idx) {
    hipError_t he = hipHostGetDevicePointer((void **)&host_dev, host_idx, 0);
    if (he != hipSuccess || !host_dev) return hip_fail(he != hipSuccess ? he : hipErrorInvalidValue);
  }

  // The batched persistent step in column slices (q8::SliceSum), binary32 or
  // int8 activations: every width 1024, 2048 or 3072, no argmax on a wider
  // matvec.  `ex` then holds the
  // launch's descriptors (a wider matvec's slices in its place, their y
  // partial outputs in `part`), and `sums` the second launch's table.
  bool sliced = (mode == Q8_GRAPH_PERSISTENT || i8x) && m >= 2 && m <= Q8_MAX_M_NARROW;
  for (int32_t i = 0; i < count && sliced; i++) {
    const q8_matvec_desc &d = descs[i];
    if (d.n != 1024 && d.n != 2048 && d.n != 3072) sliced = false;
    else if (d.n > 1024 && (d.idx || (int64_t)m * d.p > 0x7FFFFFFF)) sliced = false;
  }
  std::vector<q8_matvec_desc> ex;
  std::vector<int32_t> ex_pitch16;
  std::vector<q8::SliceSum> sums;
  int32_t sum_len = 0;
  DevBuf part;
  if (sliced) {
    size_t part_floats = 0;
    for (int32_t i = 0; i < count; i++)
      if (descs[i].n > q8::kSliceWidth)
        part_floats += (size_t)(descs[i].n / q8::kSliceWidth) * (size_t)m * (size_t)descs[i].p;
    if (part_floats) {
      hipError_t pe = hipMalloc(&part.p, part_floats * sizeof(float));
      if (pe != hipSuccess) return hip_fail(pe);
    }
    float *pb = (float *)part.p;
    size_t off = 0;
    for (int32_t i = 0; i < count; i++) {
      const q8_matvec_desc &d = descs[i];
      const int32_t pitch16 = d.n / 32 * 34 / 16;
      if (d.n == q8::kSliceWidth) {
        ex.push_back(d);
        ex_pitch16.push_back(pitch16);
        continue;
      }
      const int32_t k = d.n / q8::kSliceWidth;
      const size_t len = (size_t)m * (size_t)d.p;
      for (int32_t sl = 0; sl < k; sl++) {
        q8_matvec_desc sd = d;
        sd.w = (const uint8_t *)d.w + (size_t)sl * (q8::kSliceWidth / 32) * 34;
        sd.x = d.x + (size_t)sl * q8::kSliceWidth;
        sd.y = len ? pb + off + (size_t)sl * len : nullptr;
        sd.n = q8::kSliceWidth;
        ex.push_back(sd);
        ex_pitch16.push_back(pitch16);
      }
      if (len) {
        sums.push_back(q8::SliceSum{d.y, pb + off, k, (int32_t)len});
        off += (size_t)k * len;
        sum_len = (int32_t)len > sum_len ? (int32_t)len : sum_len;
      }
    }
    if ((int64_t)ex.size() > Q8_MAX_DESCS) sliced = false;  // (the unsliced plan then)
  }
  const q8_matvec_desc *pdescs = sliced ? ex.data() : descs;
  const int32_t pcount = sliced ? (int32_t)ex.size() : count;

  // persistent segments: all descriptors, or each run of one level
  struct Segment {
    int32_t begin, end;
    q8::StepPlan plan;
  };
  std::vector<Segment> segs;
  if (persistent && sliced) {
    segs.push_back(Segment{0, pcount, q8::StepPlan()});
    st = q8::plan_step(pdescs, pcount, m, dev, q8::kStepGroupSizeBatched, segs[0].plan, i8x,
                       false, 0, 0u, true);
    if (st) return st;
    for (int32_t i = 0; i < pcount; i++)
      segs[0].plan.descs[i].flags |= ex_pitch16[i] << q8::kDescPitchShift;
  } else if (persistent) {
    for (int32_t i = 0; i < count;) {
      int32_t j = i + 1;
      if (mode == Q8_GRAPH_LEVELS) {
        while (j < count && levels[j] == levels[i]) j++;
      } else {
        j = count;
      }
      segs.push_back(Segment{i, j, q8::StepPlan()});
      i = j;
    }
    for (auto &sg : segs) {
      st = q8::plan_step(descs + sg.begin, sg.end - sg.begin, m, dev,
                         m == 1 ? q8::kStepGroupSize : q8::kStepGroupSizeBatched,
                         sg.plan, i8x);
      if (st) return st;
    }
  }

  q8_step_graph *g = new (std::nothrow) q8_step_graph();
  if (!g) return Q8_ERR_GRAPH;
  g->magic = kGraphMagic;
  g->device = dev;
  g->mode = mode;
  g->m = m;
  g->i8x = i8x;

  // workspace: one argmax slot per argmax descriptor, then each segment's
  // descriptor table and workgroup ranges (16-byte aligned pieces)
  const size_t slot_bytes = (size_t)(nargmax ? nargmax : 1) * sizeof(q8::ArgmaxSlot);
  size_t total = slot_bytes;
  std::vector<size_t> table_off, group_off;
  for (auto &sg : segs) {
    table_off.push_back(total);
    total += sg.plan.descs.size() * sizeof(q8::StepDesc);
    group_off.push_back(total);
    total += (sg.plan.groups.size() * sizeof(q8::WgGroup) + 15) & ~(size_t)15;
  }
  const size_t sums_off = total;  // the sliced step's sums table
  total += (sums.size() * sizeof(q8::SliceSum) + 15) & ~(size_t)15;
  g->act = part.release();  // (freed with the graph)
  hipError_t e = hipMalloc(&g->workspace, total);
  if (e == hipSuccess) e = hipMemset(g->workspace, 0, total);
  if (e != hipSuccess) {
    release_graph(g);
    return hip_fail(e);
  }
  char *ws = (char *)g->workspace;
  q8::ArgmaxSlot *slots = (q8::ArgmaxSlot *)ws;
  {
    // argmax slots: keys and counters zero, arrival counts from the plans
    // (the chain's kernels count their own grids), host copy of argmax
    // descriptor a (in descriptor order) at host_idx + a * m
    std::vector<q8::ArgmaxSlot> hs(nargmax ? nargmax : 1);
    std::memset(hs.data(), 0, hs.size() * sizeof(q8::ArgmaxSlot));
    for (int a = 0; a < nargmax; a++)
      hs[a].host = host_dev ? host_dev + (size_t)a * m : nullptr;
    int a = 0;
    for (auto &sg : segs) {
      int k = 0;
      for (auto &t : sg.plan.descs) {
        if (!t.idx) continue;
        uint32_t nteams = 0;
        for (int j = 0; j < q8::kArgmaxTeams; j++) {
          hs[a].team[j].expected = sg.plan.expected[k][j];
          nteams += sg.plan.expected[k][j] ? 1u : 0u;
        }
        hs[a].top.expected = nteams;
        t.slot = &slots[a++];
        k++;
      }
    }
    e = hipMemcpy(slots, hs.data(), slot_bytes, hipMemcpyHostToDevice);
    for (size_t i = 0; i < segs.size() && e == hipSuccess; i++) {
      const q8::StepPlan &pl = segs[i].plan;
      e = hipMemcpy(ws + table_off[i], pl.descs.data(),
                    pl.descs.size() * sizeof(q8::StepDesc), hipMemcpyHostToDevice);
      if (e == hipSuccess)
        e = hipMemcpy(ws + group_off[i], pl.groups.data(),
                      pl.groups.size() * sizeof(q8::WgGroup), hipMemcpyHostToDevice);
      // the table's own length (the planner may hand back a table of another
      // length than the segment's matvecs)
      g->launches.push_back(SegmentLaunch{
          (const q8::StepDesc *)(ws + table_off[i]), (const q8::WgGroup *)(ws + group_off[i]),
          (int32_t)pl.descs.size(), pl.group_size, pl.grid, pl.lds, pl.all_staged});
      if (sliced) g->launches.back().kind = kSlicedNode;
    }
    if (sliced && !sums.empty() && e == hipSuccess) {
      e = hipMemcpy(ws + sums_off, sums.data(), sums.size() * sizeof(q8::SliceSum),
                    hipMemcpyHostToDevice);
      SegmentLaunch L{nullptr, nullptr, 0, 0, 0, 0, true};
      L.kind = kSliceSumNode;
      L.sums = (const q8::SliceSum *)(ws + sums_off);
      L.nsums = (int32_t)sums.size();
      L.sum_len = sum_len;
      g->launches.push_back(L);
    }
    if (e != hipSuccess) {
      release_graph(g);
      return hip_fail(e);
    }
  }

  if (mode == Q8_GRAPH_CHAIN) {
    return capture_graph(g, out, [&](hipStream_t cs) {
      hipError_t le = hipSuccess;
      int a = 0;
      for (int32_t i = 0; i < count && le == hipSuccess; i++) {
        const q8_matvec_desc &d = descs[i];
        q8::ArgmaxSlot *slot = d.idx ? &slots[a++] : nullptr;
        le = q8::launch_matvec((const uint8_t *)d.w, d.x, d.y, m, d.n, d.p,
                               slot, d.idx, cs);
      }
      return le;
    });
  }
  return capture_graph(g, out, [&](hipStream_t cs) {
    hipError_t le = hipSuccess;
    for (size_t i = 0; i < g->launches.size() && le == hipSuccess; i++)
      le = run_segment(g->launches[i], m, i8x, cs);
    return le;
  });
}

bool ok16(const void *p) { return p && aligned(p, 16); }

// The whole decode step: argument checks, then the plans, the workspace and
// the node list (norm; per layer q/k/v, attention, o + add + norm, gate/up +
// SwiGLU, down + add + norm; lm_head argmax), or the phase table of the
// persistent form, then the capture.
int build_decode(const q8_decode_model *md, const q8_decode_buffers *bf, int32_t *host_token,
                 q8_step_graph **out) {
  if (!out) return Q8_ERR_NULL;
  *out = nullptr;
  if (!md || !bf) return Q8_ERR_NULL;
  const q8_decode_model &M = *md;
  const q8_decode_buffers &B = *bf;
  const int64_t qw = (int64_t)M.n_heads * M.head_dim, kvw = (int64_t)M.n_kv_heads * M.head_dim;
  if (M.n_layers < 1 || M.n_layers > Q8_MAX_DESCS / 8) return Q8_ERR_SHAPE;
  if (M.head_dim != q8::kAttnHeadDim) return Q8_ERR_SHAPE;
  if (M.n_kv_heads < 1 || M.n_heads < M.n_kv_heads || M.n_heads % M.n_kv_heads ||
      M.n_heads / M.n_kv_heads > q8::kAttnMaxGroup || qw > Q8_MAX_N || kvw > Q8_MAX_N)
    return Q8_ERR_SHAPE;
  if (M.hidden < Q8_BLOCK || M.hidden > q8::kNormMaxDim || M.hidden % Q8_BLOCK)
    return Q8_ERR_SHAPE;
  if (M.inter < Q8_BLOCK || M.inter > Q8_MAX_N || M.inter % Q8_BLOCK) return Q8_ERR_SHAPE;
  if (M.vocab < 1 || M.cache_rows < 1 || M.cache_rows > 65536) return Q8_ERR_SHAPE;
  if (!(M.eps >= 0.f) || !(M.eps < INFINITY) || !(M.theta > 0.f) || !(M.theta < INFINITY))
    return Q8_ERR_SHAPE;
  if (!M.layers || !M.out_norm || !M.lm_head) return Q8_ERR_NULL;
  const void *need[] = {B.x_in, B.x, B.xn, B.q, B.k, B.v, B.attn, B.attn_out, B.xn2,
                        B.gate, B.up, B.h, B.ffn_out, B.xf, M.out_norm, M.lm_head};
  for (const void *p : need) {
    if (!p) return Q8_ERR_NULL;
    if (!aligned(p, 16)) return Q8_ERR_ALIGN;
  }
  if (!B.pos || !B.token) return Q8_ERR_NULL;
  if (!aligned(B.pos, 4) || !aligned(B.token, 4)) return Q8_ERR_ALIGN;
  if (B.logits && !aligned(B.logits, 16)) return Q8_ERR_ALIGN;
  for (int32_t l = 0; l < M.n_layers; l++) {
    const q8_decode_layer &L = M.layers[l];
    const void *lp[] = {L.wq, L.wk, L.wv, L.wo, L.w_gate, L.w_up, L.w_down, L.attn_norm,
                        L.ffn_norm, L.q_norm, L.k_norm, L.k_cache, L.v_cache};
    for (const void *p : lp) {
      if (!p) return Q8_ERR_NULL;
      if (!aligned(p, 16)) return Q8_ERR_ALIGN;
    }
  }
  if (host_token && !aligned(host_token, 4)) return Q8_ERR_ALIGN;
  if (M.form != Q8_DECODE_NODES && M.form != Q8_DECODE_PERSISTENT) return Q8_ERR_MODE;
  const bool pers = M.form == Q8_DECODE_PERSISTENT;
  const int G = M.n_heads / M.n_kv_heads;
  int dev = 0;
  int st = ensure_device(&dev);
  if (st) return st;
  int32_t *host_dev = nullptr;
  if (host_token) {
    hipError_t he = hipHostGetDevicePointer((void **)&host_dev, host_token, 0);
    if (he != hipSuccess || !host_dev) return hip_fail(he != hipSuccess ? he : hipErrorInvalidValue);
  }

  const int H = M.hidden, QW = (int)qw, KVW = (int)kvw, I = M.inter;
  // Activation buffers.  The node form uses the caller's for every layer
  // (kernel boundaries order each write before the next read), with the
  // residual stream after layer l, R_l, alternating between buf->x and a
  // buffer of its own so that a launch never overwrites what its own
  // workgroups read: R_l lives in buf->x when L - 1 - l is even (l = -1, the
  // step's input, is copied there by the first launch), so the last is in
  // buf->x.  The persistent form gives layers 0 .. L-2 their own buffers and
  // R_{-1} .. R_{L-2} one each (the last layer and R_{L-1} use the caller's),
  // so that the launch writes every buffer once (see decode_kernel).
  struct LayerBufs {
    float *xn, *q, *k, *v, *attn, *attn_out, *xn2, *gate, *up, *h, *ffn_out;
  };
  std::vector<LayerBufs> lb(M.n_layers, LayerBufs{B.xn, B.q, B.k, B.v, B.attn, B.attn_out,
                                                  B.xn2, B.gate, B.up, B.h, B.ffn_out});
  std::vector<float *> rs(M.n_layers + 1, B.x);  // rs[l + 1] = R_l
  DevBuf act;
  {
    auto fl = [](int64_t n) { return (size_t)((n + 63) & ~(int64_t)63); };  // 256-byte pieces
    const size_t per_layer = 4 * fl(H) + 2 * fl(QW) + 2 * fl(KVW) + 3 * fl(I);
    const size_t floats = pers ? (size_t)(M.n_layers - 1) * per_layer + (size_t)M.n_layers * fl(H)
                               : fl(H);
    hipError_t e = hipMalloc(&act.p, floats * sizeof(float));
    if (e != hipSuccess) return hip_fail(e);
    float *f = (float *)act.p;
    auto take_f = [&](int64_t n) {
      float *r = f;
      f += fl(n);
      return r;
    };
    if (pers) {
      for (int32_t l = 0; l + 1 < M.n_layers; l++) {
        LayerBufs &b = lb[l];
        b.xn = take_f(H);
        b.q = take_f(QW);
        b.k = take_f(KVW);
        b.v = take_f(KVW);
        b.attn = take_f(QW);
        b.attn_out = take_f(H);
        b.xn2 = take_f(H);
        b.gate = take_f(I);
        b.up = take_f(I);
        b.h = take_f(I);
        b.ffn_out = take_f(H);
      }
      for (int32_t l = -1; l + 1 < M.n_layers; l++) rs[l + 1] = take_f(H);
    } else {
      float *other = take_f(H);
      for (int32_t l = -1; l < M.n_layers; l++)
        rs[l + 1] = ((M.n_layers - 1 - l) % 2 + 2) % 2 ? other : B.x;
    }
  }
  auto resid = [&](int32_t l) { return rs[l + 1]; };
  // the matvec levels: per layer q/k/v (0), o (1), gate/up (2), down (3); then the lm_head
  auto mv = [](const void *w, const float *x, float *y, int32_t *idx, int n, int p) {
    q8_matvec_desc d;
    d.w = w;
    d.x = x;
    d.y = y;
    d.idx = idx;
    d.n = n;
    d.p = p;
    return d;
  };
  // The element-wise steps between matvecs run as prologues when every
  // launch is all staged and the vectors fit the staged x: each workgroup of
  // the consuming launch computes its x (the residual adds and norms) while
  // its first tile loads, and the gate/up launch computes the SwiGLU of the
  // rows it holds (paired tiles: the same rows of both matrices).
  // Otherwise they run as epilogues, by the last workgroup of the producing
  // launch, whose outputs then take device-scope stores.
  const bool pro_path = H <= q8::kProMaxN && I <= q8::kProMaxN &&
                        q8::step_all_staged(1, H, false) && q8::step_all_staged(1, QW, false) &&
                        q8::step_all_staged(1, I, false);
  std::vector<std::vector<q8_matvec_desc>> lv;
  for (int32_t l = 0; l < M.n_layers; l++) {
    const q8_decode_layer &L = M.layers[l];
    const LayerBufs &b = lb[l];
    lv.push_back({mv(L.wq, b.xn, b.q, nullptr, H, QW), mv(L.wk, b.xn, b.k, nullptr, H, KVW),
                  mv(L.wv, b.xn, b.v, nullptr, H, KVW)});
    lv.push_back({mv(L.wo, b.attn, b.attn_out, nullptr, QW, H)});
    if (pro_path)  // one paired descriptor (w2, y2 and h are filled after planning)
      lv.push_back({mv(L.w_gate, b.xn2, b.gate, nullptr, H, I)});
    else
      lv.push_back({mv(L.w_gate, b.xn2, b.gate, nullptr, H, I), mv(L.w_up, b.xn2, b.up, nullptr, H, I)});
    lv.push_back({mv(L.w_down, b.h, b.ffn_out, nullptr, I, H)});
  }
  lv.push_back({mv(M.lm_head, B.xf, B.logits, B.token, H, M.vocab)});
  auto paired_level = [&](size_t i) { return pro_path && i + 1 < lv.size() && i % 4 == 2; };
  // the paired gate/up descriptor of level i (after planning)
  auto pair_up = [&](size_t i, q8::StepPlan &pl) {
    if (paired_level(i)) pl.descs[0].flags |= q8::kDescPairedSilu;
  };
  std::vector<q8::StepPlan> plans(lv.size());
  for (size_t i = 0; i < lv.size(); i++) {
    st = q8::plan_step(lv[i].data(), (int32_t)lv[i].size(), 1, dev, q8::kStepGroupSize,
                       plans[i], false, true, 0, paired_level(i) ? 1u : 0u);
    if (st) return st;
    pair_up(i, plans[i]);
  }
  for (const auto &pl : plans)
    if (pro_path && !pl.all_staged) return Q8_ERR_SHAPE;  // (the shapes above are staged)
  // The persistent form: one launch of as many workgroups as are resident
  // at once with LDS for the widest staged tile and x and for an attention
  // block; every level is planned on that grid, and every output but the
  // logits is read by other workgroups of the launch (device-scope stores).
  int pgrid = 0;
  size_t plds = 0;
  if (pers) {
    if (!pro_path) return Q8_ERR_SHAPE;
    plds = q8::attention_lds_bytes(G);
    for (const auto &pl : plans) plds = pl.lds > plds ? pl.lds : plds;
    pgrid = q8::decode_persistent_grid(dev, G, plds);
    if (pgrid < 1) return Q8_ERR_SHAPE;
    for (size_t i = 0; i < lv.size(); i++) {
      st = q8::plan_step(lv[i].data(), (int32_t)lv[i].size(), 1, dev, q8::kStepGroupSize,
                         plans[i], false, true, pgrid, paired_level(i) ? 1u : 0u);
      if (st) return st;
      pair_up(i, plans[i]);
      if (i + 1 < lv.size())
        for (auto &d : plans[i].descs) d.flags |= q8::kDescDeviceOut;
    }
  }
  if (!pro_path)
    for (size_t i = 0; i + 1 < lv.size(); i++)
      if (i % 4 != 0)  // o, gate/up, down: their outputs are read by the epilogue
        for (auto &d : plans[i].descs) d.flags |= q8::kDescDeviceOut;

  q8_step_graph *g = new (std::nothrow) q8_step_graph();
  if (!g) return Q8_ERR_GRAPH;
  g->magic = kGraphMagic;
  g->device = dev;
  g->mode = Q8_GRAPH_DECODE;
  g->m = 1;
  g->i8x = false;
  g->act = act.release();

  // workspace (256-byte aligned pieces): the lm_head argmax slot, the
  // epilogues' arrival slot, the attention arrival slots, the epilogues,
  // the RoPE frequencies and the step's cos/sin table, the attention
  // partials, then each level's table and workgroup ranges
  const int chunks = q8::attn_chunks(M.cache_rows);
  size_t total = 0;
  auto take = [&](size_t bytes) {
    const size_t off = total;
    total += (bytes + 255) & ~(size_t)255;
    return off;
  };
  const size_t o_amax = take(sizeof(q8::ArgmaxSlot));
  const size_t o_earr = take(sizeof(q8::ArgmaxSlot));
  const size_t o_aarr = take(sizeof(q8::ArgmaxSlot) * (size_t)M.n_kv_heads);
  const size_t o_epi = take(sizeof(q8::Epilogue) * 3 * (size_t)M.n_layers);
  const size_t o_pro = take(sizeof(q8::Prologue) * (3 * (size_t)M.n_layers + 1));
  const size_t o_pair = take(sizeof(q8::PairOut) * (size_t)M.n_layers);
  const size_t o_freq = take(sizeof(float) * q8::kAttnHeadDim / 2);
  const size_t o_rope = take(sizeof(float) * q8::kAttnHeadDim);
  const size_t o_part = take(sizeof(float) * (size_t)M.n_heads * chunks * q8::kAttnPart);
  const int32_t nphases = pers ? 5 * M.n_layers + 1 : 0;
  const size_t o_bar = take(pers ? sizeof(q8::GridBarrier) : 0);
  const size_t o_phase = take(sizeof(q8::DecPhase) * (size_t)nphases);
  const size_t o_attn = take(pers ? sizeof(q8::AttnArgs) * (size_t)M.n_layers : 0);
  std::vector<size_t> o_tab(plans.size()), o_grp(plans.size());
  for (size_t i = 0; i < plans.size(); i++) {
    o_tab[i] = take(plans[i].descs.size() * sizeof(q8::StepDesc));
    o_grp[i] = take(plans[i].groups.size() * sizeof(q8::WgGroup));
  }
  hipError_t e = hipMalloc(&g->workspace, total);
  if (e == hipSuccess) e = hipMemset(g->workspace, 0, total);
  if (e != hipSuccess) {
    release_graph(g);
    return hip_fail(e);
  }
  char *ws = (char *)g->workspace;
  q8::ArgmaxSlot *amax = (q8::ArgmaxSlot *)(ws + o_amax);
  q8::ArgmaxSlot *earr = (q8::ArgmaxSlot *)(ws + o_earr);
  q8::Epilogue *epis = (q8::Epilogue *)(ws + o_epi);
  q8::Prologue *pros = (q8::Prologue *)(ws + o_pro);
  {
    q8::StepPlan &pl = plans.back();
    q8::ArgmaxSlot hs;
    std::memset(&hs, 0, sizeof(hs));
    uint32_t nteams = 0;
    for (int j = 0; j < q8::kArgmaxTeams; j++) {
      hs.team[j].expected = pl.expected[0][j];
      nteams += pl.expected[0][j] ? 1u : 0u;
    }
    hs.top.expected = nteams;
    hs.host = host_dev;
    pl.descs[0].slot = amax;
    e = hipMemcpy(amax, &hs, sizeof(hs), hipMemcpyHostToDevice);
  }
  std::vector<q8::Epilogue> he(3 * (size_t)M.n_layers);
  for (int32_t l = 0; l < M.n_layers && e == hipSuccess; l++) {
    const q8_decode_layer &L = M.layers[l];
    q8::Epilogue *E = &he[3 * (size_t)l];
    std::memset(E, 0, 3 * sizeof(q8::Epilogue));
    E[0].op = q8::kEpiAddNorm;  // after o: x += attn_out; xn2 = norm(x)
    E[0].n = H;
    E[0].eps = M.eps;
    E[0].x = B.x;
    E[0].r = lb[l].attn_out;
    E[0].g = L.ffn_norm;
    E[0].out = lb[l].xn2;
    E[0].arrive = earr;
    E[1].op = q8::kEpiSiluMul;  // after gate/up: h = silu(gate) * up
    E[1].n = I;
    E[1].r = lb[l].up;
    E[1].g = lb[l].gate;
    E[1].out = lb[l].h;
    E[1].arrive = earr;
    const bool lastl = l + 1 == M.n_layers;
    E[2].op = q8::kEpiAddNorm;  // after down: x += ffn_out; next layer's xn, or xf
    E[2].n = H;
    E[2].eps = M.eps;
    E[2].x = B.x;
    E[2].r = lb[l].ffn_out;
    E[2].g = lastl ? M.out_norm : M.layers[l + 1].attn_norm;
    E[2].out = lastl ? B.xf : lb[l + 1].xn;
    E[2].arrive = earr;
  }
  if (e == hipSuccess)
    e = hipMemcpy(epis, he.data(), he.size() * sizeof(q8::Epilogue), hipMemcpyHostToDevice);
  // prologues of layer l: 3l the gate/up launch's norm, 3l + 1 the down
  // launch's SwiGLU, 3l + 2 the next layer's q/k/v launch's (or the
  // lm_head's) residual add and norm; 3L the first q/k/v launch's norm of
  // x_in
  std::vector<q8::Prologue> hp(3 * (size_t)M.n_layers + 1);
  std::memset(hp.data(), 0, hp.size() * sizeof(q8::Prologue));
  for (int32_t l = 0; l < M.n_layers; l++) {
    const q8_decode_layer &L = M.layers[l];
    q8::Prologue *P = &hp[3 * (size_t)l];
    P[0].op = q8::kProAddNorm;  // xn2 = norm(R_{l-1} + attn_out)
    P[0].n = H;
    P[0].eps = M.eps;
    P[0].a = resid(l - 1);
    P[0].b = lb[l].attn_out;
    P[0].w = L.ffn_norm;
    P[0].out = lb[l].xn2;
    P[1].op = q8::kProSiluMul;  // h = silu(gate) * up
    P[1].n = I;
    P[1].a = lb[l].gate;
    P[1].b = lb[l].up;
    P[1].out = lb[l].h;
    const bool lastl = l + 1 == M.n_layers;
    P[2].op = q8::kProAddNorm;  // R_l = (R_{l-1} + attn_out) + ffn_out; the next xn, or xf
    P[2].n = H;
    P[2].eps = M.eps;
    P[2].a = resid(l - 1);
    P[2].b = lb[l].attn_out;
    P[2].c = lb[l].ffn_out;
    P[2].w = lastl ? M.out_norm : M.layers[l + 1].attn_norm;
    P[2].out = lastl ? B.xf : lb[l + 1].xn;
    P[2].resid = resid(l);
  }
  {
    q8::Prologue &P = hp[3 * (size_t)M.n_layers];
    P.op = q8::kProNorm;  // R_{-1} = x_in; xn = norm(x_in)
    P.n = H;
    P.eps = M.eps;
    P.a = B.x_in;
    P.w = M.layers[0].attn_norm;
    P.out = lb[0].xn;
    P.resid = resid(-1);
  }
  if (e == hipSuccess)
    e = hipMemcpy(pros, hp.data(), hp.size() * sizeof(q8::Prologue), hipMemcpyHostToDevice);
  // each layer's paired gate/up launch: the up matrix, and where up and
  // h = silu(gate) * up go (prologue form)
  q8::PairOut *pairs = (q8::PairOut *)(ws + o_pair);
  {
    std::vector<q8::PairOut> hq(M.n_layers);
    for (int32_t l = 0; l < M.n_layers; l++) {
      std::memset(&hq[l], 0, sizeof(q8::PairOut));
      hq[l].w2 = (const uint8_t *)M.layers[l].w_up;
      hq[l].y2 = lb[l].up;
      hq[l].h = lb[l].h;
    }
    if (e == hipSuccess)
      e = hipMemcpy(pairs, hq.data(), hq.size() * sizeof(q8::PairOut), hipMemcpyHostToDevice);
  }
  for (size_t i = 0; i < plans.size() && e == hipSuccess; i++) {
    e = hipMemcpy(ws + o_tab[i], plans[i].descs.data(),
                  plans[i].descs.size() * sizeof(q8::StepDesc), hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(ws + o_grp[i], plans[i].groups.data(),
                    plans[i].groups.size() * sizeof(q8::WgGroup), hipMemcpyHostToDevice);
  }
  auto attn_args = [&](int32_t l) {
    const q8_decode_layer &Ly = M.layers[l];
    q8::AttnArgs a{};
    a.q = lb[l].q;
    a.k = lb[l].k;
    a.v = lb[l].v;
    a.q_norm = Ly.q_norm;
    a.k_norm = Ly.k_norm;
    a.kc = Ly.k_cache;
    a.vc = Ly.v_cache;
    a.pos = B.pos;
    a.rope = (const float *)(ws + o_rope);
    a.freq = (const float *)(ws + o_freq);
    a.out = lb[l].attn;
    a.part = (float *)(ws + o_part);
    a.arrive = (q8::ArgmaxSlot *)(ws + o_aarr);
    a.n_heads = M.n_heads;
    a.n_kv = M.n_kv_heads;
    a.cache_rows = M.cache_rows;
    a.chunks = chunks;
    a.eps = M.eps;
    return a;
  };
  if (pers && e == hipSuccess) {
    // the phase table: per layer q/k/v (layer 0 normalises x_in, a later
    // layer adds the residuals of the one before), attention, o, gate/up
    // (its norm), down (the SwiGLU); then the lm_head (the last residual
    // add and the final norm)
    std::vector<q8::AttnArgs> ha(M.n_layers);
    std::vector<q8::DecPhase> ph;
    const q8::AttnArgs *dattn = (const q8::AttnArgs *)(ws + o_attn);
    auto mphase = [&](size_t i, const q8::Prologue *pro, const q8::PairOut *pair = nullptr) {
      q8::DecPhase d{};
      d.pair = pair;
      d.kind = q8::kPhaseMatvec;
      d.count = (int32_t)plans[i].descs.size();
      d.group_size = plans[i].group_size;
      d.grid = plans[i].grid;
      d.table = (const q8::StepDesc *)(ws + o_tab[i]);
      d.groups = (const q8::WgGroup *)(ws + o_grp[i]);
      d.pro = pro;
      ph.push_back(d);
    };
    for (int32_t l = 0; l < M.n_layers; l++) {
      ha[l] = attn_args(l);
      mphase(4 * (size_t)l, l ? &pros[3 * (size_t)l - 1] : &pros[3 * (size_t)M.n_layers]);
      q8::DecPhase d{};
      d.kind = q8::kPhaseAttention;
      d.attn = dattn + l;
      ph.push_back(d);
      mphase(4 * (size_t)l + 1, nullptr);
      mphase(4 * (size_t)l + 2, &pros[3 * (size_t)l], pairs + l);
      mphase(4 * (size_t)l + 3, nullptr);  // x = h, from the gate/up phase
    }
    mphase(plans.size() - 1, &pros[3 * (size_t)M.n_layers - 1]);
    e = ph.size() == (size_t)nphases ? hipSuccess : hipErrorInvalidValue;
    if (e == hipSuccess)
      e = hipMemcpy(ws + o_attn, ha.data(), ha.size() * sizeof(q8::AttnArgs),
                    hipMemcpyHostToDevice);
    if (e == hipSuccess)
      e = hipMemcpy(ws + o_phase, ph.data(), ph.size() * sizeof(q8::DecPhase),
                    hipMemcpyHostToDevice);
    // the barrier: counters zero (the workspace's memset), the token's
    // addresses for a failed wait
    int32_t *const tok[2] = {B.token, host_dev};
    if (e == hipSuccess)
      e = hipMemcpy(ws + o_bar + offsetof(q8::GridBarrier, idx), tok, sizeof(tok),
                    hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = q8::launch_rope_freq(M.theta, (float *)(ws + o_freq), nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    release_graph(g);
    return hip_fail(e);
  }

  if (pers) {
    SegmentLaunch L{nullptr, nullptr, 0, 0, pgrid, plds, true};
    L.kind = kDecodeNode;
    L.phases = (const q8::DecPhase *)(ws + o_phase);
    L.nphases = nphases;
    L.bar = (q8::GridBarrier *)(ws + o_bar);
    L.heads_per_kv = G;
    g->launches.push_back(L);
    return capture_graph(g, out, [&](hipStream_t cs) {
      return run_segment(g->launches[0], 1, false, cs);
    });
  }
  auto step_node = [&](size_t i, const q8::Epilogue *epi, const q8::Prologue *pro = nullptr,
                       const q8::PairOut *pair = nullptr) {
    const q8::StepPlan &pl = plans[i];
    SegmentLaunch L{(const q8::StepDesc *)(ws + o_tab[i]), (const q8::WgGroup *)(ws + o_grp[i]),
                    (int32_t)pl.descs.size(), pl.group_size, pl.grid, pl.lds, pl.all_staged};
    L.epi = epi;
    L.pro = pro;
    L.pair = pair;
    L.dec = true;
    g->launches.push_back(L);
  };
  {
    SegmentLaunch L{nullptr, nullptr, 0, 0, 0, 0, true};
    L.kind = kNormNode;  // the rotation; the first norm too without prologues
    L.nx = pro_path ? nullptr : B.x_in;
    L.nw = M.layers[0].attn_norm;
    L.nout = B.xn;
    L.ncopy = B.x;
    L.ndim = H;
    L.neps = M.eps;
    L.npos = B.pos;
    L.nfreq = (const float *)(ws + o_freq);
    L.rope_out = (float *)(ws + o_rope);
    g->launches.push_back(L);
  }
  for (int32_t l = 0; l < M.n_layers; l++) {
    const q8::Prologue *qkv_pro =
        l ? &pros[3 * (size_t)l - 1] : &pros[3 * (size_t)M.n_layers];
    step_node(4 * (size_t)l, nullptr, pro_path ? qkv_pro : nullptr);
    SegmentLaunch A{nullptr, nullptr, 0, 0, 0, 0, true};
    A.kind = kAttnNode;
    A.attn = attn_args(l);
    g->launches.push_back(A);
    if (pro_path) {
      step_node(4 * (size_t)l + 1, nullptr);
      step_node(4 * (size_t)l + 2, nullptr, &pros[3 * (size_t)l], pairs + l);
      step_node(4 * (size_t)l + 3, nullptr);  // x = h, stored by the gate/up node
    } else {
      step_node(4 * (size_t)l + 1, &epis[3 * (size_t)l]);
      step_node(4 * (size_t)l + 2, &epis[3 * (size_t)l + 1]);
      step_node(4 * (size_t)l + 3, &epis[3 * (size_t)l + 2]);
    }
  }
  step_node(plans.size() - 1, nullptr,
            pro_path ? &pros[3 * (size_t)M.n_layers - 1] : nullptr);
  return capture_graph(g, out, [&](hipStream_t cs) {
    hipError_t le = hipSuccess;
    for (size_t i = 0; i < g->launches.size() && le == hipSuccess; i++)
      le = run_segment(g->launches[i], 1, false, cs);
    return le;
  });
}

}  // namespace

int q8_decode_graph_build(const q8_decode_model *model, const q8_decode_buffers *buf,
                          int32_t *host_token, void *stream, q8_step_graph **out) {
  (void)stream;
  return build_decode(model, buf, host_token, out);
}

int q8_step_graph_build(const q8_matvec_desc *descs, int32_t count, int32_t m,
                        int32_t *host_idx, int32_t mode, void *stream,
                        q8_step_graph **out) {
  (void)stream;
  if (mode == Q8_GRAPH_LEVELS) return Q8_ERR_MODE;  // needs the levels
  return build_graph(descs, nullptr, count, m, host_idx, mode, out);
}

int q8_step_graph_build_levels(const q8_matvec_desc *descs, const int32_t *levels,
                               int32_t count, int32_t m, int32_t *host_idx,
                               void *stream, q8_step_graph **out) {
  (void)stream;
  return build_graph(descs, levels, count, m, host_idx, Q8_GRAPH_LEVELS, out);
}

int q8_step_graph_launch(q8_step_graph *g, void *stream) {
  if (!live_graph(g)) return Q8_ERR_BAD_HANDLE;
  hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_step_graph_launch_kernel(q8_step_graph *g, void *stream) {
  if (!live_graph(g)) return Q8_ERR_BAD_HANDLE;
  if (g->mode == Q8_GRAPH_CHAIN) return Q8_ERR_MODE;
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e);
  if (cur != g->device && (e = hipSetDevice(g->device)) != hipSuccess) return hip_fail(e);
  for (size_t i = 0; i < g->launches.size() && e == hipSuccess; i++)
    e = run_segment(g->launches[i], g->m, g->i8x, (hipStream_t)stream);
  if (cur != g->device) (void)hipSetDevice(cur);
  return e == hipSuccess ? Q8_OK : hip_fail(e);
}

int q8_step_graph_info(const q8_step_graph *g, int32_t *kernel_nodes,
                       int32_t *memcpy_nodes) {
  if (!live_graph(g)) return Q8_ERR_BAD_HANDLE;
  if (kernel_nodes) *kernel_nodes = g->kernel_nodes;
  if (memcpy_nodes) *memcpy_nodes = g->memcpy_nodes;
  return Q8_OK;
}

int q8_step_graph_destroy(q8_step_graph *g) {
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g || !g_graphs.count(g) || g->magic != kGraphMagic)
      return Q8_ERR_BAD_HANDLE;
    g_graphs.erase(g);
  }
  release_graph(g);
  return Q8_OK;
}

}  // extern "C"
