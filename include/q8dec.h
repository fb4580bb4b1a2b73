/*
 * q8dec.h - C ABI of libq8dec, the Q8_0 single-token decode matvec for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (inferno.rs "IV.4: One command buffer per token", section
 * "Eight kernels", the q8_matvec listing and the prose after it):
 *   W has p rows and n columns, stored row-major as Q8_0 blocks.  A block is
 *   34 bytes: a little-endian IEEE binary16 scale, then 32 signed 8-bit
 *   quants; block b of a row covers x[32b .. 32b+31].  Row r of W is the
 *   n/32 blocks at byte offset r * (n/32) * 34.  The weights are the raw
 *   block bytes, never repacked ("The decoder: kernels and helpers", q8_bytes).
 *     y[r] = sum_b scale(r,b) * sum_j q(r,b,j) * x[32b + j]
 *   computed in binary32 from exact binary32 products of each quant with x;
 *   the scale is applied once per block (the dequantise-in-the-dot shape the
 *   same section describes).
 * The argmax ("Eight kernels", argmax_row and the prose after it): the index
 *   of the largest logit, ties to the lowest index, so only four bytes per
 *   row leave the device.  NaN logits never win; -0 and +0 are equal; a row
 *   whose logits are all NaN yields -1.
 * The whole decode step (q8_decode_graph_build, below) adds the layer's
 *   other operations: norms, RoPE, the KV append, attention, SwiGLU.
 * The step (sections "One command buffer" and "The seam"): the 197 matvecs
 *   of one decode step (7 projections x 28 layers, then the lm_head and its
 *   argmax) are recorded once and submitted once, and one int32 comes back
 *   (written by the kernel into pinned host memory).
 *
 * Conventions for every entry point
 *   - Pointers named w, x, y, logits, idx are DEVICE pointers owned by the
 *     caller; the library never allocates, frees or retains them.  host_idx
 *     is caller-owned PINNED host memory (hipHostMalloc).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls are stream-ordered and asynchronous: results are valid once the
 *     caller has synchronised the stream.  Outputs are bit-identical from run
 *     to run for the same inputs.
 *   - Layouts: w is p rows x (n/32) blocks x 34 bytes, contiguous; x is
 *     [m][n] float32 row-major; y is [m][p] float32 row-major; idx is int32[m].
 *   - Alignment: w and x 16 bytes; y, logits and idx 4 bytes.  A pointer may
 *     be NULL only when its buffer holds zero bytes.
 *   - Every argument is validated before any HIP call; a refused call does
 *     no GPU work and returns a nonzero Q8_ERR_* status.  Q8_OK is 0.
 *   - The argmax entry points (q8_argmax, q8_matvec_argmax,
 *     q8_matvec_argmax_i8x) keep a small workspace (12.4 KB) inside the
 *     library for each stream they run on, so calls on different streams
 *     never share one and calls on one stream are ordered by it.  The null
 *     stream's is allocated by q8_init (or the first call of any entry
 *     point); another stream's by its first argmax call, which clears it in
 *     that stream's order.  That first call must not be made while the
 *     stream is capturing a graph: it is refused with Q8_ERR_GRAPH.  At most
 *     256 streams per device get a workspace (Q8_ERR_COUNT beyond); each is
 *     kept until the process ends.
 *   - Split-K: q8_matvec, q8_matvec_batched and q8_matvec_argmax with one
 *     activation row (m = 1) and a width n above 3072 that is a multiple of
 *     256 cut W's columns into slices of at most 3072 (ceil(n / 3072)
 *     slices of equal width in multiples of 256, the last one narrower),
 *     compute each slice's partial sums, then add them in slice order (the
 *     rvllm page's K-split, "The matmul pain story").  The partial sums live
 *     in the stream's workspace, (slices * p) floats, allocated or grown by
 *     the call that needs more (after the stream's earlier work is done);
 *     such a call is refused with Q8_ERR_GRAPH while the stream is
 *     capturing.  Results are deterministic (fixed slice order) and within
 *     the same bound as any other summation order.
 */
#ifndef Q8DEC_H
#define Q8DEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define Q8_OK 0
#define Q8_ERR_NULL 1        /* a required pointer is NULL                  */
#define Q8_ERR_SHAPE 2       /* bad m, n or p (see limits)                  */
#define Q8_ERR_ALIGN 3       /* a pointer breaks the alignment rule         */
#define Q8_ERR_NO_DEVICE 4   /* no HIP device is visible                    */
#define Q8_ERR_ARCH 5        /* the current device is not gfx950            */
#define Q8_ERR_CODE_OBJECT 6 /* kernels not loadable on this device; sticky */
#define Q8_ERR_HIP 7         /* a HIP call failed: see q8_last_hip_error()  */
#define Q8_ERR_GRAPH 8       /* step-graph capture or instantiation failed  */
#define Q8_ERR_BAD_HANDLE 9  /* NULL, unknown or destroyed graph handle     */
#define Q8_ERR_COUNT 10      /* descriptor count or argmax count out of range */
#define Q8_ERR_MODE 11       /* unknown step-graph mode                     */
#define Q8_ERR_LEVELS 12     /* step levels negative or decreasing          */

/* ---- limits --------------------------------------------------------- */
#define Q8_BLOCK 32                 /* quants per block                       */
#define Q8_BLOCK_BYTES 34           /* bytes per block                        */
#define Q8_MAX_M 32                 /* activation rows per batched call       */
#define Q8_MAX_M_NARROW 8           /* m above this: n a positive multiple of 256,
                                       binary32 activations only              */
#define Q8_MAX_N 65536              /* 0 <= n <= Q8_MAX_N, n % 32 == 0        */
#define Q8_MAX_P 0x7FFFFFFF         /* 0 <= p; p >= 1 where an argmax is taken */
#define Q8_MAX_DESCS 4096           /* descriptors per step graph             */
#define Q8_MAX_ARGMAX_DESCS 64      /* argmax descriptors per step graph      */

/* ---- status and device ---------------------------------------------- */

/* Name of a status code ("q8_ok", "q8_err_shape", ...); any other value
 * gives "q8_code_out_of_range".  Never touches the GPU. */
const char *q8_status_name(int status);

/* The hipError_t of the most recent HIP failure seen by this thread
 * (0 if none). */
int q8_last_hip_error(void);

/* Number of visible HIP devices (0 when none), without selecting one. */
int q8_device_count(int32_t *count);

/* Checks the current device (gfx950, kernels loadable) and allocates the
 * null stream's argmax workspace.  Optional: every entry point does it on
 * first use.  A failure is remembered for that device and returned again
 * (sticky). */
int q8_init(void);

/* ---- matvec ------------------------------------------------------------ */

/* y[p] = W x for one activation row x[n] (inferno.rs "IV.4", "Eight kernels",
 * the q8_matvec kernel; m = 1).
 * p == 0 or n == 0 is allowed (n == 0 writes zeros). */
int q8_matvec(const void *w, const float *x, float *y, int32_t n, int32_t p,
              void *stream);

/* Batched decode: y[m][p] = x[m][n] W^T with 1 <= m <= Q8_MAX_M (32); the
 * weight blocks are streamed once for all m rows (the Algenta page's batched
 * decode, where the rows of a batch share one weight sweep; rvllm's
 * linear_small loops rows inside its weight loop).  m <= 8: any width
 * (n == 0 writes zeros).  8 < m <= 32: n a positive multiple of 256, else
 * Q8_ERR_SHAPE; each output is computed from x split into two bf16 parts and
 * exact quants on the matrix cores, accumulated in binary32 (the same bound
 * as every other entry point). */
int q8_matvec_batched(const void *w, const float *x, float *y, int32_t m,
                      int32_t n, int32_t p, void *stream);

/* idx[i] = argmax over logits[i][0..p-1] for i < m; 1 <= m <= Q8_MAX_M, p >= 1. */
int q8_argmax(const float *logits, int32_t m, int32_t p, int32_t *idx,
              void *stream);

/* Fused lm_head: the matvec of q8_matvec_batched followed by the argmax of
 * each output row, without a logits round trip.  y_or_null may be NULL (no
 * logits written) or a [m][p] buffer that also receives the logits. */
int q8_matvec_argmax(const void *w, const float *x, float *y_or_null,
                     int32_t *idx, int32_t m, int32_t n, int32_t p,
                     void *stream);

/* q8_matvec_argmax for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and results (bit for bit) as
 * q8_matvec_argmax, but the argmax workspace is a fixed 12,736-byte array
 * in the library's own device memory (one per device, held until the
 * process ends) instead of a per-stream allocation: this call, and the
 * device set-up it may do on its first call on a device, call no hipMalloc,
 * hipFree or other allocating routine.  The array holds the keys of at most
 * Q8_MAX_M (32) activation rows: a larger m is refused with Q8_ERR_SHAPE.
 * Every q8_matvec_argmax_noalloc call on one device shares that array, so
 * two such calls that overlap in time on one device race and may return
 * wrong indices: issue them in one stream order.  The array is zero when
 * the library loads and each call leaves it zero.  Other arguments, layouts
 * and errors as q8_matvec_argmax. */
int q8_matvec_argmax_noalloc(const void *w, const float *x, float *y_or_null,
                             int32_t *idx, int32_t m, int32_t n, int32_t p,
                             void *stream);

/* ---- int8-activation variant ----------------------------------------------- */

/* The CPU's sdot form (inferno.rs "IV.4", the prose after the q8_matvec
 * listing in "Eight kernels", and "The correctness ladder": activations
 * quantised to int8, integer products).  Each row of x is quantised per
 * block of 32 in binary32 by the Q8_0 rule: amax = max |x_j|, d = amax/127,
 * q_j = x_j * (1/d) rounded to nearest, ties to even; d = 0 gives q = 0; a
 * block holding a NaN or an infinity gets d = NaN and q = 0.  Then
 *   y[i][r] = sum_b scale(r,b) * d(i,b) * sum_j q(r,b,j) * q_x(i,b,j)
 * with exact integer block sums and binary32 scaling and accumulation.  The
 * result differs from q8_matvec by the quantisation of x, at most
 * sum_b |scale| * d/2 * sum_j |q| per output; it is a separate operation
 * with its own bound, never a replacement for q8_matvec.
 * Widths: n a multiple of 256 with n <= 3072 (n == 0 writes zeros); other
 * widths give Q8_ERR_SHAPE.  1 <= m <= Q8_MAX_M_NARROW (8); layouts,
 * alignment, ownership and errors as q8_matvec_batched. */
int q8_matvec_i8x(const void *w, const float *x, float *y, int32_t m, int32_t n,
                  int32_t p, void *stream);

/* q8_matvec_i8x followed by the argmax of each output row (as
 * q8_matvec_argmax: ties to the lowest index, NaN skipped). */
int q8_matvec_argmax_i8x(const void *w, const float *x, float *y_or_null,
                         int32_t *idx, int32_t m, int32_t n, int32_t p,
                         void *stream);

/* ---- decode step graph --------------------------------------------------- */

/* One matvec of a step.  x is [m][n], y is [m][p]; idx != NULL asks for the
 * fused argmax (then y may be NULL). */
typedef struct q8_matvec_desc {
  const void *w;
  const float *x;
  float *y;
  int32_t *idx;
  int32_t n;
  int32_t p;
} q8_matvec_desc;

typedef struct q8_step_graph q8_step_graph;

/* How a step graph is recorded.
 *  Q8_GRAPH_CHAIN: one kernel node per descriptor, in descriptor order, each
 *    depending on the previous one (the in-order semantics of one command
 *    buffer).
 *  Q8_GRAPH_PERSISTENT: one kernel node that walks a device-side table of
 *    all descriptors with no ordering between them (valid when no
 *    descriptor reads another's output).  For 1 < m <= 8 with every width
 *    1024, 2048 or 3072 and no argmax on a matvec wider than 1024, the
 *    wider matvecs run as column slices of 1024 whose partial outputs (in
 *    a buffer the graph owns) a second kernel node adds in slice order:
 *    two kernel nodes, and the wider matvecs' outputs round as that sum
 *    does (not bit-identical to q8_matvec_batched; within the same
 *    bound of the exact result).
 *  Q8_GRAPH_PERSISTENT_I8X: as Q8_GRAPH_PERSISTENT, every matvec computed
 *    as q8_matvec_i8x (every width must be one it takes, else
 *    Q8_ERR_SHAPE), column slices included (the wider matvecs' outputs
 *    then round as the slices' sum does, not bit-identical to
 *    q8_matvec_i8x; within its bound). */
#define Q8_GRAPH_CHAIN 0
#define Q8_GRAPH_PERSISTENT 1
#define Q8_GRAPH_PERSISTENT_I8X 2
#define Q8_GRAPH_LEVELS 3  /* built by q8_step_graph_build_levels only */

/* Records the descriptors (1 <= count <= Q8_MAX_DESCS, at most
 * Q8_MAX_ARGMAX_DESCS with idx) for m activation rows into an instantiated
 * hipGraph.  If host_idx is non-NULL (pinned memory from hipHostMalloc,
 * m int32 per argmax descriptor, in descriptor order) the kernel that
 * finishes each argmax also stores its result there with system-scope
 * stores, so the token reaches host memory with no copy node: the graph
 * holds kernel nodes only.  Each host_idx entry is written once per launch,
 * with its final value; the other outputs are valid once the stream is
 * synchronised.  The descriptors' pointers are baked in: to change inputs,
 * write new values into the same x buffers.  `stream` only names the device
 * context; nothing is enqueued on it.  *out receives a handle owned by the
 * caller (free with q8_step_graph_destroy).  A host_idx that is not pinned
 * host memory is refused with Q8_ERR_HIP. */
int q8_step_graph_build(const q8_matvec_desc *descs, int32_t count, int32_t m,
                        int32_t *host_idx, int32_t mode, void *stream,
                        q8_step_graph **out);

/* A step with dependencies between its matvecs (the in-order command buffer
 * of inferno.rs "IV.4", "One command buffer", with the siblings that read the
 * same input run together): levels[i] >= 0 is descriptor i's dependency
 * level, non-decreasing over the descriptors.  Each run of equal levels
 * becomes one persistent kernel node over those descriptors (no ordering
 * among them), and the nodes run in level order, each after the previous
 * one has finished.  For a decoder layer: q, k, v at one level, o at the
 * next, gate and up at the next, down at the next.  Otherwise as
 * q8_step_graph_build (host_idx, ownership, errors); the graph's mode is
 * Q8_GRAPH_LEVELS.  Q8_ERR_NULL for levels == NULL, Q8_ERR_LEVELS for a
 * negative or decreasing level. */
int q8_step_graph_build_levels(const q8_matvec_desc *descs, const int32_t *levels,
                               int32_t count, int32_t m, int32_t *host_idx,
                               void *stream, q8_step_graph **out);

/* Enqueues the whole step with one hipGraphLaunch on `stream`. */
int q8_step_graph_launch(q8_step_graph *g, void *stream);

/* All but Q8_GRAPH_CHAIN: enqueues the same recorded step (its kernel or
 * kernels, in level or node order, with the arguments fixed at build
 * time; for Q8_GRAPH_DECODE the 5 * n_layers + 2 kernels of the decode step)
 * with kernel launches instead of hipGraphLaunch: the same work, results and
 * host_idx writes.  Runs on the graph's device whatever device is current; `stream`
 * must belong to that device.  On MI355X with ROCm 7.2 a hipGraphLaunch
 * costs ~10 us more launch latency than a kernel launch (measured).
 * Q8_ERR_MODE for a chain graph. */
int q8_step_graph_launch_kernel(q8_step_graph *g, void *stream);

/* Node counts of the instantiated graph (kernel nodes, memcpy nodes; the
 * latter are 0 since results reach host memory from the kernels): the
 * per-step dispatch budget. */
int q8_step_graph_info(const q8_step_graph *g, int32_t *kernel_nodes,
                       int32_t *memcpy_nodes);

/* Destroys the graph and its workspace; the handle becomes invalid. */
int q8_step_graph_destroy(q8_step_graph *g);

/* ---- the whole decode step ------------------------------------------------
 * inferno.rs "IV.4", "One command buffer": per layer, rms_norm_row ->
 * q, k, v projections -> QK-norm (rms_norm_row per head) -> rope_row on q
 * and k -> append_kv at row pos -> attention_decode over rows 0..pos ->
 * o projection -> add_inplace into x -> rms_norm_row -> gate, up ->
 * silu_hadamard -> down projection -> add_inplace; then the final norm, the
 * lm_head and argmax_row ("Eight kernels" defines each operation).  The
 * pages encode 18 dispatches per layer; here a layer is 5 kernel nodes: the
 * q/k/v matvecs; the attention with the QK-norm, RoPE and append folded in;
 * o; gate/up; down.  Before the first layer one node computes the RoPE
 * rotation of position pos; after the last the fused lm_head argmax runs:
 * 5 * n_layers + 2 nodes.  The element-wise work between matvecs (the
 * residual adds, the norms, SwiGLU) runs in one of two places:
 *   - prologue form, taken when every matvec width is a multiple of 256 up
 *     to 3072 and hidden, inter <= 3072 (Qwen3-0.6B's shapes): every
 *     workgroup of the launch that consumes the vector computes it into its
 *     staged x while its first weight tile loads, and workgroup 0 stores it
 *     (the first q/k/v: R = x_in and xn = norm(x_in); gate/up: xn2 =
 *     norm(R + attn_out); down: h = silu(gate) * up; the next layer's q/k/v,
 *     or the lm_head: R' = (R + attn_out) + ffn_out and its norm).  The residual stream alternates between buf->x and a
 *     workspace buffer from layer to layer, and after the last layer it is
 *     in buf->x;
 *   - epilogue form, for every other shape: the first node also copies
 *     x_in into buf->x and norms it, and the last workgroup of the launch
 *     that produces a vector computes it once every output of that launch
 *     is stored (o: x += attn_out and xn2; gate/up: h; down: x += ffn_out
 *     and the next norm); the residual stream stays in buf->x.
 * The residual adds run in the pages' order in both; a norm's sum of squares
 * is added in another order in each (results within the same bound).
 * Everything is binary32. */

#define Q8_GRAPH_DECODE 4  /* mode of graphs from q8_decode_graph_build */

/* One layer's resident weights (device pointers, caller-owned). */
typedef struct {
  const void *wq, *wk, *wv, *wo;        /* Q8_0 [out][in/32 blocks]: q [n_heads*128][hidden],
                                           k, v [n_kv_heads*128][hidden], o [hidden][n_heads*128] */
  const void *w_gate, *w_up, *w_down;   /* Q8_0: gate, up [inter][hidden], down [hidden][inter] */
  const float *attn_norm, *ffn_norm;    /* float32 [hidden] */
  const float *q_norm, *k_norm;         /* float32 [128], the per-head QK-norm weights */
  float *k_cache, *v_cache;             /* float32 [cache_rows][n_kv_heads*128]: row t is token t's
                                           key (after QK-norm and RoPE) and value */
} q8_decode_layer;

/* The model: shapes (1 <= n_layers <= 512; head_dim must be 128; n_heads a
 * multiple of n_kv_heads, at most 4 query heads per key/value head;
 * hidden <= 4096; hidden, inter multiples of 32; 1 <= cache_rows <= 65536;
 * eps >= 0 and theta > 0, finite), a HOST array of n_layers layers, the
 * final norm and lm_head (device), and the form of the recorded step:
 *   Q8_DECODE_NODES (0): 5 kernel nodes per layer + 2, as described above;
 *   Q8_DECODE_PERSISTENT (1): one kernel node that runs every phase (per
 *     layer q/k/v, attention, o, gate/up, down; then the lm_head) with all
 *     of its workgroups resident, meeting at a grid-wide barrier between
 *     phases; each workgroup requests its next phase's first weight tile
 *     (or cached rows) before it waits.  Takes the prologue form's shapes
 *     only (hidden, the query width and inter multiples of 256, at most
 *     3072; else Q8_ERR_SHAPE).  The launch must have the device to itself
 *     (all workgroups resident at once): a wait at the barrier that runs
 *     past 200 ms (another workgroup never arrived) ends the step with the
 *     token -2, after which the graph must be destroyed and built again. */
#define Q8_DECODE_NODES 0
#define Q8_DECODE_PERSISTENT 1
typedef struct {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, inter, vocab, cache_rows;
  float eps, theta;
  const q8_decode_layer *layers;
  const float *out_norm;                /* float32 [hidden] */
  const void *lm_head;                  /* Q8_0 [vocab][hidden/32 blocks] */
  int32_t form;                         /* Q8_DECODE_NODES or Q8_DECODE_PERSISTENT */
} q8_decode_model;

/* The step's activations: device buffers owned by the caller, each sized
 * for its role (float32).  The caller writes x_in (the token's embedding
 * row, inferno.rs "The decoder: kernels and helpers", embed_row) and *pos
 * (the token's position; cache rows 0..pos-1 hold the earlier tokens) before
 * each launch.  After a launch every buffer holds the last layer's values;
 * the step reads x_in and writes the rest, so a launch can be repeated. */
typedef struct {
  const float *x_in;                    /* [hidden] */
  const int32_t *pos;                   /* int32 [1] */
  float *x;                             /* [hidden] the residual stream */
  float *xn;                            /* [hidden] attention-norm output (q/k/v input) */
  float *q, *k, *v;                     /* [n_heads*128], [n_kv*128], [n_kv*128]: projections,
                                           before QK-norm and RoPE */
  float *attn;                          /* [n_heads*128] attention output */
  float *attn_out;                      /* [hidden] o projection */
  float *xn2;                           /* [hidden] ffn-norm output */
  float *gate, *up, *h;                 /* [inter] projections and their SwiGLU */
  float *ffn_out;                       /* [hidden] down projection */
  float *xf;                            /* [hidden] final-norm output (lm_head input) */
  float *logits;                        /* [vocab], or NULL: logits not stored */
  int32_t *token;                       /* int32 [1]: the argmax of the logits */
} q8_decode_buffers;

/* Records the whole decode step as one hipGraph (mode Q8_GRAPH_DECODE) that
 * q8_step_graph_launch / _launch_kernel / _info / _destroy take.  host_token
 * (pinned host memory, or NULL) also receives the token, stored by the
 * kernel.  A pos outside [0, cache_rows) writes no cache row and makes the
 * attention output NaN, so the token is -1.  Buffers and weights are baked
 * in (resident state: nothing is allocated or uploaded per step); the graph
 * owns a workspace of (n_heads * ceil(cache_rows/64) * 528 + small) bytes.
 * Two launches of one graph must not overlap.  Errors: Q8_ERR_NULL for a
 * missing pointer, Q8_ERR_SHAPE for shapes outside the limits above,
 * Q8_ERR_ALIGN for weights or activation buffers not 16-byte aligned,
 * Q8_ERR_HIP for an unpinned host_token. */
int q8_decode_graph_build(const q8_decode_model *model, const q8_decode_buffers *buf,
                          int32_t *host_token, void *stream, q8_step_graph **out);

#ifdef __cplusplus
}
#endif

#endif /* Q8DEC_H */
