/*
 * dla.h - C ABI of libdla: LongNet dilated attention on AMD MI355X (gfx950).
 *
 * Sources (web pages about LongNet, arXiv 2307.02486), cited below as:
 *   [G] the gptget.net summary page of arXiv 2307.02486; sections 方法论
 *       (method), 方法详解 (method details), 实验设计 (experiment design),
 *       原文摘要 (the English abstract);
 *   [D] the darcstar.tech research page "LongNet: Scaling Transformers to
 *       1,000,000,000 Tokens", the DarcStar commentary.
 *
 * The operator ([G] 方法论, 方法详解): for each pattern (w, r) the sequence is
 * split into segments of w rows (the last one holds whatever rows remain
 * when w does not divide N, all N rows when w > N; under the causal mask
 * this equals padding the sequence to a multiple of w); in each segment
 * every r-th row is kept,
 * starting at row (h mod r) for head h, for Q, K and V alike; dense softmax
 * attention runs inside each sparsified segment.  Patterns are merged with
 * weights exp(LSE_p - LSE), LSE = log sum_p exp(LSE_p), so the softmax
 * denominator they share stays exact ([D] commentary).  With `causal`, a row
 * attends only to rows at or before it inside its sparsified segment.  A row
 * that no pattern keeps gets O = 0 and LSE = -inf.  The method is a drop-in
 * replacement for standard attention ([G] 原文摘要): one pattern (N, 1) is
 * full softmax attention.
 *
 * Conventions for every entry point:
 *   - Tensors q, k, v, o, dout, dq, dk, dv are device pointers to
 *     [B, N, H, D] tensors with element strides (stride_b, stride_n,
 *     stride_h) and a contiguous last dimension.  D must be 64.  Element type
 *     is shape->dtype (fp32 or bf16; bf16 paths compute in bf16 with fp32
 *     accumulation).  lse is a device pointer to a contiguous fp32 [B, H, N]
 *     tensor holding natural-log log-sum-exp values.
 *   - All device pointers and strides*element size must be 16-byte aligned,
 *     unless an entry point states otherwise (the FP8 codes and scales, the
 *     lengths array).  An empty problem (B == 0 or H == 0) reads and writes
 *     nothing, so its pointers are not checked and may be null.
 *   - The caller owns every buffer, including the workspace; the library
 *     allocates and frees no device memory, keeps no device state and never
 *     synchronises (apart from dla_timing_collect, which waits for its
 *     events).  Its only global state is the opt-in timing record of
 *     dla_timing_enable (host memory: a flag, the recorded events and a
 *     pool of reusable events, behind a mutex), the thread-local error
 *     text, and dla_forward_noalloc's static device scratch (part of the
 *     library's code object, with its per-device addresses).  The
 *     exceptions are the attention layer's calls: dla_blas_create makes a
 *     hipBLASLt handle (its own host and device state), and the handle
 *     keeps, per product shape, the hipBLASLt descriptors and the algorithm
 *     chosen on the first call with that shape (host memory, freed by
 *     dla_blas_destroy).  Work is enqueued on `stream` (a hipStream_t;
 *     NULL is the null stream) and returns before it runs.
 *   - Descriptors are caller-owned host memory read only during the call.
 *   - Return value: DLA_OK or a negative DLA_E_* code.  All validation runs on
 *     the host before anything is enqueued; a failed call enqueues nothing.
 *     dla_last_error() returns the calling thread's message for its last
 *     failed call.
 */
#ifndef DLA_H_
#define DLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLA_MAX_PATTERNS 16
#define DLA_HEAD_DIM 64

#define DLA_OK 0
#define DLA_E_INVALID (-1)      /* null/misaligned pointer, bad w or r, bad scale or count */
#define DLA_E_UNSUPPORTED (-2)  /* D != 64, w % r != 0, unknown dtype, limits exceeded */
#define DLA_E_WORKSPACE (-3)    /* workspace smaller than dla_plan_check reports */
#define DLA_E_HIP (-4)          /* the HIP runtime refused a launch */

typedef enum { DLA_F32 = 0, DLA_BF16 = 1 } dla_dtype;

/* One dilation pattern: segment length w, dilation rate r ([G] 方法论). */
typedef struct {
  int32_t w;
  int32_t r;
} dla_pattern;

/* The operator: 1..16 patterns (host memory), a causal flag (0/1) and the
 * softmax scale applied to q.k (finite, > 0; 1/sqrt(D) for standard use). */
typedef struct {
  int32_t num_patterns;
  const dla_pattern* patterns;
  int32_t causal;
  float scale;
} dla_desc;

/* Problem shape and element strides of q/k/v/o (and the gradients). */
typedef struct {
  int64_t B, N, H, D;
  int32_t dtype; /* dla_dtype */
  int64_t stride_b, stride_n, stride_h;
} dla_shape;

/*
 * Validate a descriptor and shape on the host and report the workspace bytes
 * dla_forward and dla_backward need (either out-pointer may be NULL).  Needs
 * no GPU.  B == 0 or H == 0 is a valid empty problem.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED.
 */
int dla_plan_check(const dla_desc* desc, const dla_shape* shape, size_t* ws_fwd_bytes,
                   size_t* ws_bwd_bytes);

/*
 * Forward pass ([G] 方法论; [D] commentary).  Writes o ([B,N,H,D], input
 * dtype) and lse ([B,H,N] fp32).  ws must hold at least the forward workspace
 * size of dla_plan_check (it stores the per-pattern partial results of all
 * patterns but the one that keeps the most rows).
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_forward(const dla_desc* desc, const dla_shape* shape, const void* q, const void* k,
                const void* v, void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * dla_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same kernels and results as dla_forward, but the workspace is a static
 * array inside the library, DLA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU
 * the library's code is loaded on, held until the process ends; the call
 * allocates and frees nothing.  The scratch of the current device
 * (hipGetDevice) is used, so `stream` must belong to that device.  Every
 * call on one GPU shares that GPU's scratch: calls whose execution overlaps
 * on one GPU (other streams, other threads) race and must be serialised by
 * the caller; calls in one stream are ordered and safe.  Nothing in the
 * scratch needs clearing between calls (each partial result is written
 * before it is read).
 * Errors: as dla_forward; DLA_E_WORKSPACE when the problem needs more than
 * DLA_NOALLOC_SCRATCH_BYTES of workspace (dla_plan_check's ws_fwd), in
 * which case nothing is enqueued.
 */
#define DLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int dla_forward_noalloc(const dla_desc* desc, const dla_shape* shape, const void* q, const void* k,
                        const void* v, void* o, float* lse, void* stream);

/*
 * Backward pass: gradients of sum(dout * o) with respect to q, k and v, where
 * (o, lse) are the outputs of dla_forward for the same q, k, v, desc and
 * shape.  The merge weights are differentiated through (the combined output
 * is one softmax over the union of each row's keys), so each pattern uses the
 * combined lse and D = rowsum(dout * o).  dq, dk, dv have the input dtype and
 * the strides of `shape`; they are accumulated over patterns in fp32 in the
 * workspace and rounded once.  Deterministic: no atomics.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_backward(const dla_desc* desc, const dla_shape* shape, const void* q, const void* k,
                 const void* v, const void* o, const float* lse, const void* dout, void* dq,
                 void* dk, void* dv, void* ws, size_t ws_bytes, void* stream);

/*
 * ---- Batches of different lengths ----
 *
 * The same operator on a padded batch: batch b's sequence is its first
 * lengths[b] rows (segments are cut at that length as at the end of any
 * sequence); the rows after it are padding, with o = 0, lse = -inf and zero
 * gradients, and take no part in any other row's attention.  lengths is a
 * device int32 buffer of B entries, read by the kernels; an entry outside
 * [0, N] is clamped to that range.  The workspace sizes are those of
 * dla_plan_check for the padded shape.
 * Errors: as dla_forward / dla_backward, and DLA_E_INVALID for a null or
 * misaligned lengths pointer (B > 0 and H > 0).
 */
int dla_forward_varlen(const dla_desc* desc, const dla_shape* shape, const int32_t* lengths,
                       const void* q, const void* k, const void* v, void* o, float* lse,
                       void* ws, size_t ws_bytes, void* stream);
int dla_backward_varlen(const dla_desc* desc, const dla_shape* shape, const int32_t* lengths,
                        const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * ---- 8-bit keys and values ([G] 方法详解, last item: quantization combines
 * with the method) ----
 *
 * K and V are stored as FP8 E4M3 codes (the OCP 8-bit format: bias 7,
 * largest finite value 448, no infinities) with one fp32 scale per
 * (batch, head); the attention reads K = code * k_scale[b * H + h], and V
 * likewise.  Codes use the element strides of the bf16 shape, one byte per
 * element; scales are [B, H] fp32, 4-byte aligned.
 *
 * dla_quantize_fp8: codes and scales of a bf16 tensor x (shape->dtype =
 * DLA_BF16, D = 64).  Per head, amax = max |x| over its N rows and 64
 * columns; inv = 448 / amax and scale = amax / 448, both rounded to fp32
 * (inv = scale = 1 for an all-zero head); code = the E4M3 value nearest to
 * fp32(x * inv), ties to even, after clamping to +-448.  x8 is device memory
 * the caller owns; scale is written last (it holds the amaxes while the call
 * runs).  B * H <= 65535.  Asynchronous on `stream`; nothing is allocated.
 * Errors: DLA_E_INVALID (null or misaligned pointer, bad strides),
 * DLA_E_UNSUPPORTED (dtype, D, B * H), DLA_E_HIP.
 */
int dla_quantize_fp8(const dla_shape* shape, const void* x, uint8_t* x8, float* scale, void* stream);

/*
 * dla_forward with 8-bit keys and values: q, o, lse as for dla_forward
 * (shape->dtype must be DLA_BF16), k8/v8 codes and k_scale/v_scale scales as
 * above.  The same workspace as dla_forward (dla_plan_check).  The codes are
 * decoded exactly to bf16 inside the kernel; the rest of the arithmetic is
 * dla_forward's.
 * Errors: as dla_forward; DLA_E_UNSUPPORTED for an fp32 shape.
 */
int dla_forward_fp8kv(const dla_desc* desc, const dla_shape* shape, const void* q,
                      const uint8_t* k8, const uint8_t* v8, const float* k_scale,
                      const float* v_scale, void* o, float* lse, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * dla_pair_count for batches of different lengths; here lengths is host
 * memory (B entries, clamped to [0, N]).  Host only.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED.
 */
int dla_pair_count_varlen(const dla_desc* desc, const dla_shape* shape, const int32_t* lengths,
                          int64_t* pairs);

/*
 * Index map of one pattern ([G] 方法论: segment, dilation, head offset):
 * out[h * ceil(N / r) + s * (w / r) + a] = s * w + (h mod r) + a * r, the
 * original row of sparse row a of segment s, for every head h < H, or -1
 * when that row lies past the end of the sequence (a last segment cut
 * short).  out is a device int32 buffer of H * ceil(N / r) entries.  This is
 * the address generator every kernel uses, exposed so that it can be
 * compared bit for bit.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_HIP.
 */
int dla_row_map(const dla_desc* desc, int64_t N, int32_t H, int32_t pattern, int32_t* out,
                void* stream);

/*
 * Number of (query, key) pairs the operator evaluates, summed over batch,
 * heads and patterns: per segment L(L+1)/2 if causal else L^2, with
 * L = w_p / r_p (fewer in a last segment cut short, depending on the head
 * offset).  Linear in N for fixed L ([G] 方法论).  Host only.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED.
 */
int dla_pair_count(const dla_desc* desc, const dla_shape* shape, int64_t* pairs);

/*
 * ---- Sequence shards ([G] 方法论, the distributed item) ----
 *
 * The pages scale past one device by cutting the sequence along its length:
 * each device holds one contiguous piece, a segment that fits in a piece is
 * handled locally, and for a segment that crosses devices the devices
 * exchange its sparsified keys and values, so that each one attends its own
 * queries to the whole segment; the cost of the exchange does not grow with
 * the sequence.  These entry points are one device's share of that scheme:
 * the collective itself (an all-gather over the devices of a segment) is the
 * caller's.
 *
 * The device holds rows [shard_start, shard_start + N) of a sequence of
 * total_rows rows, where N is shape->N, shard_start is a multiple of N and N
 * divides total_rows.  Every w divides total_rows.  A pattern with w <= N
 * must divide N (its segments are local).  A pattern with w > N "spans":
 * N must divide w, r must divide N and N / r must be a multiple of 64.
 * Shards are implemented for bf16.
 */
typedef struct {
  int64_t total_rows;
  int64_t shard_start;
} dla_shard;

/*
 * Validate a descriptor, a shard shape and its place in the sequence on the
 * host and report the workspace bytes dla_forward_shard and
 * dla_backward_shard need (either out pointer may be NULL).
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED.
 */
int dla_plan_check_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                         size_t* ws_fwd_bytes, size_t* ws_bwd_bytes);

/*
 * Number of (query, key) pairs the shard evaluates: the pairs of
 * dla_pair_count whose query row lies in the shard.  Host only.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED.
 */
int dla_pair_count_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                         int64_t* pairs);

/*
 * This device's part of the exchange for spanning pattern `pattern`: its
 * sparse rows of the segment that contains the shard,
 *   out[b][h][i][:] = x[b][(h mod r) + i * r][h][:],  i < N / r,
 * written as a contiguous bf16 [B, H, N/r, D] tensor (x is k or v of the
 * shard, strides of `shape`).  Gathering these parts from the w/N devices of
 * the segment in device order gives the [w/N, B, H, N/r, D] buffer that
 * dla_forward_shard reads.  out is a device pointer the caller owns.
 * Errors: DLA_E_INVALID (null/misaligned pointer, pattern index out of range
 * or a pattern that does not span), DLA_E_UNSUPPORTED, DLA_E_HIP.
 */
int dla_shard_gather(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                     int32_t pattern, const void* x, void* out, void* stream);

/*
 * Forward pass of one shard: writes o and lse for the shard's rows (q, k, v,
 * o, lse shaped by `shape`, i.e. N = the shard length), equal to the rows
 * [shard_start, shard_start + N) that dla_forward computes on the whole
 * sequence.  Local patterns read the shard's k and v.  For every spanning
 * pattern p, ext_k[p] and ext_v[p] are device pointers to the gathered parts
 * of the segment that contains the shard, [w_p/N, B, H, N/r_p, D] bf16 as
 * dla_shard_gather lays them out; entries of other patterns are ignored
 * (the arrays are host memory with num_patterns entries, or NULL when no
 * pattern spans).  ws must hold dla_plan_check_shard's size.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_forward_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                      const void* q, const void* k, const void* v, const void* const* ext_k,
                      const void* const* ext_v, void* o, float* lse, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Backward pass of one shard, first half.  (o, lse) are the shard's outputs
 * of dla_forward_shard, dout its upstream gradient, ext_k/ext_v the same
 * gathered segments.  Writes:
 *   - dq for every row of the shard (bf16, final);
 *   - dk, dv for the shard's rows that no spanning pattern keeps (final);
 *   - for every spanning pattern p, ext_dk[p] and ext_dv[p]: this shard's
 *     contributions to the gradients of the whole segment's sparsified keys
 *     and values, fp32 [w_p/N, B, H, N/r_p, D] in the exchange layout (device
 *     order), already scaled.  The caller sums them over the devices of the
 *     segment and hands each device its part (a reduce-scatter), then calls
 *     dla_shard_finish.
 * The workspace (dla_plan_check_shard's backward size) carries the local
 * patterns' partial gradients to dla_shard_finish and must not change in
 * between.  The backward also needs N / r_p to be a multiple of 128 for
 * every spanning pattern (DLA_E_UNSUPPORTED otherwise).
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_backward_shard(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                       const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, const void* const* ext_k,
                       const void* const* ext_v, void* dq, void* dk, void* dv,
                       void* const* ext_dk, void* const* ext_dv, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * Backward pass of one shard, second half: for every row of the shard that
 * a spanning pattern keeps, dk and dv become the sum of the local patterns'
 * partials (from the workspace) and, for each spanning pattern p, the
 * exchanged part red_dk[p] / red_dv[p] (fp32 [B, H, N/r_p, D]: the sum over
 * the segment's devices of their ext_dk[p] / ext_dv[p] parts for this
 * shard), rounded once.  Other rows are left as dla_backward_shard wrote
 * them.  The arrays are host memory with num_patterns entries (entries of
 * local patterns are ignored).
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_shard_finish(const dla_desc* desc, const dla_shape* shape, const dla_shard* shard,
                     const float* const* red_dk, const float* const* red_dv, void* dk, void* dv,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * ---- A LongNet attention layer ([G] 实验设计: 768-dimensional model,
 * 12 heads) ----
 *
 * Y = DA(X W_q, X W_k, X W_v) W_o with W_qkv = [W_q | W_k | W_v], no bias,
 * E = 64 H model dimensions.  X, Y [B, N, E] bf16 contiguous; W_qkv [E, 3E]
 * and W_o [E, E] bf16 row-major (y = x W).  The projections are plain GEMMs
 * done by hipBLASLt (fp32 accumulation) with the caller's handle
 * (dla_blas_create); the attention is dla_forward / dla_backward.
 */

/* Create / destroy the handle the layer calls use (the only calls that
 * allocate: hipBLASLt's own host and device state, plus a per-shape cache
 * of hipBLASLt descriptors and chosen algorithms, filled on the first call
 * with each product shape and guarded by a mutex, so one handle may serve
 * several threads).  The handle is opaque; pass it to the layer calls. */
int dla_blas_create(void** handle);
int dla_blas_destroy(void* handle);

/* Workspace bytes of dla_layer_forward and dla_layer_backward.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED. */
int dla_layer_plan_check(const dla_desc* desc, int64_t B, int64_t N, int64_t H,
                         size_t* ws_fwd_bytes, size_t* ws_bwd_bytes);

/*
 * Forward.  Writes qkv ([3, B, N, H, D] bf16: q, k, v, each contiguous), the
 * attention output attn ([B, N, H, D] bf16) and lse ([B, H, N] fp32), which
 * the backward reads, and y.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_layer_forward(const dla_desc* desc, int64_t B, int64_t N, int64_t H, const void* x,
                      const void* w_qkv, const void* w_o, void* qkv, void* attn, float* lse,
                      void* y, void* blas, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of sum(dy * y): dx ([B, N, E] bf16), dw_qkv ([E, 3E] fp32) and
 * dw_o ([E, E] fp32), from the forward's x, weights, qkv, attn and lse.
 * Errors: DLA_E_INVALID, DLA_E_UNSUPPORTED, DLA_E_WORKSPACE, DLA_E_HIP.
 */
int dla_layer_backward(const dla_desc* desc, int64_t B, int64_t N, int64_t H, const void* x,
                       const void* w_qkv, const void* w_o, const void* qkv, const void* attn,
                       const float* lse, const void* dy, void* dx, float* dw_qkv, float* dw_o,
                       void* blas, void* ws, size_t ws_bytes, void* stream);

/*
 * Opt-in launch timing, a profiling aid.  While enabled (on != 0), every
 * kernel launch made by the library is bracketed by two HIP events recorded
 * on the caller's stream (host-side bookkeeping only; the kernels are
 * unchanged).  This record is process-wide: the one global state of the
 * library besides the thread-local error text.  Events are taken from a
 * pool that dla_timing_collect refills, so a timed launch creates no event
 * once the pool holds as many as are in flight.  Kernel families:
 * "attn_fwd" (bf16 forward attention), "attn_fwd_f32", "attn_fwd_fp8" (8-bit
 * keys and values), "combine", "bwd_prep", "attn_bwd", "bwd_finalize",
 * "shard_gather" (a shard's exchange parts and relayouts), "shard_finish",
 * "quantize_fp8".
 */
int dla_timing_enable(int on);

/*
 * Wait for the recorded events of kernel family `name`, return the number of
 * timed launches and their summed duration in milliseconds, and forget them.
 * Errors: DLA_E_INVALID (null argument), DLA_E_HIP.
 */
int dla_timing_collect(const char* name, int64_t* launches, double* total_ms);

/* Static text for an error code. */
const char* dla_strerror(int code);

/* The calling thread's message for its last failed call ("" if none). */
const char* dla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DLA_H_ */
