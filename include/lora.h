/*
 * lora.h -- C ABI of liblora_mi355x.so: the multi-LoRA batched linear on MI355X (gfx950).
 *
 * Source pages, cited by title and section:
 *   [P1] "Multi-LoRA Serving: Why 100 Adapters Fit on One GPU" (dev.to)
 *   [P2] "Serving Many LoRA Adapters From One Base Model" (ai-tldr.dev)
 *   [P3] "Multi-LoRA Serving: Sharing One GPU Across Adapters" (cloudai.pt)
 *
 * The layer ([P1], "Why can't you just merge LoRA weights into the base model?", the
 * layer equation):
 *
 *     y[m, :] = x[m, :] W  +  (x[m, :] A_i) B_i * (alpha_i / r_i),   i = ids[m]
 *
 * for a mixed batch in which every row names its own adapter, and id -1 means the bare
 * base model ([P2], "A worked example: the memory math", the adapter=None request).
 * The shared term is one GEMM over the whole batch; the delta is computed for all adapters
 * in one pass over the full batch, an index vector mapping rows to adapter ids, and a
 * stacked adapter tensor ([P1], "How does one batch run 30 different adapters at once?"),
 * in two steps, shrink (x A_i, down to the rank) and expand (times B_i, back to d_out)
 * ([P3], "MoE Models Raise the Bar").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers.  All array arguments are DEVICE pointers (hipMalloc'd or torch CUDA tensors),
 *    row-major and contiguous.  x, W, A, B, y and t must be 16-byte aligned; the workspace
 *    256-byte aligned.  Scalars are passed by value.
 *  - Types.  x, W, A, B hold bfloat16 bit patterns (uint16).  y is bfloat16 or float32
 *    (lora_dtype_t).  t is float32.  scale is float32, ranks and ids are int32.
 *  - Shapes.  x[M, d_in], W[d_in, d_out], A[n_adapters, d_in, r_max],
 *    B[n_adapters, r_max, d_out], y[M, d_out], t[M, r_max].  A_i is stored d_in x r_max and
 *    B_i r_max x d_out: the transposes of [P1]'s "A: r x d_in, B: d_out x r" in "How much
 *    memory does one LoRA adapter actually cost?", same r * (d_in + d_out) parameters.
 *  - Limits.  0 <= M <= LORA_MAX_ROWS (M = 0 is a no-op that returns LORA_OK);
 *    d_in, d_out positive multiples of 8; 1 <= r_max <= 64 (the pages' static maximum rank,
 *    vLLM's max_lora_rank, [P1] "What does a working multi-LoRA config look like?");
 *    1 <= n_adapters <= LORA_MAX_ADAPTERS.  The kernels work at the rank bucket of r_max
 *    (8, 16, 32 or 64); any r_max is exact, since padded ranks add exact zeros.
 *  - Pool contents (caller's contract).  Every adapter is padded to r_max ([P1], "What
 *    does a working multi-LoRA config look like?" and "Where does multi-LoRA serving
 *    actually break?", rank padding): ranks[i] in [1, r_max], and the entries of A_i beyond
 *    column ranks[i] and of B_i beyond row ranks[i] are zero.  scale[i] = alpha_i / ranks[i]
 *    is computed by the caller.  ranks may be NULL, meaning every adapter has rank r_max.
 *    Registering an adapter is a plain device copy into slot i of A and B plus ranks[i] and
 *    scale[i] ([P2], "How it works", "Loading and swapping adapters"); no call is needed.
 *  - ids.  ids[m] in [-1, n_adapters).  An id outside that range is treated as base-only on
 *    the device (and counted in meta[2] where segments are built); nothing faults.  Callers
 *    that want the error reported pass LORA_MODE_CHECKED (below).
 *  - Streams.  `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; none synchronises, except the checked mode and the
 *    measurement aids (named below).  The library keeps no state between calls and
 *    allocates no device memory: the caller owns every buffer, including the workspace.
 *    Calls that share a workspace or segment buffers must not overlap in time.
 *  - Errors.  Arguments are validated on the host before anything is enqueued; on a
 *    validation error nothing is enqueued and the call returns the status.  LORA_ERR_HIP
 *    reports a failed launch; lora_last_hip_error() names the HIP error.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_TILE_ROWS 16        /* rows per work tile of a segment */
#define LORA_MAX_ADAPTERS 16384  /* pool slots one call can address */
#define LORA_MAX_ROWS (1 << 22)  /* rows per call */
#define LORA_MAX_PROJ 4          /* projections per lora_linear_multi call */

/* The three enums below are passed as int.  Any int value may reach the library (an
 * unknown status or dtype, a mode with LORA_MODE_CHECKED OR-ed in), so in C++ they are given
 * int as their fixed underlying type, which makes every int value a valid value of the type
 * and keeps the C representation. */
#ifdef __cplusplus
#define LORA_ENUM_INT : int
#else
#define LORA_ENUM_INT
#endif

typedef enum LORA_ENUM_INT {
    LORA_OK = 0,
    LORA_ERR_NULL = 1,      /* a required pointer is NULL */
    LORA_ERR_SHAPE = 2,     /* M, d_in, d_out or n_adapters out of range */
    LORA_ERR_RANK = 3,      /* r_max outside [1, 64]; (checked mode) a rank outside [1, r_max] */
    LORA_ERR_ALIGN = 4,     /* a pointer is not aligned as required */
    LORA_ERR_WORKSPACE = 5, /* ws_bytes smaller than lora_workspace_bytes() */
    LORA_ERR_DTYPE = 6,     /* unknown lora_dtype_t */
    LORA_ERR_HIP = 7,       /* a kernel launch failed */
    LORA_ERR_BAD_ID = 8,    /* (checked mode) an id outside [-1, n_adapters) */
    LORA_ERR_MODE = 9,      /* unknown lora_mode_t */
    LORA_ERR_POOL = 10      /* (checked mode) a compact-pool adapter's rows leave the pool */
} lora_status_t;

typedef enum LORA_ENUM_INT { LORA_BF16 = 0, LORA_F32 = 1 } lora_dtype_t;

/* How lora_linear runs the layer ([P1], "How does one batch run 30 different adapters at
 * once?": decode is bound by the weight bytes read, prefill by the xW GEMM, which dilutes
 * the delta further):
 * DECODE: the decode sequence -- a split-K or stream-K GEMM whose partial sums are added
 *   with the delta in one pass that rounds y once.
 * PREFILL: x W on the large-tile GEMM with the delta added in its epilogue before the only
 *   store: scale * t enters the epilogue's bf16 MFMAs as a pair of bf16 values (the value
 *   rounded to bf16 and the remainder rounded to bf16), about 16 significant bits.
 * AUTO: PREFILL when M >= LORA_PREFILL_MIN_ROWS, else DECODE.
 * LORA_MODE_CHECKED may be OR-ed into any mode (lora_linear, lora_linear_compact): the call
 * first waits for `stream`, copies ids, ranks and rank_offsets to host memory and checks
 * them -- ids in [-1, n_adapters) (else LORA_ERR_BAD_ID), ranks in [1, r_max] (else
 * LORA_ERR_RANK), compact adapters inside the pool (else LORA_ERR_POOL) -- and enqueues
 * nothing when one fails.  For tests and debugging; not for graph capture. */
typedef enum LORA_ENUM_INT { LORA_MODE_AUTO = 0, LORA_MODE_DECODE = 1, LORA_MODE_PREFILL = 2 } lora_mode_t;
#define LORA_MODE_CHECKED 0x100
#define LORA_PREFILL_MIN_ROWS 768 /* measured: decode and prefill sequences cost the same at 768 rows (4096 x 4096, r 16) */

/* Rows grouped by adapter, as built by lora_build_segments.  All device buffers, owned by
 * the caller, sized for the M and n_adapters of the batch:
 *   perm        int32[M]                  rows of adapter 0 in ascending row order, then
 *                                         adapter 1, ..., then base-only rows (id -1 or
 *                                         invalid) in ascending row order
 *   offsets     int32[n_adapters + 1]     offsets[i] = first position of adapter i in perm;
 *                                         offsets[n_adapters] = number of LoRA rows
 *   seg_adapter int32[max(1, min(M, n))]  adapters with at least one row, ascending
 *   tiles       int32[2 * lora_max_tiles(M, n)]
 *                                         every segment cut into runs of LORA_TILE_ROWS
 *                                         positions of perm: {first position, adapter}
 *   meta        int32[4]                  {segments, LoRA rows, invalid ids, tiles} */
typedef struct {
    int32_t *perm;
    int32_t *offsets;
    int32_t *seg_adapter;
    int32_t *tiles;
    int32_t *meta;
} lora_segments_t;

/* Upper bound on the number of tiles: min(M, n_adapters) + M / LORA_TILE_ROWS.  Sizing of
 * the segment buffers that lora_build_segments fills ([P1], "How does one batch run 30
 * different adapters at once?": no padding of the token dimension).  Returns 0 when M <= 0
 * or n_adapters <= 0. */
int32_t lora_max_tiles(int32_t M, int32_t n_adapters);

/* Workspace bytes needed by lora_linear, lora_linear_compact, lora_shrink and
 * lora_shrink_compact for these sizes (0 when M = 0): the segment buffers, t and the split-K
 * partial sums of the shrink and of the base GEMM ([P3], "MoE Models Raise the Bar": split-K
 * for the skinny products).  Returns 0 for arguments that the calls would reject.  The
 * workspace is caller-owned device memory; its contents need no initialisation. */
size_t lora_workspace_bytes(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                            int32_t n_adapters);

/* Group the rows of a batch by adapter: a histogram of ids, a prefix sum into offsets,
 * and a stable scatter into perm, all on the device in one launch.  The grouping is what
 * lets one pass serve every adapter of the batch ([P1], "How does one batch run 30
 * different adapters at once?"; [P2], "Going deeper", grouping by adapter).
 * ids: int32[M] (device).  Output: seg (see lora_segments_t; caller-owned device buffers).
 * Invalid ids are counted in meta[2] and grouped with the base-only rows.  Deterministic.
 * Errors: LORA_ERR_SHAPE (M or n_adapters out of range), LORA_ERR_NULL, LORA_ERR_ALIGN
 * (4-byte ids and buffers, 8-byte tiles), LORA_ERR_HIP. */
lora_status_t lora_build_segments(const int32_t *ids, int32_t M, int32_t n_adapters,
                                  lora_segments_t seg, void *stream);

/* Shrink, the first step of the delta ([P3], "MoE Models Raise the Bar"; the [B, d_in] x
 * [d_in, r] product of [P1], "How does one batch run 30 different adapters at once?"):
 * t[m, j] = sum_k x[m, k] A[ids[m], k, j] for rows with an adapter (j < r_max; columns
 * beyond the adapter's rank are 0), t[m, :] = 0 for base-only rows.
 * x[M, d_in], A[n_adapters, d_in, r_max] (padded pool), t[M, r_max] fp32 (device; t is
 * written, 16-byte aligned at its start).  seg must have been built for the same ids, M and
 * n_adapters.  ws: at least lora_workspace_bytes(M, d_in, 8, r_max, n_adapters) bytes
 * (split-K partial sums).  The partial sums are added in a fixed order: deterministic.
 * Errors: as lora_linear's validation (LORA_ERR_SHAPE, _RANK, _NULL, _ALIGN, _WORKSPACE). */
lora_status_t lora_shrink(const void *x, const void *A, const int32_t *ranks, int32_t M,
                          int32_t d_in, int32_t r_max, int32_t n_adapters,
                          lora_segments_t seg, float *t, void *ws, size_t ws_bytes,
                          void *stream);

/* Shrink on a rank-compact pool (layout as for lora_linear_compact): the same t[M, r_max] as
 * lora_shrink on the adapters zero-padded to r_max ([P1], "Where does multi-LoRA serving
 * actually break?": padding wastes bandwidth when ranks differ).  ranks and rank_offsets
 * are required (LORA_ERR_NULL); pool_rows in [1, n_adapters * round_up(r_max, 8)]
 * (LORA_ERR_SHAPE). */
lora_status_t lora_shrink_compact(const void *x, const void *A, const int32_t *ranks,
                                  const int32_t *rank_offsets, int32_t pool_rows, int32_t M,
                                  int32_t d_in, int32_t r_max, int32_t n_adapters,
                                  lora_segments_t seg, float *t, void *ws, size_t ws_bytes,
                                  void *stream);

/* Expand, the second step of the delta, scaled as in the layer equation ([P3], "MoE Models
 * Raise the Bar"; [P1], "Why can't you just merge LoRA weights into the base model?"):
 * y[m, :] += scale[i] * sum_{j < ranks[i]} t[m, j] B[i, j, :] for every row m with adapter
 * i = ids[m] >= 0; base-only rows of y are neither read nor written.  t[M, r_max] fp32
 * (4-byte aligned), B[n_adapters, r_max, d_out], y[M, d_out] in y_dtype (read and written).
 * One rounding per element of y.  seg as for lora_shrink.  No workspace.
 * Errors: LORA_ERR_SHAPE, _RANK, _DTYPE, _NULL, _ALIGN, _HIP. */
lora_status_t lora_expand(const float *t, const void *B, const float *scale,
                          const int32_t *ranks, int32_t M, int32_t d_out, int32_t r_max,
                          int32_t n_adapters, lora_segments_t seg, void *y,
                          lora_dtype_t y_dtype, void *stream);

/* Expand on a rank-compact pool (layout as for lora_linear_compact; same cite as
 * lora_shrink_compact): B is [pool_rows][d_out].  ranks and rank_offsets are required. */
lora_status_t lora_expand_compact(const float *t, const void *B, const float *scale,
                                  const int32_t *ranks, const int32_t *rank_offsets,
                                  int32_t pool_rows, int32_t M, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, lora_segments_t seg, void *y,
                                  lora_dtype_t y_dtype, void *stream);

/* The whole layer of [P1], "Why can't you just merge LoRA weights into the base model?":
 * y = x W + (x A_i) B_i scale_i, overwriting y[M, d_out]; one shared GEMM over the mixed
 * batch plus every row's own delta ([P2], "How it works", "Batching across different
 * adapters"), rows with id -1 bit-identical to a base-only call.
 * segs: NULL to build the segments inside the workspace from ids, or segments already
 * built for these ids (lets several projections of one batch share one build).
 * ws: at least lora_workspace_bytes(M, d_in, d_out, r_max, n_adapters) bytes.
 * mode: see lora_mode_t (LORA_MODE_CHECKED may be OR-ed in).
 * Errors: LORA_ERR_SHAPE, _RANK, _DTYPE, _MODE, _NULL, _ALIGN, _WORKSPACE before anything
 * is enqueued; with LORA_MODE_CHECKED also _BAD_ID, _RANK; LORA_ERR_HIP on a failed launch. */
lora_status_t lora_linear(const void *x, const void *W, const void *A, const void *B,
                          const float *scale, const int32_t *ranks, const int32_t *ids,
                          int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                          int32_t n_adapters, const lora_segments_t *segs, void *y,
                          lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                          size_t ws_bytes, void *stream);

/* The whole layer, as lora_linear, on a rank-compact adapter pool: no adapter is padded to
 * r_max.  Padding every adapter to the largest rank wastes memory and bandwidth when ranks
 * differ ([P1], "Where does multi-LoRA serving actually break?"); serving mixed ranks is
 * what good systems support ([P2], "Limits and pitfalls"), S-LoRA by keeping adapters of
 * different ranks together in one pool ([P3], "How S-LoRA Proved the Model").  Layout (all
 * device memory, caller-owned):
 *   ranks[i]         rank r_i of adapter i, any value in [1, r_max]; the adapter occupies
 *                    w_i = round_up(r_i, 8) rank rows (so every k row of A_i starts 16-byte
 *                    aligned), rank rows r_i .. w_i - 1 zero
 *   rank_offsets[i]  its first rank row: w_0 + ... + w_{i-1} for a packed pool (any
 *                    non-overlapping placement with rank_offsets[i] + w_i <= pool_rows works)
 *   A                bf16 [pool_rows * d_in]: A_i = [d_in][w_i] row-major at element
 *                    rank_offsets[i] * d_in
 *   B                bf16 [pool_rows][d_out]: B_i = rows rank_offsets[i] .. + w_i - 1
 *   pool_rows        rank rows in the pool, 1 <= pool_rows <= n_adapters * round_up(r_max, 8)
 * scale[i] = alpha_i / r_i as for lora_linear.  Tables that break this contract never make a
 * kernel read outside the pool: an adapter whose rows leave it adds nothing, and a rank above
 * r_max is clamped; LORA_MODE_CHECKED reports both (LORA_ERR_POOL, LORA_ERR_RANK).
 * Returns LORA_ERR_NULL when ranks or rank_offsets is NULL, LORA_ERR_SHAPE when pool_rows is
 * out of range, otherwise as lora_linear.  The result equals lora_linear's on the same
 * adapters zero-padded to r_max (up to the order of fp32 additions). */
lora_status_t lora_linear_compact(const void *x, const void *W, const void *A, const void *B,
                                  const float *scale, const int32_t *ranks,
                                  const int32_t *rank_offsets, int32_t pool_rows,
                                  const int32_t *ids, int32_t M, int32_t d_in, int32_t d_out,
                                  int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
                                  void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                  size_t ws_bytes, void *stream);

/* Several projections of one layer that read the same input rows, each with its own adapter
 * pool: [P1], "How much memory does one LoRA adapter actually cost?", names the MLP's
 * gate_proj, up_proj and down_proj as adapted modules; gate and up both read the layer's
 * hidden state.  For p < n_proj:
 *     y[p] = x W[p] + scale_i (x A[p]_i) B[p]_i   (i = ids[m] per row, as lora_linear)
 * W, A, B and y are HOST arrays of n_proj device pointers (1 <= n_proj <= LORA_MAX_PROJ, else
 * LORA_ERR_SHAPE; a NULL array gives LORA_ERR_NULL), each laid out and aligned as the
 * lora_linear argument of the same name; the projections share x, d_in, d_out, r_max, the
 * adapter tables (scale, ranks, ids: one adapter owns a pair A[p]_i, B[p]_i in every
 * projection) and segs.  ws: lora_workspace_bytes_multi() bytes (else LORA_ERR_WORKSPACE).
 * The pointer arrays are read during the call only; the caller owns every buffer.
 * Decode batches of 257-1024 rows that take lora_linear's stream-K sequence build the
 * segments once (unless segs is given) and run the projections' shrinks as one launch, their
 * GEMMs as one (their column panels end to end on one K line) and their reductions as one;
 * the K sums are then split at other points than in separate calls, so the bits may differ
 * from lora_linear's by the order of fp32 additions.  Every other batch runs lora_linear's
 * launches per projection (same bits).  Errors as lora_linear, for the first projection
 * whose arguments fail. */
size_t lora_workspace_bytes_multi(int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, int32_t n_proj);
lora_status_t lora_linear_multi(const void *x, int32_t n_proj, const void *const *W,
                                const void *const *A, const void *const *B, const float *scale,
                                const int32_t *ranks, const int32_t *ids, int32_t M, int32_t d_in,
                                int32_t d_out, int32_t r_max, int32_t n_adapters,
                                const lora_segments_t *segs, void *const *y, lora_dtype_t y_dtype,
                                lora_mode_t mode, void *ws, size_t ws_bytes, void *stream);
/* Measurement aid: lora_linear_profiled for lora_linear_multi's arguments. */
lora_status_t lora_linear_multi_profiled(
    const void *x, int32_t n_proj, const void *const *W, const void *const *A,
    const void *const *B, const float *scale, const int32_t *ranks, const int32_t *ids, int32_t M,
    int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
    void *const *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws, size_t ws_bytes, void *stream,
    float *kernel_ms, const char **kernel_names, int32_t max_kernels, int32_t *n_kernels);

/* The whole layer with a quantized base ([P1], "Where does multi-LoRA serving actually
 * break?", item 4: a base stored at low precision served beside higher-precision adapters,
 * so the delta runs in another type than the base and the base -- the denominator of the
 * LoRA overhead -- gets cheaper).  The base weight is fp8: W8 holds E4M3 codes of the OCP
 * 8-bit floating point format (1 sign, 4 exponent bits of bias 7, 3 mantissa bits;
 * subnormals; no infinity), laid out W8[d_out][d_in] (each output column's d_in codes
 * contiguous, 16-byte aligned), with one fp32 scale per output column, w_scale[d_out]:
 *     y = x W_eff + (x A_i) B_i scale_i,   W_eff[k, c] = w_scale[c] * dec(W8[c, k]).
 * x, A, B, scale, ranks, ids, y, segs and the workspace as for lora_linear (bf16 adapters,
 * padded pool, any r_max in [1, 64]).  Decode batches: M <= 256, d_in a multiple of 32 and at
 * least 128 (else LORA_ERR_SHAPE); mode LORA_MODE_AUTO or LORA_MODE_DECODE, LORA_MODE_CHECKED
 * may be OR-ed in (LORA_MODE_PREFILL gives LORA_ERR_MODE).  Workspace: lora_workspace_bytes()
 * of the same sizes.  Errors as lora_linear. */
lora_status_t lora_linear_fp8w(const void *x, const void *W8, const float *w_scale, const void *A,
                               const void *B, const float *scale, const int32_t *ranks,
                               const int32_t *ids, int32_t M, int32_t d_in, int32_t d_out,
                               int32_t r_max, int32_t n_adapters, const lora_segments_t *segs,
                               void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                               size_t ws_bytes, void *stream);

/* Measurement aid: lora_linear_profiled for lora_linear_fp8w's arguments. */
lora_status_t lora_linear_fp8w_profiled(const void *x, const void *W8, const float *w_scale,
                                        const void *A, const void *B, const float *scale,
                                        const int32_t *ranks, const int32_t *ids, int32_t M,
                                        int32_t d_in, int32_t d_out, int32_t r_max,
                                        int32_t n_adapters, const lora_segments_t *segs, void *y,
                                        lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                        size_t ws_bytes, void *stream, float *kernel_ms,
                                        const char **kernel_names, int32_t max_kernels,
                                        int32_t *n_kernels);

/* For callers that cannot allocate (code under HIP graph capture, serving loops or
 * harnesses that forbid hipMalloc): lora_linear without a caller workspace.  The call uses a
 * scratch array of LORA_NOALLOC_SCRATCH_BYTES that the library keeps in device memory, one
 * per GPU (held until the process ends; its device address is looked up once per device,
 * at the first call on it), and calls no hipMalloc, hipFree or allocating routine.  Every
 * call on one GPU shares that scratch: calls that overlap in time on one GPU (other streams,
 * other host threads) race on it and must be serialised by the caller.  No part of the
 * scratch needs clearing between calls.  Returns LORA_ERR_WORKSPACE when the call would need
 * more than LORA_NOALLOC_SCRATCH_BYTES (lora_workspace_bytes() of its sizes: decode batches
 * up to 256 rows at 4096 x 11008, and prefill batches of 4096 rows at 4096 x 4096, fit);
 * otherwise the statuses and the result of lora_linear with the same arguments. */
#define LORA_NOALLOC_SCRATCH_BYTES (32u << 20)
lora_status_t lora_linear_noalloc(const void *x, const void *W, const void *A, const void *B,
                                  const float *scale, const int32_t *ranks, const int32_t *ids,
                                  int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                  int32_t n_adapters, const lora_segments_t *segs, void *y,
                                  lora_dtype_t y_dtype, lora_mode_t mode, void *stream);

/* Measurement aid, not for serving loops (it times the per-kernel costs that [P1], "How does
 * one batch run 30 different adapters at once?", attributes to decode and prefill; the pages
 * define no such call): the same launches as lora_linear, each launched
 * with a start and a stop HIP event that the GPU stamps from that kernel's own dispatch (no
 * extra packet between kernels), so the times are kernel durations.  It then waits for the
 * last kernel and writes, in launch order, each kernel's duration in milliseconds to
 * kernel_ms[i] and its name (a static string) to kernel_names[i], for at most max_kernels
 * kernels; *n_kernels receives the number written.  kernel_ms, kernel_names and n_kernels
 * are HOST pointers.  Creates and destroys its own events; not for use during graph capture. */
lora_status_t lora_linear_profiled(const void *x, const void *W, const void *A, const void *B,
                                   const float *scale, const int32_t *ranks, const int32_t *ids,
                                   int32_t M, int32_t d_in, int32_t d_out, int32_t r_max,
                                   int32_t n_adapters, const lora_segments_t *segs, void *y,
                                   lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                   size_t ws_bytes, void *stream, float *kernel_ms,
                                   const char **kernel_names, int32_t max_kernels,
                                   int32_t *n_kernels);

/* MoE-LoRA ([P3], "MoE Models Raise the Bar": in a routed expert layer each adapted
 * projection of each expert carries the request's adapter, and the adapter's shrink and
 * expand are folded into the expert-routed kernel, with split-K for the skinny products).
 * Token m is routed to top_k experts topk_ids[m][j] (-1: the slot has no expert) with
 * routing weights topk_w[m][j]; it carries adapter ids[m] (-1: the bare base).  Per (token,
 * slot), with e = topk_ids[m][j] and i = ids[m]:
 *     y[m][j][:] = topk_w[m][j] * ( x[m] W[e] + scale_i (x[m] A[i][e]) B[i][e] )
 * (the adapter term only when i >= 0) and y[m][j][:] = 0 for a slot with no expert.  Layouts,
 * row-major, device memory, 16-byte aligned:
 *   x         bf16 [M][d_in]                 W   bf16 [n_experts][d_in][d_out]
 *   A         bf16 [n_adapters][n_experts][d_in][r_max]  (zero past each adapter's rank)
 *   B         bf16 [n_adapters][n_experts][r_max][d_out] (zero past each adapter's rank)
 *   scale     fp32 [n_adapters] = alpha_i / r_i;  ranks int32 [n_adapters] (NULL: all r_max)
 *   ids       int32 [M];  topk_ids int32 [M][top_k];  topk_w fp32 [M][top_k] (NULL: weight 1)
 *   y         bf16 or fp32 [M][top_k][d_out] (per slot; the caller sums slots if it wants)
 * Limits: 1 <= top_k <= 64, 1 <= n_experts <= 4096, M * top_k <= LORA_MOE_MAX_PAIRS, d_in a
 * multiple of 32 and at least 128, d_out a multiple of 8 (else LORA_ERR_SHAPE); r_max a
 * multiple of 8 in [8, 64] (else LORA_ERR_RANK).  mode: LORA_MODE_AUTO or LORA_MODE_DECODE
 * (else LORA_ERR_MODE), LORA_MODE_CHECKED may be OR-ed in: it also reports a topk_ids entry
 * outside [-1, n_experts) as LORA_ERR_BAD_ID.  Without it, such a slot is a zero row and an
 * id outside [-1, n_adapters) adds no adapter term.  ws: at least lora_moe_workspace_bytes()
 * of the same sizes, 256-byte aligned, contents need not be initialised.  M = 0 is a no-op.
 * Two launches on `stream`, no allocation, no host synchronisation (except checked mode). */
#define LORA_MOE_MAX_PAIRS 8192
size_t lora_moe_workspace_bytes(int32_t M, int32_t top_k, int32_t n_experts, int32_t d_in,
                                int32_t d_out, int32_t r_max, int32_t n_adapters);
lora_status_t lora_moe_linear(const void *x, const void *W, const void *A, const void *B,
                              const float *scale, const int32_t *ranks, const int32_t *ids,
                              const int32_t *topk_ids, const float *topk_w, int32_t M,
                              int32_t top_k, int32_t n_experts, int32_t d_in, int32_t d_out,
                              int32_t r_max, int32_t n_adapters, void *y, lora_dtype_t y_dtype,
                              lora_mode_t mode, void *ws, size_t ws_bytes, void *stream);

/* Measurement aid: lora_linear_profiled for lora_moe_linear's arguments. */
lora_status_t lora_moe_linear_profiled(const void *x, const void *W, const void *A, const void *B,
                                       const float *scale, const int32_t *ranks,
                                       const int32_t *ids, const int32_t *topk_ids,
                                       const float *topk_w, int32_t M, int32_t top_k,
                                       int32_t n_experts, int32_t d_in, int32_t d_out,
                                       int32_t r_max, int32_t n_adapters, void *y,
                                       lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
                                       size_t ws_bytes, void *stream, float *kernel_ms,
                                       const char **kernel_names, int32_t max_kernels,
                                       int32_t *n_kernels);

/* Measurement aid: lora_linear_profiled for lora_linear_compact's arguments. */
lora_status_t lora_linear_compact_profiled(
    const void *x, const void *W, const void *A, const void *B, const float *scale,
    const int32_t *ranks, const int32_t *rank_offsets, int32_t pool_rows, const int32_t *ids,
    int32_t M, int32_t d_in, int32_t d_out, int32_t r_max, int32_t n_adapters,
    const lora_segments_t *segs, void *y, lora_dtype_t y_dtype, lora_mode_t mode, void *ws,
    size_t ws_bytes, void *stream, float *kernel_ms, const char **kernel_names,
    int32_t max_kernels, int32_t *n_kernels);

/* Human-readable name of a status (error reporting of this ABI; no passage of the pages
 * defines it).  Never NULL; unknown values give "unknown lora_status_t". */
const char *lora_status_string(lora_status_t status);

/* The HIP error string of the last call on this host thread that returned LORA_ERR_HIP
 * ("no error" otherwise).  Each call clears errors that were pending before it. */
const char *lora_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
