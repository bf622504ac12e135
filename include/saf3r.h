/*
 * saf3r.h -- C ABI of the MI355X (gfx950) head-wise dynamic sparse global
 * attention library (libsaf3r.so).
 *
 * The operation is the one described in "SAF3R: Dynamic Sparse Attention for
 * Feed-Forward 3D Reconstruction Transformers" (arXiv 2607.03612): every head
 * of a cross-view global attention layer is given a role, each role selects
 * a key/value set per query, and attention is computed exactly over that set
 * (softmax over the selected logits, scale 1/sqrt(d)):
 *
 *   O[h, i] = sum_{j in K_h(i)} softmax_j(q_i . k_j / sqrt(d)) v_j
 *
 * Roles (Sec. 3 Observation #2; Sec. 4.1 "Tailored Sparse Attention Kernels"):
 *   SAF_POSITION       static set: every special token, every token of the
 *                      anchor frame and every token of the query's own frame.
 *   SAF_VERTICAL       one set shared by all queries: the top-`budget` keys of
 *                      the mean-query probe qbar K^T / sqrt(d), where qbar is
 *                      the mean of all N queries (Sec. 4.3, "Query-Probe
 *                      Top-K Kernel").  Ties go to the lower token index.
 *   SAF_CORRESPONDENCE per-query set: the cached DINO cosine top-K of the
 *                      query's patch against the patches of the other frames
 *                      (Sec. 4.1 "DINO Top-K Kernel", Sec. 4.3).  Special
 *                      tokens carry no DINO feature; their queries attend to
 *                      every key.
 *   SAF_SCANNING       keys on a fixed stride `budget` of the global token
 *                      index (phase 0) plus every special token (Sec. 4.1
 *                      "Uniform Sampling Kernel").
 *   SAF_DENSE          every key (full global attention).
 *   SAF_CORR_STRIDE    a patch query's cached correspondence keys united with
 *                      the SAF_SCANNING set of stride `budget` (the union the
 *                      paper names, in its analysis of the DINO Top-K kernel,
 *                      to cover regions DINO features miss); special queries
 *                      attend to every key.
 *   SAF_BROADCAST      static set that broadcasts the first frame's local
 *                      attention map to the other frames (Sec. 4.1 "Static
 *                      Kernel", given there as an example): a patch query at
 *                      grid position (y, x) attends, in every frame, to the
 *                      patches (y', x') with |y' - y| <= r and |x' - x| <= r,
 *                      plus every special token.  r = `budget`; the grid is
 *                      `anchor_frame` patches wide (rows of that many patches,
 *                      row-major), or, with anchor_frame = 0, one row of P
 *                      patches (a window along the patch index).  Special
 *                      queries attend to every key.
 *
 * Token layout: frame f holds T = ns + P tokens, the ns special tokens
 * (camera, registers) first, then P patch tokens; token j = f * T + t.  Patch
 * number u = f * P + p is token f * T + ns + p.  Key sets are sets: a token
 * is never counted twice.
 *
 * Conventions for every call:
 *   - Pointers named dev_* / q / k / v / o / ws / dino are device pointers;
 *     the caller owns them.  The context owns only the correspondence index
 *     cache and small internal buffers.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     the call returns without waiting.  Argument errors are detected on the
 *     host, before anything is enqueued, and returned synchronously; faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - No call throws.  On error the status is returned and a message is kept
 *     in the context (saf_last_error).  A context is not thread-safe; separate
 *     contexts are independent.
 *   - Q, K, V and O share one element type (geometry.dtype) and one layout:
 *     element (h, j, c) sits at h * head_stride + j * token_stride + c, with
 *     the d channels contiguous.  [H, N, d] and [N, H, d] are both covered.
 *     Rows must be 16-byte aligned (head_stride, token_stride multiples of 8
 *     for bf16 and 4 for fp32; base pointers 16-byte aligned).
 *   - head_dim must be 64.
 */
#ifndef SAF3R_H
#define SAF3R_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SAF_OK = 0,
    SAF_EINVAL = -1,        /* bad argument (null pointer, size, role, budget, layout) */
    SAF_ENOMEM = -2,        /* device or host allocation failed */
    SAF_EHIP = -3,          /* the HIP runtime reported an error */
    SAF_EUNSUPPORTED = -4,  /* valid request outside what the library implements */
    SAF_ESTATE = -5         /* call out of order (e.g. no correspondence index yet) */
} saf_status_t;

typedef enum { SAF_F32 = 0, SAF_BF16 = 1 } saf_dtype_t;

typedef enum {
    SAF_POSITION = 0,
    SAF_VERTICAL = 1,
    SAF_CORRESPONDENCE = 2,
    SAF_SCANNING = 3,
    SAF_DENSE = 4,
    SAF_CORR_STRIDE = 5,
    SAF_BROADCAST = 6
} saf_role_t;

/* Correspondence top-K per query: over all other frames together, or K per
 * other frame. */
typedef enum { SAF_CORR_TOTAL = 0, SAF_CORR_PER_FRAME = 1, SAF_CORR_PER_FRAME_STORED = 2 } saf_corr_mode_t;

typedef struct {
    int32_t num_frames;          /* S >= 1 */
    int32_t specials_per_frame;  /* ns >= 0 (5 for VGGT: 1 camera + 4 register) */
    int32_t patches_per_frame;   /* P >= 1 */
    int32_t num_heads;           /* H, 1..64 */
    int32_t head_dim;            /* d, must be 64 */
    int32_t dtype;               /* saf_dtype_t of Q, K, V, O */
} saf_geometry_t;

typedef struct {
    int64_t head_stride;   /* elements between heads */
    int64_t token_stride;  /* elements between tokens */
} saf_layout_t;

typedef struct {
    int32_t role;          /* saf_role_t */
    int32_t budget;        /* VERTICAL: K >= 1 (clamped to N); SCANNING: stride >= 1;
                              CORRESPONDENCE: 0, the cached index's row length Kc
                              or the K requested when it was built (before
                              clamping); CORR_STRIDE: stride >= 1; BROADCAST:
                              window radius r >= 0; others: 0 */
    int32_t anchor_frame;  /* POSITION: anchor frame in [0, S); BROADCAST: patch
                              grid width, a divisor of P, or 0; others ignored */
    int32_t flags;         /* must be 0 */
} saf_head_plan_t;

typedef struct saf_ctx saf_ctx_t;

/* Create a context for one geometry.  Touches no device.  *out receives the
 * context; NULL on failure.  Errors: SAF_EINVAL (bad geometry, or N = S (ns +
 * P) >= 2^30),
 * SAF_EUNSUPPORTED (head_dim != 64), SAF_ENOMEM. */
saf_status_t saf_create(const saf_geometry_t *geometry, saf_ctx_t **out);

/* Release the context and its device memory (waits for the device). NULL ok. */
void saf_destroy(saf_ctx_t *ctx);

/* Message of the last failing call on this context ("" if none).  Valid until
 * the next call on the context.  With ctx == NULL: the last saf_create error. */
const char *saf_last_error(const saf_ctx_t *ctx);

/* Bytes of device workspace that saf_sparse_attention / saf_dense_attention /
 * saf_build_vertical_index need for this plan (plan: H entries, host memory;
 * NULL = the dense call).  The workspace needs no initialisation. */
saf_status_t saf_workspace_size(const saf_ctx_t *ctx, const saf_head_plan_t *plan, size_t *bytes);

/* Build the correspondence index (Sec. 4.3, "DINO Top-K Kernel") from DINO
 * features of the S*P patches (row u = patch number u, Df channels contiguous,
 * rows dino_row_stride elements apart, dtype dino_dtype, 16-byte aligned rows).
 * For every patch u: cosine c_uv = f_u.f_v / (|f_u||f_v|) (0 when a norm is 0)
 * against the patches v of the other frames, ranked by (c desc, token asc).
 *   SAF_CORR_TOTAL:     the first min(K, (S-1)P) over all other frames;
 *                       Kc = that count (at most 1024).
 *   SAF_CORR_PER_FRAME: the first min(K, P) of every other frame (P <= 4096);
 *                       Kc = (S-1) min(K, P).  With bf16 features, Df a
 *                       multiple of 64, P >= 256 and K <= 8 the cosines are
 *                       never stored: a pass over a 128-patch sample of
 *                       every frame bounds each (row, frame)'s K-th best, one
 *                       pass over the symmetric square keeps what reaches
 *                       the bounds, and a row short of candidates is
 *                       recomputed exactly; otherwise as the next mode.
 *   SAF_CORR_PER_FRAME_STORED: the same index built by writing every row's
 *                       cosines (fp32, in row chunks of about 512 MB) and
 *                       selecting each frame's K best from them.
 * Each row of Kc global token indices is stored ascending.  The index is kept
 * in the context and reused by every later saf_sparse_attention call (the
 * cache of Sec. 4.3) until rebuilt.  The device scratch the build needs is
 * owned by the context (allocated on first use, grown when a larger build
 * needs more).
 * Errors: SAF_EINVAL (S < 2, K < 1, Df < 1, bad mode/stride/pointer),
 * SAF_EUNSUPPORTED (Df > 4096, TOTAL with Kc > 1024, the per-frame modes
 * with P > 4096), SAF_ENOMEM. */
saf_status_t saf_build_corr_index(saf_ctx_t *ctx, const void *dino, int32_t dino_dtype,
                                  int32_t Df, int64_t dino_row_stride, int32_t K,
                                  int32_t mode, void *stream);

/* Correspondence index taken from one head's own attention logits instead
 * of DINO features (the first direction the paper names for improving the
 * DINO Top-K kernel: indices from the first correspondence head).  For every
 * patch u (token i) the patch tokens j of other frames are ranked by
 * (q_i . k_j desc, token asc) -- the 1/sqrt(d) scale does not change the
 * order -- using head `head` of q and k (context dtype, layout as for
 * attention); TOTAL keeps the first min(K, (S-1)P) (at most 1024), PER_FRAME
 * (or PER_FRAME_STORED, the same build here: q and k differ, so the cosine
 * rows are always written) the first min(K, P) of every other frame.  The result replaces the cached
 * index exactly like saf_build_corr_index and serves every later
 * correspondence head.
 * Errors: SAF_EINVAL (S < 2, bad head/K/mode/layout/pointer),
 * SAF_EUNSUPPORTED (TOTAL with Kc > 1024, the per-frame modes with P > 4096),
 * SAF_ENOMEM. */
saf_status_t saf_build_corr_index_qk(saf_ctx_t *ctx, const void *q, const void *k, saf_layout_t layout,
                                     int32_t head, int32_t K, int32_t mode, void *stream);

/* Block-wise variant of the correspondence index (Sec. 4.3: block-level
 * similarities averaged over tokens, a cheaper build).  A block is `block`
 * consecutive patches of one frame (block must divide P; block = the patch
 * grid width makes it one row of patches).  The similarity of blocks A and B
 * is the token cosine averaged over their block x block patch pairs, i.e. the
 * dot product of the blocks' mean unit features (fp32; zero features count
 * as 0).  For every query block the blocks of other frames are ranked by
 * (similarity desc, block asc):
 *   SAF_CORR_TOTAL:     the first min(K, (S-1)P/block) blocks (at most 1024);
 *   SAF_CORR_PER_FRAME: the first min(K, P/block) of every other frame.
 * Every patch of the query block gets the patches of those blocks, so
 * Kc = kept blocks * block global token indices per row, ascending.  The
 * result replaces the cached index exactly like saf_build_corr_index, and a
 * correspondence head's budget may name Kc or the K kept here.
 * Errors: SAF_EINVAL (S < 2, K < 1, Df < 1, block not dividing P, bad
 * mode/stride/pointer), SAF_EUNSUPPORTED (Df > 4096, too many blocks),
 * SAF_ENOMEM. */
saf_status_t saf_build_corr_index_blocks(saf_ctx_t *ctx, const void *dino, int32_t dino_dtype,
                                         int32_t Df, int64_t dino_row_stride, int32_t block,
                                         int32_t K, int32_t mode, void *stream);

/* Replace the cached index with caller data: dev_idx holds S*P rows of Kc
 * global token indices (int32, device memory), each row a set of distinct
 * patch tokens of other frames.  The data is copied (stream-ordered).
 * Errors: SAF_EINVAL (S < 2, Kc < 1, Kc > (S-1)P, null pointer), SAF_ENOMEM. */
saf_status_t saf_set_corr_index(saf_ctx_t *ctx, const int32_t *dev_idx, int32_t Kc, void *stream);

/* Copy the cached index ([S*P, Kc] int32, rows ascending) to dev_out (may be
 * NULL to query Kc only).  Errors: SAF_ESTATE (no index), SAF_EINVAL. */
saf_status_t saf_get_corr_index(const saf_ctx_t *ctx, int32_t *dev_out, int32_t *Kc, void *stream);

/* Diagnostics of the last index build (saf_build_corr_index or
 * saf_build_corr_index_qk in SAF_CORR_TOTAL mode with bf16 operands, the
 * matrix-core engine, or saf_build_corr_index's fused SAF_CORR_PER_FRAME
 * build): the patch numbers of the rows whose fast pass could not prove its
 * result exact (a candidate buffer overflowed, the row's top-K threshold
 * guessed for the filtered pass was not confirmed, or a frame kept fewer
 * than K candidates) and which were therefore recomputed exactly.  Writes min(*count, max_rows) patch numbers,
 * in no particular order, to host_rows (host memory; may be NULL with
 * max_rows = 0) and the number of such rows to *count.  Unlike the other
 * calls this one is synchronous: it waits for `stream`, on which the build
 * must have been enqueued.  The list is the build's own bookkeeping and does
 * not change the index (Sec. 4.3 defines only the top-K itself).
 * Errors: SAF_EINVAL (null ctx/count, max_rows < 0, host_rows NULL with
 * max_rows > 0), SAF_ESTATE (no build, or the last build kept no list: the
 * stored-cosine per-frame build, block-wise, fp32 features, an imported
 * index), SAF_EHIP. */
saf_status_t saf_corr_recomputed_rows(saf_ctx_t *ctx, int32_t *host_rows, int32_t max_rows,
                                      int32_t *count, void *stream);

/* Vertical-line key set of one head (Sec. 4.3): qbar = mean of the N query
 * rows of head `head` (fp32), r_j = qbar . k_j / sqrt(d) (fp32), the top
 * min(K, N) by (r desc, j asc), written ascending to dev_idx_out (int32).
 * ws: workspace of at least saf_workspace_size() for a plan holding this
 * head as VERTICAL with budget K.  Errors: SAF_EINVAL. */
saf_status_t saf_build_vertical_index(saf_ctx_t *ctx, const void *q, const void *k,
                                      saf_layout_t layout, int32_t head, int32_t K,
                                      int32_t *dev_idx_out, void *ws, size_t ws_bytes,
                                      void *stream);

/* One sparse global-attention layer: every head h by plan[h] (H entries, host
 * memory).  Vertical heads build their key set in this call unless vert_idx
 * is given: then vert_idx + h * vert_ld holds head h's min(K, N) key indices
 * (int32, device, ascending) for every vertical head h.  Correspondence heads
 * use the cached index.  O gets the input element type.
 * Errors: SAF_EINVAL (bad plan/layout/pointer, workspace too small),
 * SAF_ESTATE (a correspondence head and no cached index, or a budget that
 * differs from the index's K), SAF_EHIP. */
saf_status_t saf_sparse_attention(saf_ctx_t *ctx, const saf_head_plan_t *plan, const void *q,
                                  const void *k, const void *v, void *o, saf_layout_t layout,
                                  const int32_t *vert_idx, int64_t vert_ld, void *ws,
                                  size_t ws_bytes, void *stream);

/* saf_sparse_attention for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, bit for bit, with its workspace taken from a
 * static device array of 64 MiB that the library holds on every GPU it runs
 * on until the process ends, instead of a caller's buffer.  The call itself
 * allocates nothing and creates no stream or event: every launch goes on
 * `stream` (the regular entry point runs the gathered rows on a side stream)
 * and per-launch timing is skipped.  Inputs, outputs, the cached index and
 * vert_idx are as for saf_sparse_attention.  The array needs no clearing
 * (every kernel writes the parts it reads first), but every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other contexts, other host threads) race and must be serialised by the
 * caller.  Errors: as saf_sparse_attention, plus SAF_EUNSUPPORTED when the
 * plan's workspace (saf_workspace_size, less the vertical sets' share when
 * vert_idx is given) exceeds 64 MiB. */
saf_status_t saf_sparse_attention_noalloc(saf_ctx_t *ctx, const saf_head_plan_t *plan, const void *q,
                                          const void *k, const void *v, void *o, saf_layout_t layout,
                                          const int32_t *vert_idx, int64_t vert_ld, void *stream);

/* Dense global attention over every key, all heads: O = softmax(Q K^T /
 * sqrt(d)) V over the N x N logits that the sparse kernels avoid (the full
 * pre-softmax attention matrix of Sec. 4.3, whose column means the query
 * probe reproduces; the "Full" row of Sec. 5.3, Table 6).  This is the
 * speedup baseline and the reference output of the profiling error of
 * Eq. 1 (Sec. 4.2).  Layout and dtype as for saf_sparse_attention; ws: at
 * least saf_workspace_size(ctx, NULL) bytes, 16-byte aligned (bf16: the
 * heads' largest key norms, which bound every logit and give the softmax a
 * fixed shift; fp32 needs none and ws may be NULL).  Errors: SAF_EINVAL (null
 * or misaligned pointer, bad layout, workspace too small), SAF_EHIP. */
saf_status_t saf_dense_attention(saf_ctx_t *ctx, const void *q, const void *k, const void *v,
                                 void *o, saf_layout_t layout, void *ws, size_t ws_bytes,
                                 void *stream);

/* Per-launch timing (tracing).  With enable != 0 every kernel launch group
 * the context enqueues (one entry per group: "shared_attention",
 * "gather_attention", "split_combine", "vertical_index", "corr_index",
 * "dense_attention") is bracketed by two HIP events on the call's stream.
 * Timing adds two event records per launch group and nothing else; it is
 * off by default.  Errors: SAF_EINVAL. */
saf_status_t saf_set_kernel_timing(saf_ctx_t *ctx, int32_t enable);

/* Read and clear the recorded launches.  Call after the streams involved
 * have been synchronised.  Writes up to max entries (names: static strings,
 * ms: elapsed milliseconds) and the total number recorded to *count.
 * Errors: SAF_EINVAL (null ctx/count), SAF_EHIP (an event is not complete). */
saf_status_t saf_read_kernel_timing(saf_ctx_t *ctx, int32_t max, const char **names, float *ms,
                                    int32_t *count);

/* Testing hook for the error paths: after `allowed` further successful
 * device allocations by this library (process-wide, every context), each
 * allocation fails as if the device were out of memory, so the calling entry
 * point returns SAF_ENOMEM with its message.  allowed < 0 removes the limit
 * (the default).  A failed index build or copy leaves the previously cached
 * index untouched when the failure happens before anything is enqueued.
 * Always returns SAF_OK.  Host only. */
saf_status_t saf_debug_fail_alloc(int32_t allowed);

/* ---- Offline head profiling (Sec. 4.2) ---------------------------------- */

/* Error sums of Eq. 1 for every head: dev_out[2h] = sum over the head's N x d
 * outputs of (o_full - o_sparse)^2 and dev_out[2h + 1] = sum of o_full^2,
 * accumulated in fp64 in a fixed order (dev_out: 2H doubles, device memory).
 * Both outputs have the context's dtype and the given layout.  The context
 * keeps a small partial-sum buffer (allocated on first use).
 * Errors: SAF_EINVAL (null pointer, bad layout), SAF_ENOMEM, SAF_EHIP. */
saf_status_t saf_head_nmse(saf_ctx_t *ctx, const void *o_full, const void *o_sparse, saf_layout_t layout,
                           double *dev_out, void *stream);

/* Eq. 1 for every head, accumulated over calibration samples: with the
 * sums above, dev_err[h * err_stride] += weight * sum (o_full - o_sparse)^2 /
 * sum o_full^2 (fp64; a head whose full output is all zero adds NaN, where
 * the definition has no value).  Called once per calibration sample with
 * weight = 1 / (number of samples) on a zeroed accumulator, it leaves E(c) of
 * Eq. 1 -- the expectation over the calibration set of each head's
 * normalised squared error -- in dev_err (device memory, the caller's; the
 * stride lets one [H, configurations] table collect every configuration).
 * Stream-ordered like every other call.  Errors: SAF_EINVAL (null pointer,
 * bad layout, err_stride < 1, a weight that is negative or not finite),
 * SAF_ENOMEM, SAF_EHIP. */
saf_status_t saf_head_nmse_accumulate(saf_ctx_t *ctx, const void *o_full, const void *o_sparse,
                                      saf_layout_t layout, double weight, double *dev_err,
                                      int64_t err_stride, void *stream);

/* Query-key pairs one head computes under *head at this geometry (its
 * floating-point work, the cost of Eq. 2, is 4 head_dim per pair).  For a
 * correspondence head corr_kc is the index row length (<= 0: the cached
 * index's).  Host only.  Errors: SAF_EINVAL (bad role/budget/anchor, a
 * broadcast grid width that does not divide P), SAF_ESTATE (correspondence
 * with no row length). */
saf_status_t saf_head_pairs(const saf_ctx_t *ctx, const saf_head_plan_t *head, int32_t corr_kc,
                            int64_t *pairs);

/* Eq. 2's cost Omega(c) of one head under *head (Sec. 4.2): its floating-point
 * work, 4 head_dim per query-key pair (2 head_dim for q.k, 2 head_dim for
 * p.v) over the pairs saf_head_pairs counts, written to *flops.  Host only.
 * Errors: as saf_head_pairs, and SAF_EINVAL for a null flops. */
saf_status_t saf_head_cost(const saf_ctx_t *ctx, const saf_head_plan_t *head, int32_t corr_kc, double *flops);

/* Eq. 2 by progressive substitution: entry 0 is the baseline; walking
 * entries 1 .. n-1 in order, an entry replaces the current choice when its
 * error is strictly lower and its cost does not exceed the baseline's.
 * Returns the chosen index, or -1 for n < 1 or null arrays.  Host only. */
int32_t saf_profile_select(const double *errors, const double *costs, int32_t n);

/* Stride of the uniform-sampling baseline with sparsity ratio sigma in
 * [0, 1): the smallest stride keeping at most a fraction 1 - sigma of the
 * keys.  Returns -1 for sigma outside [0, 1).  Host only. */
int32_t saf_baseline_stride(double sigma);

#ifdef __cplusplus
}
#endif

#endif /* SAF3R_H */
