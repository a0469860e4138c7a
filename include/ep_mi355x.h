/*
 * ep_mi355x.h: C ABI of the MI355X (gfx950) MoE expert-parallel hot path,
 * taken at one GPU's share: every expert is resident locally (a world of
 * one), so there are no peers and no collectives.
 *
 *   ep_layout    topk_idx -> per-expert counts, aligned exclusive offsets,
 *                a destination slot per (token, k), receive metadata
 *   ep_dispatch  permute-copy token rows (bf16, fp32, or fp8 e4m3 / fp4x2
 *                bytes with optional fp32 per-128-value scales) into the
 *                expert-major expand buffer
 *   ep_combine   gather each token's top-k expert-output rows (bf16 or fp32),
 *                weight them by the router weights, sum in binary32 in k
 *                order, store in the rows' type
 *
 * and around them: ep_layout_dispatch (layout + dispatch in one launch for a
 * one-tile batch), the non-expand mode (ep_dispatch_compact,
 * ep_combine_compact, ep_layout_dispatch_compact: one row per received
 * token), ep_zero_padding (zero the alignment rows), the CU-limited mode
 * (ep_set_workgroup_limit / ep_get_workgroup_limit) and the helpers
 * ep_layout_workspace_bytes, ep_layout_dispatch_workspace_bytes, ep_supported
 * and ep_last_error; ep_layout_noalloc
 * runs ep_layout on a fixed scratch array for callers that cannot allocate.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers owned by the caller; the library
 *   never allocates, frees, copies to the host or synchronises. Every call
 *   only enqueues kernels on `stream` (a hipStream_t passed as void*; NULL
 *   is the default stream) and returns; results are ready when the stream
 *   reaches that point. Calls are stream-ordered and capturable.
 * - Arrays are dense and row-major with the shapes given below. Row pointers
 *   of x, expand_x, expert_out, out and the scale arrays must be 16-byte
 *   aligned; int32 / fp32 arrays 4-byte aligned.
 * - Return value: EP_OK (0) on success, a negative EP_E* code on error.
 *   Arguments are checked on the host before anything is enqueued; on an
 *   error nothing is launched and ep_last_error() returns a message (per
 *   calling thread). No entry point throws or aborts.
 * - Shapes (hidden, topk, dtype) select kernels compiled ahead of time with
 *   those values as template constants; a shape outside the compiled set is
 *   rejected with EP_EUNSUPPORTED before any work (capability gate).
 * - dtype numbering follows the MORI v2 EpDType enumeration ("MORI JIT v2",
 *   section 3.7): bf16 = 0, fp32 = 1, fp8 = 2, fp4x2 = 3.
 *
 * Sources: "DeepEP 整体架构分析" (DeepEP overall architecture), the EPHandle
 * structure and the dispatch / combine data-flow figure; "MORI JIT v2",
 * section 3.5 (invalid configurations are rejected before any work: token
 * bytes 16-byte aligned, topk within one wavefront, receive capacity covers
 * the worst case), section 3.7 (dtype is a transport attribute: dispatch
 * moves bytes, combine reduces and rejects byte dtypes), section 4 (no
 * compile, allocation or host synchronisation on the launch path; graph
 * capture), section 6 (every C entry point reports errors by return value
 * plus a last-error string).
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define EP_OK 0
#define EP_EINVAL (-1)        /* an argument is out of range or misaligned        */
#define EP_EUNSUPPORTED (-2)  /* no compiled kernel for this (hidden, topk, dtype) */
#define EP_ECAPACITY (-3)     /* capacity_rows cannot hold the worst case          */
#define EP_EHIP (-4)          /* the HIP runtime reported an error on launch       */

/* Element types (MORI v2 EpDType numbering). */
#define EP_BF16 0
#define EP_FP32 1
#define EP_FP8_E4M3 2
#define EP_FP4X2 3

/* Largest expert count and top-k the layout kernels accept. */
#define EP_MAX_EXPERTS 1024
#define EP_MAX_TOPK 64

/*
 * Bytes of device workspace ep_layout needs for (num_tokens, topk,
 * num_experts): per-tile expert histograms and per-tile received-token
 * counts passed between its kernels when num_tokens*topk is above 2^14
 * (smaller inputs take one launch and need none: the result is 0), plus,
 * when there are many tiles per expert, their per-tile prefixes and totals.
 * Returns 0 for out-of-range arguments. The workspace is scratch: its
 * contents on entry do not matter and are overwritten; two ep_layout calls
 * in flight at once must not share one workspace.
 */
size_t ep_layout_workspace_bytes(int32_t num_tokens, int32_t topk, int32_t num_experts);

/*
 * Workspace bytes that let ep_layout_dispatch walk a dispatch plan: the
 * layout's own workspace (ep_layout_workspace_bytes), rounded up to 256 bytes,
 * plus 8 bytes per (token, k) entry for the plan. ep_layout_dispatch needs
 * only ep_layout_workspace_bytes; given this much, a batch of more than one
 * layout tile also has the layout write the plan into the tail of the
 * workspace and dispatch follow it (measured on MI355X: prefill step 171.4
 * against 176.4 us, mori_default 47.9 against 49.7; with x evicted from the
 * last-level cache 193.5 against 232.1, 52.9 against 63.5). Results are
 * identical either way. Returns 0 for out-of-range arguments.
 */
size_t ep_layout_dispatch_workspace_bytes(int32_t num_tokens, int32_t topk, int32_t num_experts);

/*
 * Routing layout (DeepEP overall architecture, EPHandle fields
 * num_unaligned_recv_tokens_perpert, psum_num_recv_tokens_per_expert,
 * dst_buffer_slot_idx, recv_src_metadata, num_recv_tokens,
 * num_expanded_tokens; in the dispatch data-flow figure the notify warps count
 * entries per expert and compute each entry's target slot).
 *
 * Inputs
 *   topk_idx          int32 [num_tokens, topk]: expert id of each (t, k);
 *                     an id outside [0, num_experts) masks the entry
 *                     (it gets no slot and is not counted).
 *   num_tokens        T >= 0
 *   topk              K in 1 .. EP_MAX_TOPK (compiled set, see EP_EUNSUPPORTED)
 *   num_experts       E in 1 .. EP_MAX_EXPERTS
 *   expert_alignment  A >= 1: every expert segment is padded to a multiple of A
 *   capacity_rows     rows of the expand buffer the caller will dispatch into;
 *                     must be >= T*K + E*(A-1) (the worst case), else
 *                     EP_ECAPACITY
 * Outputs (device, written in full unless noted)
 *   counts            int32 [E]: unmasked entries routed to each expert
 *   offsets           int32 [E+1]: offsets[0] = 0, offsets[e+1] = offsets[e]
 *                     + A*ceil(counts[e]/A); offsets[E] = num_expanded_tokens
 *   dst_slot          int32 [T, K]: expand row of (t, k), or -1 when masked.
 *                     Inside an expert segment rows are handed out in
 *                     token-major (t, then k) order starting at offsets[e];
 *                     the padding rows of a segment belong to nobody.
 *   recv_src_metadata int32 [T, K+2]: row i describes the i-th token (in
 *                     ascending t) with at least one unmasked entry:
 *                     [t, source rank (always 0 here), dst_slot[t, 0..K-1]].
 *                     Rows i >= *num_recv are left untouched.
 *   num_recv          int32 [1]: number of such tokens (stays on the device)
 *   workspace         device scratch of >= ep_layout_workspace_bytes(T, K, E)
 *   dispatch_plan     optional (NULL: not written), int32 [T*K, 2], 8-byte
 *                     aligned: the order in which ep_dispatch copies rows
 *                     fastest. The entries are cut into tiles of whole tokens,
 *                     floor(W / K) tokens each, where W = 1024 for E <= 256,
 *                     512 for E <= 512 and 256 above. Each tile's span
 *                     lists its unmasked entries by ascending slot as
 *                     (t*K + k, dst_slot[t, k]), then (-1, -1) once per
 *                     masked entry. This array is not part of the pages'
 *                     handle: it is a gfx950-specific write-order aid, and
 *                     every other output is the same with or without it.
 *                     Measured on MI355X (steps with ep_dispatch following
 *                     the plan against token-major): prefill with 470 MB of
 *                     rows 167.5 against 175.9 us with the rows cached,
 *                     190.9 against 231.5 us with them evicted; mori_default
 *                     (1024 tokens) 46.0 against 49.7 and 52.5 against
 *                     63.5 us. The layout pays 0.1-0.4 us for it.
 *   prefetch,         optional read-ahead (NULL and 0: none): device memory
 *   prefetch_bytes    the caller reads next, typically the token rows x
 *                     (and their scale rows) that ep_dispatch copies. The
 *                     layout leaves most compute units idle; workgroups
 *                     added to its launches read one 4-byte word of every
 *                     128-byte line of the first min(prefetch_bytes, 128 MiB)
 *                     bytes with ordinary loads, which brings those lines
 *                     into the last-level cache while the layout runs. It
 *                     reads only inside [prefetch, prefetch + prefetch_bytes),
 *                     writes nothing there and changes no result. Ignored
 *                     under a workgroup cap. The pointer must be 4-byte
 *                     aligned; NULL with nonzero bytes is EP_EINVAL.
 *                     Measured on MI355X (prefill step, 4096 tokens of
 *                     hidden 7168, 58.7 MB of rows): with the rows not in the
 *                     cache the step takes 177 us with the read-ahead against
 *                     191 us without; with the rows cached, 172 against 167
 *                     us (the reads then only add work). Worth asking for
 *                     when x was produced long before dispatch.
 * Results are a pure function of the inputs (no atomics whose order matters).
 */
int ep_layout(const int32_t *topk_idx, int32_t num_tokens, int32_t topk, int32_t num_experts,
              int32_t expert_alignment, int64_t capacity_rows, int32_t *counts,
              int32_t *offsets, int32_t *dst_slot, int32_t *recv_src_metadata,
              int32_t *num_recv, void *workspace, size_t workspace_bytes,
              int32_t *dispatch_plan, const void *prefetch, size_t prefetch_bytes,
              void *stream);

/*
 * Bytes of the library's fixed layout scratch, one copy per GPU (8 MiB):
 * the largest ep_layout_workspace_bytes() that ep_layout_noalloc accepts. It
 * covers batches of up to 4,176,896 (token, k) entries at 256 experts
 * (522,112 tokens at top-8), 1,046,016 at 512 and 261,632 at 1024; batches
 * of at most 2^14 entries need no scratch at all.
 */
#define EP_LAYOUT_SCRATCH_BYTES 8388608 /* 8 MiB */

/*
 * ep_layout without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, outputs, checks and errors as
 * ep_layout; the workspace is instead a fixed device array of
 * EP_LAYOUT_SCRATCH_BYTES inside the library, one copy per GPU, kept until
 * the process ends. The call allocates nothing: on the first call on a GPU it
 * looks up that GPU's copy (with the GPU current), then only enqueues kernels.
 *
 * Extra rules:
 * - `stream` must belong to the current device (EP_EINVAL otherwise).
 * - ep_layout_workspace_bytes(num_tokens, topk, num_experts) must not exceed
 *   EP_LAYOUT_SCRATCH_BYTES (EP_EINVAL, with the sizes in the message).
 * - Every call on one GPU shares that GPU's scratch and nothing in it is
 *   cleared between calls (no word needs to start at zero): two calls in
 *   flight at once on one GPU (on different streams, or overlapping graph
 *   replays) race and may return wrong results. Calls on one stream are
 *   ordered and safe.
 * - The first call on a GPU fails with EP_EHIP if the runtime cannot resolve
 *   the scratch address; a failed lookup is retried on the next call.
 */
int ep_layout_noalloc(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                      int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                      int32_t *counts, int32_t *offsets, int32_t *dst_slot,
                      int32_t *recv_src_metadata, int32_t *num_recv, int32_t *dispatch_plan,
                      const void *prefetch, size_t prefetch_bytes, void *stream);

/*
 * Dispatch in the expand layout (DeepEP overall architecture, dispatch copy
 * epilogue writing token data and scale factors; "MORI JIT v2", section 3.7:
 * the payload is moved as bytes whatever its dtype, fp8 / fp4x2 arrive
 * already quantised, and for fp4x2 hidden counts bytes).
 *
 * For every (t, k) with 0 <= dst_slot[t, k] < capacity_rows:
 *   expand_x[dst, :]        = x[t, :]            (bytes of one row)
 *   expand_scales[dst, :]   = x_scales[t, :]     (only if both are non-NULL)
 *   expand_weights[dst]     = topk_weights[t, k] (only if both are non-NULL)
 * Rows no entry points at (alignment padding) are not written. Entries
 * outside [0, capacity_rows) are skipped.
 *
 *   x               EP_BF16: bf16 [T, hidden]; EP_FP32: fp32 [T, hidden];
 *                   EP_FP8_E4M3: e4m3 bytes [T, hidden];
 *                   EP_FP4X2: packed e2m1 pairs, [T, hidden] bytes (2*hidden values)
 *   x_scales        fp32 [T, S] with S = values per row / 128, or NULL; only for
 *                   fp8 and fp4x2 (values per row a multiple of 128). The
 *                   scale rows are optional for both byte dtypes, fp8
 *                   included: the payload travels as bytes either way ("MORI
 *                   JIT v2" section 3.7; its HIP backend moves fp8 rows with
 *                   no scales), so fp8 with x_scales = NULL is accepted and
 *                   moves the rows alone, and the multiple-of-128 rule
 *                   applies only when scales are given. A stricter contract,
 *                   fp8 always with scales, is left to the caller.
 *   topk_weights    fp32 [T, K] or NULL
 *   dst_slot        int32 [T, K], as produced by ep_layout
 *   expand_x        [capacity_rows, hidden] of the same element type as x
 *   expand_scales   fp32 [capacity_rows, S], given exactly when x_scales is
 *   expand_weights  fp32 [capacity_rows] or NULL
 *   dispatch_plan   optional (NULL: token-major order): the plan ep_layout
 *                   wrote in the same call as dst_slot. It changes only the
 *                   order of the copies, never their result. Entries of the
 *                   plan outside [0, T*K) and slots outside
 *                   [0, capacity_rows) are skipped. A plan that does not
 *                   match dst_slot copies what the plan says.
 * Errors: EP_EINVAL for a NULL required pointer, misalignment, row bytes
 * not a multiple of 16, scales for bf16 / fp32 or only one scale pointer;
 * EP_EUNSUPPORTED for (hidden, topk, dtype) outside the compiled set.
 */
int ep_dispatch(const void *x, const float *x_scales, const float *topk_weights,
                const int32_t *dst_slot, int32_t num_tokens, int32_t hidden, int32_t topk,
                int32_t dtype, int64_t capacity_rows, void *expand_x, float *expand_scales,
                float *expand_weights, const int32_t *dispatch_plan, void *stream);

/*
 * Layout and dispatch in one call (the DeepEP overall-architecture page,
 * dispatch data-flow figure: the dispatch kernel's notify warps count per
 * expert and compute each token's target slot before the copy epilogue
 * moves the data). It produces everything ep_layout and ep_dispatch produce,
 * with the same arguments, meanings, checks and errors as those two calls
 * (the dispatch arguments take their slots from this layout). When T*K fits
 * one layout tile (the floor(W / K) tokens of ep_layout's dispatch_plan,
 * W = 1024, 512 or 256 by num_experts: a decode step, say) it runs as a
 * single launch: workgroup 0 ranks all entries and writes the layout's
 * outputs, and the copying workgroups find their entries' slots in their own
 * LDS (with expert_alignment 1 and no workgroup cap, by counting the entries
 * whose (expert id, entry index) is smaller; otherwise by ranking all entries
 * as workgroup 0 does). This saves a launch and the trip of dst_slot through
 * memory. Larger batches run the launches of ep_layout and ep_dispatch (no
 * read-ahead), walking a dispatch plan kept in the workspace when the
 * workspace holds ep_layout_dispatch_workspace_bytes, token-major otherwise. Results are identical either way.
 */
int ep_layout_dispatch(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                       int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                       int32_t *counts, int32_t *offsets, int32_t *dst_slot,
                       int32_t *recv_src_metadata, int32_t *num_recv, void *workspace,
                       size_t workspace_bytes, const void *x, const float *x_scales,
                       const float *topk_weights, int32_t hidden, int32_t dtype, void *expand_x,
                       float *expand_scales, float *expand_weights, void *stream);

/*
 * Gather combine (DeepEP overall architecture, combine reduce epilogue
 * weighting expert outputs by topk_weights and adding a bias; "MORI JIT v2",
 * section 3.7: combine reduces bf16 or fp32 rows, writes the same type, and
 * rejects byte dtypes).
 *
 * For every token t and channel h:
 *   acc = +0.0f
 *   for k = 0 .. K-1 with 0 <= dst_slot[t, k] < capacity_rows:
 *       acc = acc + w[t, k] * float(expert_out[dst_slot[t, k], h])
 *   if bias: acc = acc + float(bias[t, h])
 *   out[t, h] = acc stored as dtype (bf16: round to nearest even)
 * Each product and each sum is rounded to binary32 on its own (no fused
 * multiply-add), in k order, so the result is a pure function of the inputs.
 * w[t, k] = topk_weights[t, k], or 1 when topk_weights is NULL.
 *
 *   expert_out      [capacity_rows, hidden] of dtype EP_BF16 or EP_FP32
 *   topk_weights    fp32 [T, K] or NULL
 *   bias            [T, hidden] of the same dtype, or NULL
 *   dst_slot        int32 [T, K]
 *   out             [T, hidden] of the same dtype; every row is written
 * Errors: EP_EINVAL for a byte dtype (fp8 / fp4x2), NULL or misaligned
 * pointers; EP_EUNSUPPORTED for (hidden, topk, dtype) outside the compiled set.
 */
int ep_combine(const void *expert_out, const float *topk_weights, const void *bias,
               const int32_t *dst_slot, int32_t num_tokens, int32_t hidden, int32_t topk,
               int32_t dtype, int64_t capacity_rows, void *out, void *stream);

/*
 * Non-expand dispatch (DeepEP overall architecture: EPHandle do_expand =
 * false; the dispatch copy epilogue writes recv_x, recv_topk_idx and
 * recv_topk_weights): one row per received token instead of one per
 * (token, k). In a world of one the received tokens are those with an
 * unmasked entry, in ascending order, as ep_layout lists them in
 * recv_src_metadata. For i < *num_recv, with t = recv_src_metadata[i][0]:
 *   recv_x[i]            = x[t]                      (bytes of one row)
 *   recv_scales[i]       = x_scales[t]               (only if both are non-NULL)
 *   recv_topk_idx[i][k]  = dst_slot[t][k] >= 0 ? topk_idx[t][k] : -1
 *   recv_topk_weights[i] = topk_weights[t]           (only if both are non-NULL)
 * Rows i >= *num_recv are not written. x, x_scales, dtype and hidden as for
 * ep_dispatch; recv_x [T, hidden], recv_scales [T, S], recv_topk_idx int32
 * [T, K], recv_topk_weights fp32 [T, K] (room for every token); topk_idx,
 * dst_slot, recv_src_metadata and num_recv as written by ep_layout.
 * Shapes are run-time values (no capability gate). Errors: EP_EINVAL.
 */
int ep_dispatch_compact(const void *x, const float *x_scales, const int32_t *topk_idx,
                        const float *topk_weights, const int32_t *dst_slot,
                        const int32_t *recv_src_metadata, const int32_t *num_recv,
                        int32_t num_tokens, int32_t hidden, int32_t topk, int32_t dtype,
                        void *recv_x, float *recv_scales, int32_t *recv_topk_idx,
                        float *recv_topk_weights, void *stream);

/*
 * Layout and non-expand dispatch in one call (the DeepEP overall-architecture
 * page: EPHandle do_expand = false, with the dispatch kernel's notify warps
 * computing the layout before its copy epilogue writes recv_x, recv_topk_idx
 * and recv_topk_weights). It produces everything ep_layout and
 * ep_dispatch_compact produce, with the same arguments, meanings, checks and
 * errors as those two calls (the dispatch reads this layout's dst_slot,
 * recv_src_metadata and num_recv). When T*K fits one layout tile (the
 * floor(W / K) tokens of ep_layout's dispatch_plan: a decode step, say) it
 * runs as a single launch in which every workgroup ranks the entries and the
 * received tokens itself and workgroup 0 writes the layout's outputs; larger
 * batches run the launches of ep_layout and ep_dispatch_compact. Results are
 * identical either way.
 */
int ep_layout_dispatch_compact(const int32_t *topk_idx, int32_t num_tokens, int32_t topk,
                               int32_t num_experts, int32_t expert_alignment,
                               int64_t capacity_rows, int32_t *counts, int32_t *offsets,
                               int32_t *dst_slot, int32_t *recv_src_metadata, int32_t *num_recv,
                               void *workspace, size_t workspace_bytes, const void *x,
                               const float *x_scales, const float *topk_weights, int32_t hidden,
                               int32_t dtype, void *recv_x, float *recv_scales,
                               int32_t *recv_topk_idx, float *recv_topk_weights, void *stream);

/*
 * Non-expand combine (DeepEP overall architecture: combine reduce epilogue
 * with bias, do_expand = false). The expert side returns one row per
 * received token with that token's experts already reduced, so in a world
 * of one combine only puts rows back in token order and adds the bias:
 *   out[t] = float(expert_out[i]) + float(bias[t])  for t = recv_src_metadata[i][0]
 *   out[t] = +0.0 + float(bias[t])                   for a token with no unmasked entry
 * in binary32, one rounded add per value, stored in the rows' type (bf16:
 * round to nearest even; fp32: as is); without a bias, the row's bits, or
 * +0. dtype EP_BF16 or EP_FP32 ("MORI JIT v2" section 3.7: combine takes bf16
 * or fp32 rows and writes the same type). expert_out [T, hidden] (rows
 * >= *num_recv are not read), bias [T, hidden] of the same type or NULL, out
 * [T, hidden] of the same type, every row written. Errors: EP_EINVAL (byte
 * dtypes and unknown dtypes rejected, NULL or misaligned pointers).
 */
int ep_combine_compact(const void *expert_out, const void *bias, const int32_t *dst_slot,
                       const int32_t *recv_src_metadata, const int32_t *num_recv,
                       int32_t num_tokens, int32_t hidden, int32_t topk, int32_t dtype, void *out,
                       void *stream);

/*
 * Optional clean-up of the expand layout: zero the alignment padding rows of
 * every expert segment, rows [offsets[e] + counts[e], offsets[e+1]), so a
 * consumer that walks whole aligned segments (DeepEP overall architecture,
 * EPHandle expert_alignment; the pages leave padding content open and
 * ep_dispatch does not write it) reads zeros there. Real rows are untouched.
 *
 *   expand_x        [capacity_rows, row_bytes] bytes (row_bytes a positive multiple of 16)
 *   expand_scales   fp32 [capacity_rows, scale_cols], or NULL with scale_cols = 0
 *   expand_weights  fp32 [capacity_rows] or NULL
 *   counts, offsets int32 [E] and [E+1] as written by ep_layout (device)
 *   expert_alignment the A given to ep_layout (A = 1: nothing to do)
 * Rows at or beyond capacity_rows are never written. Errors: EP_EINVAL for
 * out-of-range scalars, NULL or misaligned pointers.
 */
int ep_zero_padding(void *expand_x, int64_t row_bytes, float *expand_scales, int64_t scale_cols,
                    float *expand_weights, const int32_t *counts, const int32_t *offsets,
                    int32_t num_experts, int32_t expert_alignment, int64_t capacity_rows,
                    void *stream);

/*
 * CU-limited mode ("MORI JIT v2" section 5.1: geometry buckets prefer the
 * smaller workgroup count when times are close, because compute units left
 * free overlap with the expert GEMM, and the workgroup count never exceeds the
 * CU count; the EpCfg default of sections 3.2 and 3.5 is 64 workgroups. DeepEP overall
 * architecture, design goals: communication on a few SMs, 4 to 64).
 *
 * Caps every kernel this library launches on `stream` (a hipStream_t; NULL
 * is the null stream) at max_workgroups workgroups, each sized to keep one
 * compute unit busy (1024 threads; 512 for combine), whose waves loop over
 * the work; the other compute units stay free for kernels on other streams.
 * Results are identical with and without a cap. max_workgroups = 0 removes
 * the cap (the default: grids cover all work with 256-thread workgroups);
 * values above the current device's compute-unit count are clamped to it.
 * The cap is kept per stream handle, process-wide, until changed: clear it
 * (0) before destroying the stream, since HIP may reuse the handle.
 * Thread-safe; takes effect for launches made after it returns. Errors:
 * EP_EINVAL for max_workgroups < 0, EP_EHIP if the compute-unit count cannot
 * be read (no device).
 */
int ep_set_workgroup_limit(void *stream, int32_t max_workgroups);

/* The cap in effect for `stream` (after clamping), or 0 if none; EP_EHIP only if the
 * registry's lock cannot be taken. */
int ep_get_workgroup_limit(void *stream);

/* Message for the last failed call on the calling thread ("" if none). */
const char *ep_last_error(void);

/*
 * 1 if (hidden, topk, dtype) has compiled kernels for the given pass
 * (0 = layout, which ignores hidden and dtype; 1 = dispatch; 2 = combine),
 * else 0. Never fails.
 */
int ep_supported(int32_t pass, int32_t hidden, int32_t topk, int32_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
