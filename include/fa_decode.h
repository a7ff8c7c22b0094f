/*
 * fa_decode.h -- single-query GQA decode attention for MI355X (gfx950).
 *
 * One query token per request attends over that request's K/V history.  For a
 * request b and query/output head h the KV head is g = h / (Hq / Hkv): runs of
 * Hq/Hkv consecutive query heads share one KV head (ferrox-cuda 0.15.2,
 * src/attn.rs, kernel source gqa_decode: the group-size and KV-head index).
 * With L_b valid K/V rows,
 *
 *     x_j      = scale * <q[b,h,:], K_b[g,j,:]>          j = 0 .. L_b - 1
 *     o[b,h,:] = sum_j softmax(x)_j * V_b[g,j,:]
 *     lse[b,h] = ln sum_j exp(x_j)                        (natural log, f32)
 *
 * (ferrum-kernels 0.7.7, src/backend/cuda/decode_attention.rs, module doc: the
 * scores, a numerically stable softmax, and the score-weighted sum of V;
 * baracuda-kernels 0.0.1-alpha.68, src/attention/batch_paged_decode.rs, module
 * doc "Query / output": the per-row log-sum-exp, always f32.)
 * A request with L_b = 0 gets o = 0 and lse = -inf.
 *
 * Conventions common to every entry point:
 *   - All buffer pointers are DEVICE pointers to dense, row-major (C-order)
 *     arrays with no padding between rows.  Element type T is given by dtype;
 *     indices, indptr and last_page_len are int32; lse is always f32.
 *   - Arithmetic: products and sums in f32, o rounded once to T
 *     (round-to-nearest-even).
 *   - Ownership: the caller allocates and frees every buffer (inputs, outputs,
 *     workspace).  The library allocates no device memory and keeps no state
 *     between calls, except the static scratch array of
 *     fa_decode_paged_noalloc (below).
 *   - Streams: work is enqueued on `stream` (0 = the null stream) and the call
 *     returns without synchronising; outputs are ready when the stream reaches
 *     that point.  No host<->device copies are made.
 *   - Determinism: for a fixed argument set, results are bit-identical from
 *     run to run on one device.  Long requests are split into units whose
 *     partial results are combined in unit order, whichever workgroup ends
 *     last; the only atomics are the counters that find that workgroup.
 *   - Graph capture: a call may be captured into a HIP graph and replayed;
 *     replays of one captured call must not overlap each other.
 *   - Errors: arguments are checked on the host in the order listed for each
 *     entry point; any status other than FA_OK means nothing was enqueued,
 *     except FA_ERR_LAUNCH, which reports a failed kernel launch.
 *   - o and lse must not overlap any input or the workspace.
 *   - Concurrent calls on different streams must use different workspaces.
 */
#ifndef FA_DECODE_H
#define FA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, K, V and o (baracuda-kernels page, module doc
 * "Constraints": f16, bf16 or f32). */
typedef enum { FA_DTYPE_F32 = 0, FA_DTYPE_F16 = 1, FA_DTYPE_BF16 = 2 } fa_dtype_t;

/* Status codes.  The three problem classes follow the error kinds the
 * baracuda-kernels plan returns (BatchPagedDecodePlan::select, can_implement
 * and run): an invalid problem, an unsupported one, and a workspace that is too
 * small; FA_ERR_LAUNCH mirrors the launch-failure error of the ferrum-kernels
 * and ferrox-cuda host wrappers. */
typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_PROBLEM = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_WORKSPACE_TOO_SMALL = 3,
  FA_ERR_LAUNCH = 4
} fa_status_t;

/* Bytes of device workspace a call needs (baracuda-kernels page,
 * BatchPagedDecodePlan::workspace_size: auxiliary buffers the launcher fills on
 * every call; ours also hold the split-KV partial results).
 *
 * A pure function of its arguments; it makes no device query.
 *   paged calls:       fa_decode_workspace_size(batch, Hq, Hkv, D, page_size, total_used_pages)
 *   contiguous calls:  fa_decode_workspace_size(1, Hq, Hkv, D, max_kv_len, 1)
 * Returns 0 when the arguments are not a valid problem or one no entry point
 * launches (the entry point then reports why); otherwise a positive size.  The workspace holds the split
 * partial results, one arrival counter per (request, head block) and one
 * counter that hands out work items to the workgroups of a launch that start
 * after its first resident round.  A counter at rest carries a fixed mark and
 * a count of zero, and each call leaves its counters at rest; a counter
 * without the mark is reset by the first workgroup that meets it.  So the workspace needs no initialisation and may
 * hold anything between calls (a first use costs each counter one extra
 * compare-and-swap). */
size_t fa_decode_workspace_size(int batch, int num_qo_heads, int num_kv_heads, int head_dim,
                                int page_size, int total_used_pages);

/* Decode against a contiguous cache (ferrum-kernels page, decode_attention and
 * its argument list).
 *
 *   q        [Hq, D]              T   the single query token's heads
 *   k_cache  [Hkv, max_kv_len, D] T   heads-major cache; rows >= valid_kv_len
 *   v_cache  [Hkv, max_kv_len, D] T   are never read into the result
 *   o        [Hq, D]              T   output
 *   lse      [Hq]                 f32 output; may be NULL (not written)
 *   scale    the score multiplier, usually 1/sqrt(D)
 *   workspace, workspace_bytes   >= fa_decode_workspace_size(1, Hq, Hkv, D, max_kv_len, 1)
 *
 * Checks, in order:
 *   dtype not one of fa_dtype_t                              -> FA_ERR_UNSUPPORTED
 *   num_qo_heads, num_kv_heads or max_kv_len <= 0            -> FA_ERR_INVALID_PROBLEM
 *   num_qo_heads % num_kv_heads != 0                         -> FA_ERR_INVALID_PROBLEM
 *   head_dim not 64, 128 or 256                              -> FA_ERR_UNSUPPORTED
 *   num_qo_heads > 65535                                     -> FA_ERR_UNSUPPORTED
 *   q, k_cache, v_cache or o NULL                            -> FA_ERR_INVALID_PROBLEM
 *   q, k_cache, v_cache, o or workspace not 16-byte aligned,
 *     or lse not 4-byte aligned                              -> FA_ERR_INVALID_PROBLEM
 *   valid_kv_len < 0 or > max_kv_len                         -> FA_ERR_INVALID_PROBLEM
 *   Hkv * max_kv_len * D >= 10^15 elements                   -> FA_ERR_UNSUPPORTED
 *   workspace NULL or workspace_bytes short                  -> FA_ERR_WORKSPACE_TOO_SMALL
 *   a kernel launch fails                                    -> FA_ERR_LAUNCH */
fa_status_t fa_decode_contig(fa_dtype_t dtype, int num_qo_heads, int num_kv_heads,
                             int head_dim, int max_kv_len, int valid_kv_len, float scale,
                             const void *q, const void *k_cache, const void *v_cache,
                             void *o, float *lse, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Batched decode against a paged K/V store (baracuda-kernels page: module doc
 * "Layout" and "Query / output", the descriptor structs and
 * BatchPagedDecodePlan::run).  Every request contributes one query row.
 *
 *   q              [batch, Hq, D]                   T
 *   k_data, v_data [num_total_pages, Hkv, page_size, D] T  heads-major inside a page
 *   indices        [total_used_pages]               int32 physical page ids,
 *                                                   in [0, num_total_pages)
 *   indptr         [batch + 1]                      int32 request b owns pages
 *                                                   indices[indptr[b] .. indptr[b+1])
 *   last_page_len  [batch]                          int32 rows used in the last page,
 *                                                   in [0, page_size]
 *   o              [batch, Hq, D]                   T   output
 *   lse            [batch, Hq]                      f32 output (required)
 *   sm_scale       the score multiplier, usually 1/sqrt(D)
 *   workspace, workspace_bytes   >= fa_decode_workspace_size(batch, Hq, Hkv, D,
 *                                                            page_size, total_used_pages)
 *
 * Request b has L_b = (n_b - 1) * page_size + last_page_len[b] rows, where
 * n_b = indptr[b+1] - indptr[b]; L_b = 0 when n_b = 0.  Only row positions
 * inside those L_b rows are read into the result.
 *
 * The page table lives in device memory and is not checked here: indptr[0] = 0,
 * indptr non-decreasing, indptr[batch] <= total_used_pages, page ids in range
 * and last_page_len in [0, page_size] are the caller's contract (the
 * baracuda-kernels plan checks shapes only).  A table that breaks it gives
 * unspecified results but never reads or writes outside the buffers described
 * above.  The page table and its allocator stay with the caller.
 *
 * Checks, in order:
 *   dtype not one of fa_dtype_t                               -> FA_ERR_UNSUPPORTED
 *   batch, Hq, Hkv, page_size or num_total_pages <= 0         -> FA_ERR_INVALID_PROBLEM
 *   num_qo_heads % num_kv_heads != 0                          -> FA_ERR_INVALID_PROBLEM
 *   head_dim not 64, 128 or 256                               -> FA_ERR_UNSUPPORTED
 *   total_used_pages < 0                                      -> FA_ERR_INVALID_PROBLEM
 *   num_qo_heads > 65535                                      -> FA_ERR_UNSUPPORTED
 *   q, k_data, v_data, indptr, last_page_len, o or lse NULL,
 *     or indices NULL with total_used_pages > 0               -> FA_ERR_INVALID_PROBLEM
 *   q, k_data, v_data, o or workspace not 16-byte aligned, or
 *     indices, indptr, last_page_len or lse not 4-byte aligned -> FA_ERR_INVALID_PROBLEM
 *   total_used_pages * page_size >= 2^31 (row index range)    -> FA_ERR_UNSUPPORTED
 *   num_total_pages * Hkv * page_size * D >= 10^15 elements   -> FA_ERR_UNSUPPORTED
 *   (batch + total_used_pages * page_size / chunk) * Hq / G >= 2^31, where
 *     chunk and G (query heads per workgroup) are fa_debug_plan's chunk_rows
 *     and heads_per_unit (more workgroups than a launch takes) -> FA_ERR_UNSUPPORTED
 *   workspace NULL or workspace_bytes short                   -> FA_ERR_WORKSPACE_TOO_SMALL
 *   a kernel launch fails                                     -> FA_ERR_LAUNCH */
fa_status_t fa_decode_paged(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                            int head_dim, int page_size, int num_total_pages,
                            int total_used_pages, float sm_scale, const void *q,
                            const void *k_data, const void *v_data, const int32_t *indices,
                            const int32_t *indptr, const int32_t *last_page_len, void *o,
                            float *lse, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/* Size in bytes of the library's static scratch array used by
 * fa_decode_paged_noalloc (one copy per GPU). */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* fa_decode_paged for callers that cannot allocate device memory: code under
 * HIP graph capture that has no buffer to hand over as a workspace, tight
 * serving loops, and harnesses that forbid hipMalloc.  Same arguments, checks,
 * conventions and results as fa_decode_paged (bit-identical outputs), minus
 * workspace and workspace_bytes.  The split partials and counters live in a
 * static device array of FA_NOALLOC_SCRATCH_BYTES bytes inside the library:
 * each GPU the library runs on holds one copy until the process ends, and no
 * call allocates or frees anything.
 *   - The problem's fa_decode_workspace_size(batch, Hq, Hkv, D, page_size,
 *     total_used_pages) must not exceed FA_NOALLOC_SCRATCH_BYTES; a larger one
 *     -> FA_ERR_WORKSPACE_TOO_SMALL (checked after every check of
 *     fa_decode_paged before its workspace check; nothing is enqueued).
 *   - The first call on a GPU looks up the device address of that GPU's copy
 *     of the array (hipGetSymbolAddress, with that GPU current) and keeps it;
 *     if the lookup fails -> FA_ERR_LAUNCH.  A caller that captures calls
 *     should make its first call on each GPU outside capture.
 *   - Every call on one GPU uses that GPU's one array, which keeps what the
 *     last call left there.  Calls that may overlap on one GPU (on different
 *     streams, or concurrent replays of captured calls) race on it and give
 *     undefined results; calls on one stream are ordered and safe.  Nothing in
 *     the array needs clearing between calls (as for a workspace, its contents
 *     before a call do not matter). */
fa_status_t fa_decode_paged_noalloc(fa_dtype_t dtype, int batch, int num_qo_heads,
                                    int num_kv_heads, int head_dim, int page_size,
                                    int num_total_pages, int total_used_pages, float sm_scale,
                                    const void *q, const void *k_data, const void *v_data,
                                    const int32_t *indices, const int32_t *indptr,
                                    const int32_t *last_page_len, void *o, float *lse,
                                    hipStream_t stream);

/* Token-major variants (ferrox-cuda 0.15.2, src/attn.rs: the gqa_decode kernel
 * source and the k_cache / v_cache shape in its doc comment put row t of KV
 * head g at (t * Hkv + g) * D).  Same arguments, checks, conventions and
 * results as the entry points above; only the K/V layout differs:
 *
 *   fa_decode_contig_nhd:  k_cache, v_cache  [max_kv_len, Hkv, D]  T
 *   fa_decode_paged_nhd:   k_data, v_data    [num_total_pages, page_size, Hkv, D]  T
 *                          (all heads of one token adjacent inside a page; the
 *                          pages print no paged token-major layout, this is the
 *                          page-level form of the contiguous one)
 *
 * For the same logical rows the outputs are bit-identical to the heads-major
 * entry points'. */
fa_status_t fa_decode_contig_nhd(fa_dtype_t dtype, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int max_kv_len, int valid_kv_len, float scale,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 void *o, float *lse, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

fa_status_t fa_decode_paged_nhd(fa_dtype_t dtype, int batch, int num_qo_heads,
                                int num_kv_heads, int head_dim, int page_size,
                                int num_total_pages, int total_used_pages, float sm_scale,
                                const void *q, const void *k_data, const void *v_data,
                                const int32_t *indices, const int32_t *indptr,
                                const int32_t *last_page_len, void *o, float *lse,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Layout and score variants for fa_decode_paged_opts / fa_decode_contig_opts.
 * The baracuda-kernels page lists a sliding window and logits soft-capping as
 * not supported by its plan (module doc "Constraints") and defines neither;
 * the readings here:
 *   kv_layout        0: heads-major K/V (as fa_decode_paged / fa_decode_contig),
 *                    1: token-major (as the _nhd entry points)
 *   window           > 0: each request's query (its newest token, at row
 *                    L_b - 1) attends only rows j >= L_b - window; 0: all rows
 *   logits_soft_cap  > 0: every scaled score x becomes cap * tanh(x / cap)
 *                    before the softmax, and lse sums exp of the capped scores;
 *                    0: off
 *   alibi_slopes     device f32 [num_qo_heads] or NULL: query head h adds
 *                    alibi_slopes[h] * (j - (L_b - 1)) to row j's scaled score
 *                    (0 at the query's own row, more negative further back),
 *                    before any cap; the pages list ALiBi as unsupported too
 *   custom_mask      device uint8 bit array or NULL: one bit per K/V row of
 *                    every request, requests back to back in request order, so
 *                    row j of request b is bit R_b + j with R_b = L_0 + .. +
 *                    L_{b-1} (a contiguous cache: bit j), bit i at byte i / 8,
 *                    bit i % 8.  A set bit keeps the row; a clear bit removes
 *                    it from the softmax (kept rows keep their positions, so
 *                    ALiBi distances do not change).  A row must pass both the
 *                    window and the mask; a request left with no row gets o = 0
 *                    and lse = -inf.  The pages list custom masks as
 *                    unsupported and define none; this is the plainest reading
 *                    for one query row per request.  K/V rows are read in
 *                    32-row tiles (16 for f32), per wave of the kernel: a tile
 *                    with no kept row is not read; a tile with one is read
 *                    whole.  Groups of more than 16 query heads at head_dim
 *                    256 (f32 K/V: 128 and 256) read every tile.
 *   custom_mask_bytes  size of custom_mask in bytes (ignored when it is NULL):
 *                    ceil(sum L_b / 8) covers every row (ceil(valid_kv_len / 8)
 *                    for a contiguous cache).  Bits at or past 8 *
 *                    custom_mask_bytes read as 0 (row dropped), so a short
 *                    mask never makes the library read past it.
 * A window keeps whole 16-row blocks of rows below it in the read set (they are
 * masked, never weighted), so the bytes read grow by at most 15 rows per
 * request. */
typedef struct {
  int kv_layout;
  int window;
  float logits_soft_cap;
  const float *alibi_slopes;
  const uint8_t *custom_mask;
  size_t custom_mask_bytes;
} fa_decode_options_t;

/* fa_decode_paged / fa_decode_contig with options (opts may be NULL: all
 * defaults, identical to the plain entry points).  Checked before the plain
 * entry point's own checks:
 *   opts->kv_layout not 0 or 1                                 -> FA_ERR_UNSUPPORTED
 *   opts->window < 0, or logits_soft_cap negative or not finite,
 *     or alibi_slopes not 4-byte aligned, or custom_mask set with
 *     custom_mask_bytes 0                                        -> FA_ERR_INVALID_PROBLEM */
fa_status_t fa_decode_paged_opts(const fa_decode_options_t *opts, fa_dtype_t dtype, int batch,
                                 int num_qo_heads, int num_kv_heads, int head_dim, int page_size,
                                 int num_total_pages, int total_used_pages, float sm_scale,
                                 const void *q, const void *k_data, const void *v_data,
                                 const int32_t *indices, const int32_t *indptr,
                                 const int32_t *last_page_len, void *o, float *lse,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

fa_status_t fa_decode_contig_opts(const fa_decode_options_t *opts, fa_dtype_t dtype,
                                  int num_qo_heads, int num_kv_heads, int head_dim,
                                  int max_kv_len, int valid_kv_len, float scale, const void *q,
                                  const void *k_cache, const void *v_cache, void *o, float *lse,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Decode-time KV append (baracuda-kernels page, module doc "Companion plans":
 * the new K/V slices are written into the paged store before decode; the page
 * names the plan but prints no signature).  Writes one new K row and one new V
 * row per request:
 *
 *   k_new, v_new      [batch, Hkv, D]  T   the new token's K and V, per request
 *   k_data, v_data    the paged store, [num_total_pages, Hkv, page_size, D]
 *                     (fa_append_paged) or [num_total_pages, page_size, Hkv, D]
 *                     (fa_append_paged_nhd); updated in place
 *   indices, indptr, last_page_len   the page table AFTER the caller's
 *                     allocator has made room for the new token: request b's
 *                     row goes to its last valid row L_b - 1 (in the
 *                     second-to-last page when last_page_len[b] = 0); a request
 *                     with L_b = 0 receives nothing
 *
 * Nothing else in the store changes.  A table that gives two requests the same
 * page, or breaks the contract of fa_decode_paged, gives unspecified contents
 * but never a write outside k_data / v_data.  k_new and v_new must not overlap
 * the store.  No workspace.  Asynchronous on stream, so a following decode
 * call on the same stream sees the new rows.
 *
 * Checks, in order:
 *   dtype not one of fa_dtype_t                                -> FA_ERR_UNSUPPORTED
 *   batch, Hkv, page_size or num_total_pages <= 0              -> FA_ERR_INVALID_PROBLEM
 *   head_dim not 64, 128 or 256                                -> FA_ERR_UNSUPPORTED
 *   total_used_pages < 0                                       -> FA_ERR_INVALID_PROBLEM
 *   k_new, v_new, indptr, last_page_len, k_data or v_data NULL,
 *     or indices NULL with total_used_pages > 0                -> FA_ERR_INVALID_PROBLEM
 *   k_new, v_new, k_data or v_data not 16-byte aligned, or
 *     indices, indptr or last_page_len not 4-byte aligned      -> FA_ERR_INVALID_PROBLEM
 *   total_used_pages * page_size >= 2^31                       -> FA_ERR_UNSUPPORTED
 *   num_total_pages * Hkv * page_size * D >= 10^15 elements    -> FA_ERR_UNSUPPORTED
 *   batch * Hkv >= 2^31                                        -> FA_ERR_UNSUPPORTED
 *   a kernel launch fails                                      -> FA_ERR_LAUNCH */
fa_status_t fa_append_paged(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                            int page_size, int num_total_pages, int total_used_pages,
                            const void *k_new, const void *v_new, const int32_t *indices,
                            const int32_t *indptr, const int32_t *last_page_len, void *k_data,
                            void *v_data, hipStream_t stream);

fa_status_t fa_append_paged_nhd(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                int page_size, int num_total_pages, int total_used_pages,
                                const void *k_new, const void *v_new, const int32_t *indices,
                                const int32_t *indptr, const int32_t *last_page_len,
                                void *k_data, void *v_data, hipStream_t stream);

/* Merge of split partial results: the combine step of split-KV decode as a
 * call of its own, for partials made outside one decode call -- the shares of
 * a request's K/V rows decoded on different devices and gathered onto one, or
 * a caller's own split of the rows.  It follows from the per-row log-sum-exp
 * the decode calls return (baracuda-kernels page, module doc "Query /
 * output"): with the rows of a query split into S disjoint parts, part s
 * giving o_s (normalised over its rows) and lse_s,
 *
 *     lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s,
 *
 * which is exactly the result over all the rows.  fa_decode_paged and
 * fa_decode_contig make the same combination inside one call when they split
 * a long request.
 *
 *   o_parts    [num_parts, num_rows, head_dim] f32   partial outputs, each
 *              normalised over its part (f32: the element type of partials)
 *   lse_parts  [num_parts, num_rows]           f32   natural-log LSE of each
 *              part; -inf marks an empty part, whose o_parts row may hold
 *              anything (it does not reach the result)
 *   o          [num_rows, head_dim]            T     output, rounded once to T
 *   lse        [num_rows]                      f32   output; may be NULL
 * A row is any flattening of the caller's (request, query head) pairs.  A row
 * whose parts are all empty gets o = 0 and lse = -inf.  The parts of a row
 * are combined in index order, so results are bit-identical from run to run.
 * Inputs must not overlap the outputs.  No workspace.  Asynchronous on stream.
 *
 * Checks, in order:
 *   dtype not one of fa_dtype_t                               -> FA_ERR_UNSUPPORTED
 *   num_rows < 0 or num_parts <= 0                            -> FA_ERR_INVALID_PROBLEM
 *   head_dim not 64, 128 or 256                               -> FA_ERR_UNSUPPORTED
 *   num_rows == 0                                             -> FA_OK, nothing enqueued
 *   o_parts, lse_parts or o NULL                              -> FA_ERR_INVALID_PROBLEM
 *   o_parts or o not 16-byte aligned, or lse_parts or lse
 *     not 4-byte aligned                                      -> FA_ERR_INVALID_PROBLEM
 *   num_parts * num_rows * head_dim >= 10^15                  -> FA_ERR_UNSUPPORTED
 *   a kernel launch fails                                     -> FA_ERR_LAUNCH */
fa_status_t fa_merge_states(fa_dtype_t dtype, int num_rows, int num_parts, int head_dim,
                            const float *o_parts, const float *lse_parts, void *o, float *lse,
                            hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *fa_status_string(fa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* FA_DECODE_H */
