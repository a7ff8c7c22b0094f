/*
 * fa_decode_debug.h -- test and measurement hooks of the decode library.
 *
 * Not needed to run attention.  The gather hook exposes the page-table address
 * generation of the decode kernels so a test can compare it bit for bit with an
 * independent gather; the timing hooks let a benchmark time the dominant
 * kernel with HIP events on the stream it is launched on.
 */
#ifndef FA_DECODE_DEBUG_H
#define FA_DECODE_DEBUG_H

#include "fa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Resolve a paged store through its page table (baracuda-kernels 0.0.1-alpha.68,
 * src/attention/batch_paged_decode.rs, module doc "Layout") exactly as the
 * decode kernels do -- the same split units and workgroup size, the same page
 * ids staged in LDS, the same tile loads (one KV head per workgroup) -- and
 * write the valid rows, as raw element bits, to out laid out
 * [sum_b L_b, Hkv, D]: request 0's rows first, each request's rows in order.
 *
 *   data           [num_total_pages, Hkv, page_size, D]  element size from dtype
 *   indices, indptr, last_page_len   as for fa_decode_paged (same contract)
 *   out            [out_rows, Hkv, D]; rows past out_rows are not written
 *   workspace      >= fa_decode_workspace_size(batch, Hkv, Hkv, D, page_size,
 *                                              total_used_pages)
 * Checks are those of fa_decode_paged that apply (dtype, extents, head_dim,
 * NULL pointers, alignment -- data, out and workspace 16 bytes, the int32
 * arrays 4 --, row range, launch size, workspace), plus out_rows < 0 ->
 * FA_ERR_INVALID_PROBLEM.
 * Asynchronous on stream, like the decode calls. */
fa_status_t fa_debug_gather_paged(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                  int page_size, int num_total_pages, int total_used_pages,
                                  const void *data, const int32_t *indices,
                                  const int32_t *indptr, const int32_t *last_page_len,
                                  void *out, int64_t out_rows, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* The split-unit schedule of a paged decode call with these arguments, as the
 * decode kernels compute it on the device (same code): for every work index
 * w < units_bound (see fa_debug_plan), 8 int32 values at out[8 w .. 8 w + 7]:
 * the request b (-1 for indices past the real unit count, the rest 0), the
 * unit's index c within the request, the request's unit count, L_b, the
 * request's first partial-result slot, its page base, and the low and high
 * 32-bit words of L_0 + .. + L_{b-1}.  Request b's pages are indices[s_b ..
 * s_{b+1}) with s_b the largest of indptr[0 .. b] clamped into [0,
 * total_used_pages]: indptr[b] for a table that keeps its contract; for any
 * other, ranges that do not overlap, so the units never exceed units_bound.
 *   indptr, last_page_len   as for fa_decode_paged (same contract)
 *   out                     device int32 [out_entries], at least 8 * units_bound
 * Checks: dtype, extents, head_dim and total_used_pages as fa_decode_paged;
 * indptr, last_page_len or out NULL or not 4-byte aligned ->
 * FA_ERR_INVALID_PROBLEM; more query heads, rows or work items than
 * fa_decode_paged takes -> FA_ERR_UNSUPPORTED; out_entries short ->
 * FA_ERR_WORKSPACE_TOO_SMALL; a failed launch -> FA_ERR_LAUNCH.
 * Asynchronous on stream. */
fa_status_t fa_debug_schedule(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                              int head_dim, int page_size, int total_used_pages,
                              const int32_t *indptr, const int32_t *last_page_len,
                              int32_t *out, int64_t out_entries, hipStream_t stream);

/* Counters of a workspace left part counted: writes to out[0] how many of the
 * arrival counters a paged call with these arguments uses (one per request
 * and query head, the bound on head blocks), plus the work-ticket counter,
 * hold the rest mark with a non-zero count.  Every decode call leaves the
 * counters it used at rest (count 0), so after calls that ran to completion
 * this is 0; a counter left part counted would make the next call on the
 * workspace merge a request's partials too early.  Counters without the mark
 * (a fresh workspace) are not counted: the next call resets them.
 *   workspace   >= fa_decode_workspace_size(batch, Hq, Hkv, D, page_size,
 *                                           total_used_pages) bytes
 *   out         device int32, at least 1
 * Extents, head_dim, total_used_pages as fa_decode_paged; out NULL or not
 * 4-byte aligned, or workspace not 16-byte aligned -> FA_ERR_INVALID_PROBLEM;
 * more query heads, rows or work items than fa_decode_paged takes ->
 * FA_ERR_UNSUPPORTED; workspace NULL or short -> FA_ERR_WORKSPACE_TOO_SMALL.
 * Asynchronous: read out after the stream reaches the call. */
fa_status_t fa_debug_counters_in_use(int batch, int num_qo_heads, int num_kv_heads,
                                     int head_dim, int page_size, int total_used_pages,
                                     const void *workspace, size_t workspace_bytes,
                                     int32_t *out, hipStream_t stream);

/* Read-bandwidth probe: reads every byte of buf (device memory, bytes > 0 and a
 * multiple of 8192) once with the load shape of the attention kernels (1 KiB
 * contiguous per wave instruction, non-temporal), so a benchmark can compare
 * the attention kernel with what that shape reaches on the device.  sink is a
 * device uint32 that is left unchanged unless the folded data happen to equal
 * one fixed 32-bit constant.  NULL pointers, buf not 16-byte or sink not
 * 4-byte aligned, or a bad size -> FA_ERR_INVALID_PROBLEM; a failed launch ->
 * FA_ERR_LAUNCH.  Asynchronous. */
fa_status_t fa_debug_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                                hipStream_t stream);

/* fa_debug_gather_paged for a token-major store: data is
 * [num_total_pages, page_size, Hkv, D]; out is laid out as above. */
fa_status_t fa_debug_gather_paged_nhd(fa_dtype_t dtype, int batch, int num_kv_heads,
                                      int head_dim, int page_size, int num_total_pages,
                                      int total_used_pages, const void *data,
                                      const int32_t *indices, const int32_t *indptr,
                                      const int32_t *last_page_len, void *out, int64_t out_rows,
                                      void *workspace, size_t workspace_bytes,
                                      hipStream_t stream);

/* Kernel timing.  While enabled, every decode call records a HIP event pair on
 * its stream around its main attention kernel (the one that streams K and V),
 * and another around the whole call.  fa_debug_timing_read waits for the
 * recorded events, returns the summed milliseconds and the number of calls
 * since the last reset, and resets.  Process-wide; meant for one benchmarking
 * thread.  Returns FA_ERR_LAUNCH if a HIP event call fails. */
fa_status_t fa_debug_timing_enable(int enable);
fa_status_t fa_debug_timing_read(double *main_kernel_ms, double *whole_call_ms, int *calls);

/* The launch plan a decode call with these arguments would use (host-side
 * arithmetic only): KV rows per split unit, the bound on split units, query
 * heads per workgroup, and which attention kernel runs (always 1, the
 * matrix-core kernel, for every element type).  Returns
 * FA_ERR_INVALID_PROBLEM for arguments the entry points would reject on
 * extents. */
fa_status_t fa_debug_plan(fa_dtype_t dtype, int batch, int num_qo_heads, int num_kv_heads,
                          int head_dim, int page_size, int total_used_pages, int *chunk_rows,
                          int *units_bound, int *heads_per_unit, int *kernel_kind);

#ifdef __cplusplus
}
#endif

#endif /* FA_DECODE_DEBUG_H */
