// fa_plan.hpp -- the host side of every call that needs no device: argument
// checks in the documented order, the launch plan (split size, unit bound,
// head blocks) and the workspace layout.  Plain C++ (no device code, no HIP
// call), so the same code also builds with a host compiler for sanitizer runs.
#pragma once

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "../../include/fa_decode.h"
#include "fa_limits.hpp"

namespace fa_plan {

// Split sizing: aim for about this many decode workgroups per call, so the
// 256 CUs each get several and the tail is short.
constexpr int64_t kTargetWorkgroups = 1024;
constexpr int64_t kChunkQuantum = 128;  // KV rows; a multiple of every tile (32 rows)
constexpr int64_t kMaxChunk = int64_t(1) << 30;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The attention kernel of a call: 1, the matrix-core kernel, for every element
// type and head dim (the value fa_debug_plan reports).
constexpr int kKernelMfma = 1;

struct HostPlan {
  int group = 0, gt = 0, nb = 1, n_gblocks = 0, planes = 0;
  int chunk = 0, units_bound = 0, kind = 0;
  // workspace byte offsets
  size_t part_lse = 0, part_o = 0, arrivals = 0, tickets = 0, total = 0;
};

inline bool extents_ok(int batch, int hq, int hkv, int page_size) {
  return batch > 0 && hq > 0 && hkv > 0 && page_size > 0 && hq % hkv == 0;
}

inline bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

// grid.y is Hkv * (workgroups per KV head) and must stay within the launch limit
inline bool grid_ok(int hq, int hkv) { return hq / hkv > 0 && hkv * (hq / hkv) <= 65535; }

inline bool dtype_ok(fa_dtype_t dt) {
  return dt == FA_DTYPE_F32 || dt == FA_DTYPE_F16 || dt == FA_DTYPE_BF16;
}

// The kernels move q, K, V, o and workspace data 16 bytes per access and
// int32 / f32 arrays 4 bytes per access; row strides (D * element size >= 128
// bytes) keep every row at the alignment of its base.  NULL counts as aligned.
inline bool aligned(const void *ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0;
}

inline bool all_aligned(std::initializer_list<const void *> wide,
                        std::initializer_list<const void *> narrow) {
  for (const void *ptr : wide)
    if (!aligned(ptr, 16)) return false;
  for (const void *ptr : narrow)
    if (!aligned(ptr, 4)) return false;
  return true;
}

// Elements of a [pages, Hkv, P, D] pool must stay far inside int64 offsets.
inline bool pool_size_ok(int pages, int hkv, int page_size, int d) {
  const double n = double(pages) * hkv * page_size * d;
  return n < 1.0e15;
}

// Row indices of a paged call (total_used_pages * page_size) must fit an int.
inline bool rows_ok(int total_used_pages, int page_size) {
  return int64_t(total_used_pages) * page_size < (int64_t(1) << 31);
}

// The plan for a call; `page_size` is max_kv_len and total_used_pages 1 for a
// contiguous cache.  Pure host arithmetic; callers have checked the extents.
inline HostPlan make_plan(int batch, int hq, int hkv, int d, int page_size,
                          int total_used_pages, bool contig) {
  HostPlan hp;
  hp.kind = kKernelMfma;
  hp.group = hq / hkv;
  // Head blocks: the whole group when it fits the 16-column MFMA block (one
  // workgroup per split unit and KV head); else blocks of 16 with a shorter
  // last one, two per workgroup, so K/V are read once per 32 query heads.
  if (hp.group <= 16) {
    hp.gt = hp.group;
    hp.nb = 1;
  } else {
    hp.gt = 16;
    hp.nb = 2;
  }
  hp.n_gblocks = (hp.group - 1) / (hp.gt * hp.nb) + 1;  // group >= 1; no overflow
  hp.planes = hkv * hp.n_gblocks;
  // The split size depends on the KV heads only (not on the kernel's head
  // blocking), so the workspace size is the same for every element type.
  const int64_t rows_ub = int64_t(std::max(total_used_pages, 0)) * page_size;
  int64_t want = (rows_ub * hkv + kTargetWorkgroups - 1) / kTargetWorkgroups;
  want = std::max<int64_t>(want, kChunkQuantum);
  int64_t chunk = (want + kChunkQuantum - 1) / kChunkQuantum * kChunkQuantum;
  chunk = std::min(chunk, kMaxChunk);
  if (!contig && page_size % 16 == 0) {
    // the matrix-core kernel stages a unit's page ids in LDS: at most 1024
    // whole pages per unit (plus a partial page at each end)
    static_assert(1024 + 2 <= fa::kPageTable, "page table slice");
    const int64_t cap = std::max<int64_t>(
        kChunkQuantum, 1024 * int64_t(page_size) / kChunkQuantum * kChunkQuantum);
    chunk = std::min(chunk, cap);
  }
  hp.chunk = int(chunk);
  // Units: a request of L rows has max(1, ceil(L / chunk)) of them, which is at
  // most 1 + floor(L / chunk); summed, at most batch + floor(sum L / chunk).
  // (saturated at INT32_MAX: launch_ok then rejects the problem)
  const int64_t units = contig ? std::max<int64_t>(1, (int64_t(page_size) + chunk - 1) / chunk)
                               : int64_t(batch) + rows_ub / chunk;
  hp.units_bound = int(std::min<int64_t>(units, INT32_MAX));
  size_t off = 0;
  hp.part_lse = off;    off = align_up(off + sizeof(float) * size_t(hp.units_bound) * hq);
  hp.part_o = off;      off = align_up(off + sizeof(float) * size_t(hp.units_bound) * hq * d);
  // one counter line per (request, head block); Hq per request bounds the blocks
  hp.arrivals = off;
  off = align_up(off + sizeof(uint64_t) * fa::kArrivalStride * size_t(batch) * hq);
  // and one line for the counter that hands out work items past the first round
  hp.tickets = off;
  off = align_up(off + sizeof(uint64_t) * fa::kArrivalStride);
  hp.total = off;
  return hp;
}

// Work indices (split units times head blocks) must fit a launch and an int;
// a unit bound saturated by make_plan never passes.
inline bool launch_ok(const HostPlan &hp) {
  return int64_t(hp.units_bound) * hp.planes < int64_t(INT32_MAX);
}

// fa_decode_workspace_size: 0 for arguments that are not a valid problem,
// including ones no entry point launches (too many query heads or work items;
// which also keeps every size product far inside size_t).
inline size_t workspace_size(int batch, int hq, int hkv, int d, int page_size,
                             int total_used_pages) {
  if (!extents_ok(batch, hq, hkv, page_size) || !head_dim_ok(d) || total_used_pages < 0)
    return 0;
  if (!grid_ok(hq, hkv) || !rows_ok(total_used_pages, page_size)) return 0;
  const HostPlan hp = make_plan(batch, hq, hkv, d, page_size, total_used_pages, false);
  return launch_ok(hp) ? hp.total : 0;
}

// Layout and score variants of one call (fa_decode_options_t, validated).
struct Variant {
  int nhd = 0;
  int window = 0;
  float softcap = 0.0f;
  const float *alibi = nullptr;
  const uint8_t *mask = nullptr;
  uint32_t mask_bytes = 0;
};

// FA_OK, or why opts is rejected; fills v.
inline fa_status_t read_options(const fa_decode_options_t *opts, Variant &v) {
  if (!opts) return FA_OK;
  if (opts->kv_layout != 0 && opts->kv_layout != 1) return FA_ERR_UNSUPPORTED;
  if (opts->window < 0 || !(opts->logits_soft_cap >= 0.0f) ||
      !std::isfinite(opts->logits_soft_cap) || !aligned(opts->alibi_slopes, 4) ||
      (opts->custom_mask && opts->custom_mask_bytes == 0))
    return FA_ERR_INVALID_PROBLEM;
  v.nhd = opts->kv_layout;
  v.window = opts->window;
  v.softcap = opts->logits_soft_cap;
  v.alibi = opts->alibi_slopes;
  v.mask = opts->custom_mask;
  // rows are int-indexed, so no bit past 2^31 is ever asked for
  v.mask_bytes = uint32_t(std::min<size_t>(opts->custom_mask_bytes, size_t(1) << 28));
  return FA_OK;
}

// Every check of a paged call that comes before the workspace check, in the
// documented order (the workspace pointer's alignment included).
inline fa_status_t paged_checks(fa_dtype_t dtype, int batch, int num_qo_heads,
                                int num_kv_heads, int head_dim, int page_size,
                                int num_total_pages, int total_used_pages, const void *q,
                                const void *k_data, const void *v_data,
                                const int32_t *indices, const int32_t *indptr,
                                const int32_t *last_page_len, const void *o, const float *lse,
                                const void *workspace) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(batch, num_qo_heads, num_kv_heads, page_size) || num_total_pages <= 0)
    return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (total_used_pages < 0) return FA_ERR_INVALID_PROBLEM;
  if (!grid_ok(num_qo_heads, num_kv_heads)) return FA_ERR_UNSUPPORTED;
  if (!q || !k_data || !v_data || !indptr || !last_page_len || !o || !lse ||
      (!indices && total_used_pages > 0))
    return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({q, k_data, v_data, o, workspace}, {indices, indptr, last_page_len, lse}))
    return FA_ERR_INVALID_PROBLEM;
  if (!rows_ok(total_used_pages, page_size)) return FA_ERR_UNSUPPORTED;
  if (!pool_size_ok(num_total_pages, num_kv_heads, page_size, head_dim))
    return FA_ERR_UNSUPPORTED;
  const HostPlan hp = make_plan(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                total_used_pages, false);
  if (!launch_ok(hp)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Every check of a contiguous call before the workspace check, in order.
inline fa_status_t contig_checks(fa_dtype_t dtype, int num_qo_heads, int num_kv_heads,
                                 int head_dim, int max_kv_len, int valid_kv_len,
                                 const void *q, const void *k_cache, const void *v_cache,
                                 const void *o, const float *lse, const void *workspace) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(1, num_qo_heads, num_kv_heads, max_kv_len)) return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (!grid_ok(num_qo_heads, num_kv_heads)) return FA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !o) return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({q, k_cache, v_cache, o, workspace}, {lse})) return FA_ERR_INVALID_PROBLEM;
  if (valid_kv_len < 0 || valid_kv_len > max_kv_len) return FA_ERR_INVALID_PROBLEM;
  if (!pool_size_ok(1, num_kv_heads, max_kv_len, head_dim)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Every check of the decode-time append, in order.
inline fa_status_t append_checks(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                 int page_size, int num_total_pages, int total_used_pages,
                                 const void *k_new, const void *v_new, const int32_t *indices,
                                 const int32_t *indptr, const int32_t *last_page_len,
                                 const void *k_data, const void *v_data) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(batch, num_kv_heads, num_kv_heads, page_size) || num_total_pages <= 0)
    return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (total_used_pages < 0) return FA_ERR_INVALID_PROBLEM;
  if (!k_new || !v_new || !indptr || !last_page_len || !k_data || !v_data ||
      (!indices && total_used_pages > 0))
    return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({k_new, v_new, k_data, v_data}, {indices, indptr, last_page_len}))
    return FA_ERR_INVALID_PROBLEM;
  if (!rows_ok(total_used_pages, page_size)) return FA_ERR_UNSUPPORTED;
  if (!pool_size_ok(num_total_pages, num_kv_heads, page_size, head_dim))
    return FA_ERR_UNSUPPORTED;
  if (int64_t(batch) * num_kv_heads >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Every check of the gather hook before its workspace check, in order.
inline fa_status_t gather_checks(fa_dtype_t dtype, int batch, int num_kv_heads, int head_dim,
                                 int page_size, int num_total_pages, int total_used_pages,
                                 const void *data, const int32_t *indices,
                                 const int32_t *indptr, const int32_t *last_page_len,
                                 const void *out, int64_t out_rows, const void *workspace) {
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (!extents_ok(batch, num_kv_heads, num_kv_heads, page_size) || num_total_pages <= 0)
    return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (total_used_pages < 0 || out_rows < 0) return FA_ERR_INVALID_PROBLEM;
  if (!data || !indptr || !last_page_len || !out || (!indices && total_used_pages > 0))
    return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({data, out, workspace}, {indices, indptr, last_page_len}))
    return FA_ERR_INVALID_PROBLEM;
  if (!rows_ok(total_used_pages, page_size)) return FA_ERR_UNSUPPORTED;
  if (!pool_size_ok(num_total_pages, num_kv_heads, page_size, head_dim))
    return FA_ERR_UNSUPPORTED;
  if (!launch_ok(make_plan(batch, num_kv_heads, num_kv_heads, head_dim, page_size,
                           total_used_pages, false)))
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Every check of the standalone merge, in order; *empty is set when there is
// nothing to do (no rows: FA_OK and nothing enqueued).
inline fa_status_t merge_checks(fa_dtype_t dtype, int num_rows, int num_parts, int head_dim,
                                const float *o_parts, const float *lse_parts, const void *o,
                                const float *lse, bool *empty) {
  *empty = false;
  if (!dtype_ok(dtype)) return FA_ERR_UNSUPPORTED;
  if (num_rows < 0 || num_parts <= 0) return FA_ERR_INVALID_PROBLEM;
  if (!head_dim_ok(head_dim)) return FA_ERR_UNSUPPORTED;
  if (num_rows == 0) {
    *empty = true;
    return FA_OK;
  }
  if (!o_parts || !lse_parts || !o) return FA_ERR_INVALID_PROBLEM;
  if (!all_aligned({o_parts, o}, {lse_parts, lse})) return FA_ERR_INVALID_PROBLEM;
  if (double(num_parts) * num_rows * head_dim >= 1.0e15) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace fa_plan
