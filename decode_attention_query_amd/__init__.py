"""MI355X-native single-query GQA decode attention.

The computation runs in libfadecode.so (hand-written HIP kernels for gfx950);
this package is its binding.  The C entry points are available under their
own names (fa_decode_contig, fa_decode_paged, fa_decode_workspace_size, and
the fa_debug_* hooks); decode_contig, decode_paged, merge_states and
append_paged below are conveniences that read the dimensions off the tensors
and allocate outputs and workspace.
"""
import torch

from ._binding import (CODE_TORCH_DTYPES, DTYPE_CODES, EXPORTED, FA_DTYPE_BF16, FA_DTYPE_F16,
                       FA_DTYPE_F32, FA_ERR_INVALID_PROBLEM, FA_ERR_LAUNCH, FA_ERR_UNSUPPORTED,
                       FA_ERR_WORKSPACE_TOO_SMALL, FA_OK, LIB_PATH, STATUS_NAMES,
                       TORCH_DTYPE_CODES, FaError, fa_debug_gather_paged, fa_debug_plan,
                       fa_debug_read_probe, fa_debug_schedule, fa_debug_timing_enable,
                       fa_debug_timing_read, fa_decode_contig, fa_decode_contig_nhd,
                       fa_decode_paged, fa_decode_paged_nhd, fa_decode_workspace_size,
                       fa_append_paged, fa_append_paged_nhd, fa_merge_states, fa_status_string,
                       load_library,
                       DecodeOptions, fa_decode_paged_opts, fa_decode_contig_opts,
                       fa_decode_paged_noalloc, FA_NOALLOC_SCRATCH_BYTES,
                       fa_debug_counters_in_use)


def _code(t):
    try:
        return TORCH_DTYPE_CODES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported element type {t.dtype}") from None


def _options(layout, window, softcap, alibi, mask, hq):
    slopes = None
    if alibi is not None:
        if not (isinstance(alibi, torch.Tensor) and alibi.device.type == "cuda" and
                alibi.dtype == torch.float32 and alibi.is_contiguous() and alibi.numel() == hq):
            raise ValueError(f"alibi must be a contiguous f32 device tensor of {hq} slopes")
        slopes = alibi.data_ptr()
    mask_ptr, mask_bytes = None, 0
    if mask is not None:
        if not (isinstance(mask, torch.Tensor) and mask.device.type == "cuda" and
                mask.dtype == torch.uint8 and mask.is_contiguous() and mask.numel() > 0):
            raise ValueError("mask must be a non-empty contiguous uint8 device tensor of packed bits")
        mask_ptr, mask_bytes = mask.data_ptr(), mask.numel()
    return DecodeOptions(int(layout == "nhd"), int(window), float(softcap), slopes, mask_ptr,
                         mask_bytes)


def workspace_paged(batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_used_pages,
                    device="cuda"):
    n = fa_decode_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                                 total_used_pages)
    if n == 0:
        raise FaError("fa_decode_workspace_size", FA_ERR_INVALID_PROBLEM)
    return torch.empty(n, dtype=torch.uint8, device=device)


def decode_paged(q, k_data, v_data, indices, indptr, last_page_len, sm_scale, o=None, lse=None,
                 workspace=None, stream=None, layout="hnd", window=0, softcap=0.0, alibi=None,
                 mask=None):
    """q [B, Hq, D]; k_data/v_data [pages, Hkv, P, D] (layout "nhd": [pages, P, Hkv, D]);
    int32 page table; alibi: f32 device tensor [Hq] of slopes; mask: uint8 device
    tensor of packed keep-bits, one per row of every request, requests back to back.
    Returns (o [B, Hq, D] in q's dtype, lse [B, Hq] f32)."""
    batch, hq, d = q.shape
    if layout == "nhd":
        pages, page_size, hkv, d2 = k_data.shape
    elif layout == "hnd":
        pages, hkv, page_size, d2 = k_data.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    if d2 != d or tuple(v_data.shape) != tuple(k_data.shape):
        raise ValueError("q, k_data and v_data disagree on shape")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((batch, hq), dtype=torch.float32, device=q.device)
    used = indices.numel()
    if workspace is None:
        workspace = workspace_paged(batch, hq, hkv, d, page_size, used, q.device)
    args = (_code(q), batch, hq, hkv, d, page_size, pages, used, sm_scale, q, k_data, v_data,
            indices if used else None, indptr, last_page_len, o, lse, workspace, stream)
    if window or softcap or alibi is not None or mask is not None:
        fa_decode_paged_opts(_options(layout, window, softcap, alibi, mask, hq), *args)
    else:
        (fa_decode_paged_nhd if layout == "nhd" else fa_decode_paged)(*args)
    return o, lse


def decode_contig(q, k_cache, v_cache, valid_kv_len, scale, o=None, lse=None, workspace=None,
                  stream=None, layout="hnd", window=0, softcap=0.0, alibi=None, mask=None):
    """q [Hq, D]; k_cache/v_cache [Hkv, max_kv_len, D] (layout "nhd": [max_kv_len, Hkv, D]);
    mask: uint8 device tensor of packed keep-bits, bit j for row j.
    Returns (o [Hq, D] in q's dtype, lse [Hq] f32)."""
    hq, d = q.shape
    if layout == "nhd":
        max_kv_len, hkv, d2 = k_cache.shape
    elif layout == "hnd":
        hkv, max_kv_len, d2 = k_cache.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    if d2 != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("q, k_cache and v_cache disagree on shape")
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq,), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = workspace_paged(1, hq, hkv, d, max_kv_len, 1, q.device)
    args = (_code(q), hq, hkv, d, max_kv_len, valid_kv_len, scale, q, k_cache, v_cache, o, lse,
            workspace, stream)
    if window or softcap or alibi is not None or mask is not None:
        fa_decode_contig_opts(_options(layout, window, softcap, alibi, mask, hq), *args)
    else:
        (fa_decode_contig_nhd if layout == "nhd" else fa_decode_contig)(*args)
    return o, lse


def append_paged(k_new, v_new, k_data, v_data, indices, indptr, last_page_len, stream=None,
                 layout="hnd"):
    """Writes request b's new K/V rows (k_new, v_new [B, Hkv, D]) at its last
    valid row, in place in k_data / v_data ([pages, Hkv, P, D]; layout "nhd":
    [pages, P, Hkv, D]).  The page table must already count the new token."""
    batch, hkv, d = k_new.shape
    if layout == "nhd":
        pages, page_size, hkv2, d2 = k_data.shape
    elif layout == "hnd":
        pages, hkv2, page_size, d2 = k_data.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    if (hkv2, d2) != (hkv, d) or tuple(v_data.shape) != tuple(k_data.shape) or \
            tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError("k_new, v_new, k_data and v_data disagree on shape")
    used = indices.numel()
    fn = fa_append_paged_nhd if layout == "nhd" else fa_append_paged
    fn(_code(k_new), batch, hkv, d, page_size, pages, used, k_new, v_new,
       indices if used else None, indptr, last_page_len, k_data, v_data, stream)


def merge_states(o_parts, lse_parts, out_dtype=torch.float32, o=None, lse=None, stream=None):
    """Combines split partials: o_parts [S, ..., D] f32 and lse_parts [S, ...] f32
    (natural log; -inf marks an empty part) -> o [..., D] in out_dtype and
    lse [...] f32, the result over the union of the parts' rows."""
    if o_parts.dim() < 2 or tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError("o_parts must be [S, ..., D] and lse_parts [S, ...]")
    s, d = o_parts.shape[0], o_parts.shape[-1]
    rows = 1
    for n in lse_parts.shape[1:]:
        rows *= int(n)
    if o is None:
        o = torch.empty(tuple(o_parts.shape[1:]), dtype=out_dtype, device=o_parts.device)
    if lse is None:
        lse = torch.empty(tuple(lse_parts.shape[1:]), dtype=torch.float32,
                          device=o_parts.device)
    fa_merge_states(_code(o), rows, s, d, o_parts, lse_parts, o, lse, stream)
    return o, lse
