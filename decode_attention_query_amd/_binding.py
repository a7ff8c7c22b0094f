"""ctypes binding of libfadecode.so: the C entry points under their own names.

Argument marshalling only: buffers are torch tensors (device memory), their
shapes, dtypes, devices and contiguity are checked on the host against the
dimensions passed (so no kernel is launched on operands smaller than it
assumes), pointers and the current HIP stream are handed to the library, and
a non-OK status raises FaError.  Every step of the computation runs in the HIP
library; there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfadecode.so")

FA_DTYPE_F32, FA_DTYPE_F16, FA_DTYPE_BF16 = 0, 1, 2
DTYPE_CODES = {"f32": FA_DTYPE_F32, "f16": FA_DTYPE_F16, "bf16": FA_DTYPE_BF16}
TORCH_DTYPE_CODES = {torch.float32: FA_DTYPE_F32, torch.float16: FA_DTYPE_F16,
                     torch.bfloat16: FA_DTYPE_BF16}
CODE_TORCH_DTYPES = {v: k for k, v in TORCH_DTYPE_CODES.items()}

FA_OK, FA_ERR_INVALID_PROBLEM, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE_TOO_SMALL, FA_ERR_LAUNCH = \
    range(5)
FA_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/fa_decode.h
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_INVALID_PROBLEM", 2: "FA_ERR_UNSUPPORTED",
                3: "FA_ERR_WORKSPACE_TOO_SMALL", 4: "FA_ERR_LAUNCH"}

# every symbol the public headers declare
EXPORTED = ("fa_decode_workspace_size", "fa_decode_contig", "fa_decode_paged",
            "fa_decode_paged_noalloc",
            "fa_decode_contig_nhd", "fa_decode_paged_nhd", "fa_append_paged",
            "fa_append_paged_nhd", "fa_decode_paged_opts", "fa_decode_contig_opts",
            "fa_merge_states", "fa_status_string",
            "fa_debug_gather_paged", "fa_debug_gather_paged_nhd", "fa_debug_timing_enable",
            "fa_debug_timing_read", "fa_debug_plan", "fa_debug_schedule",
            "fa_debug_read_probe", "fa_debug_counters_in_use")


class DecodeOptions(ctypes.Structure):
    """fa_decode_options_t: K/V layout (0 heads-major, 1 token-major), sliding
    window (rows, 0 = off), logits soft-cap (0 = off), the device address of
    f32 ALiBi slopes [Hq] (None = off) and of a packed custom mask with its
    size in bytes (None = off)."""
    _fields_ = [("kv_layout", ctypes.c_int), ("window", ctypes.c_int),
                ("logits_soft_cap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p),
                ("custom_mask", ctypes.c_void_p), ("custom_mask_bytes", ctypes.c_size_t)]


class FaError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}")


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_I64 = ctypes.c_int64


def load_library():
    """Loads libfadecode.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_decode_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I]
    lib.fa_decode_workspace_size.restype = _SZ
    for name in ("fa_decode_contig", "fa_decode_contig_nhd"):
        getattr(lib, name).argtypes = [_I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _SZ,
                                       _P]
        getattr(lib, name).restype = _I
    for name in ("fa_decode_paged", "fa_decode_paged_nhd"):
        getattr(lib, name).argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P,
                                       _P, _P, _P, _P, _SZ, _P]
        getattr(lib, name).restype = _I
    lib.fa_decode_paged_noalloc.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P,
                                            _P, _P, _P, _P, _P, _P]
    lib.fa_decode_paged_noalloc.restype = _I
    lib.fa_status_string.argtypes = [_I]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_decode_contig_opts.argtypes = [_P] + list(lib.fa_decode_contig.argtypes)
    lib.fa_decode_contig_opts.restype = _I
    lib.fa_decode_paged_opts.argtypes = [_P] + list(lib.fa_decode_paged.argtypes)
    lib.fa_decode_paged_opts.restype = _I
    for name in ("fa_append_paged", "fa_append_paged_nhd"):
        getattr(lib, name).argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P,
                                       _P]
        getattr(lib, name).restype = _I
    for name in ("fa_debug_gather_paged", "fa_debug_gather_paged_nhd"):
        getattr(lib, name).argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I64,
                                       _P, _SZ, _P]
        getattr(lib, name).restype = _I
    lib.fa_merge_states.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, _P]
    lib.fa_merge_states.restype = _I
    lib.fa_debug_timing_enable.argtypes = [_I]
    lib.fa_debug_timing_enable.restype = _I
    lib.fa_debug_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int)]
    lib.fa_debug_timing_read.restype = _I
    lib.fa_debug_plan.argtypes = [_I, _I, _I, _I, _I, _I, _I] + [ctypes.POINTER(_I)] * 4
    lib.fa_debug_plan.restype = _I
    lib.fa_debug_schedule.argtypes = [_I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I64, _P]
    lib.fa_debug_schedule.restype = _I
    lib.fa_debug_counters_in_use.argtypes = [_I, _I, _I, _I, _I, _I, _P, _SZ, _P, _P]
    lib.fa_debug_counters_in_use.restype = _I
    lib.fa_debug_read_probe.argtypes = [_P, _SZ, _P, _P]
    lib.fa_debug_read_probe.restype = _I
    _lib = lib
    return lib


# ------------------------------------------------------------ marshalling

def _dev_buf(t, name, numel, dtype=None, allow_none=False):
    """Device pointer of a dense tensor holding exactly `numel` elements."""
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t.data_ptr()


def _workspace(ws, need):
    if ws is None:
        raise ValueError("workspace is required")
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    return ws.data_ptr(), nbytes


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn, status):
    if status != FA_OK:
        raise FaError(fn, status)


# --------------------------------------------------------- the C entry points

def fa_decode_workspace_size(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                             total_used_pages):
    return int(load_library().fa_decode_workspace_size(batch, num_qo_heads, num_kv_heads,
                                                       head_dim, page_size, total_used_pages))


def _contig(fn, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
            scale, q, k_cache, v_cache, o, lse, workspace, stream, opts=None):
    lib = load_library()
    call = getattr(lib, fn)
    if opts is not None:
        raw = call
        call = lambda *a: raw(ctypes.byref(opts), *a)  # noqa: E731
    tdt = CODE_TORCH_DTYPES.get(dtype)
    if tdt is None:  # let the library report the unsupported dtype
        _check(fn, call(dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                        scale, None, None, None, None, None, None, 0, None))
    kv_numel = num_kv_heads * max_kv_len * head_dim
    args = (
        _dev_buf(q, "q", num_qo_heads * head_dim, tdt),
        _dev_buf(k_cache, "k_cache", kv_numel, tdt),
        _dev_buf(v_cache, "v_cache", kv_numel, tdt),
        _dev_buf(o, "o", num_qo_heads * head_dim, tdt),
        _dev_buf(lse, "lse", num_qo_heads, torch.float32, allow_none=True),
    )
    ws_ptr, ws_bytes = _workspace(workspace, None)
    _check(fn, call(dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                    float(scale), *args, ws_ptr, ws_bytes, _stream(stream)))


def fa_decode_contig(dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                     scale, q, k_cache, v_cache, o, lse, workspace, stream=None):
    """k_cache, v_cache [Hkv, max_kv_len, D] (heads-major)."""
    _contig("fa_decode_contig", dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
            valid_kv_len, scale, q, k_cache, v_cache, o, lse, workspace, stream)


def fa_decode_contig_nhd(dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                         scale, q, k_cache, v_cache, o, lse, workspace, stream=None):
    """k_cache, v_cache [max_kv_len, Hkv, D] (token-major)."""
    _contig("fa_decode_contig_nhd", dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
            valid_kv_len, scale, q, k_cache, v_cache, o, lse, workspace, stream)


def _paged(fn, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size, num_total_pages,
           total_used_pages, sm_scale, q, k_data, v_data, indices, indptr, last_page_len, o,
           lse, workspace, stream, opts=None):
    lib = load_library()
    call = getattr(lib, fn)
    if opts is not None:
        raw = call
        call = lambda *a: raw(ctypes.byref(opts), *a)  # noqa: E731
    tdt = CODE_TORCH_DTYPES.get(dtype)
    if tdt is None:
        _check(fn, call(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                        num_total_pages, total_used_pages, sm_scale, *([None] * 9), 0, None))
    pool = num_total_pages * num_kv_heads * page_size * head_dim
    args = (
        _dev_buf(q, "q", batch * num_qo_heads * head_dim, tdt),
        _dev_buf(k_data, "k_data", pool, tdt),
        _dev_buf(v_data, "v_data", pool, tdt),
        _dev_buf(indices, "indices", total_used_pages, torch.int32,
                 allow_none=total_used_pages == 0),
        _dev_buf(indptr, "indptr", batch + 1, torch.int32),
        _dev_buf(last_page_len, "last_page_len", batch, torch.int32),
        _dev_buf(o, "o", batch * num_qo_heads * head_dim, tdt),
        _dev_buf(lse, "lse", batch * num_qo_heads, torch.float32),
    )
    ws_ptr, ws_bytes = _workspace(workspace, None)
    _check(fn, call(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                    num_total_pages, total_used_pages, float(sm_scale), *args, ws_ptr, ws_bytes,
                    _stream(stream)))


def fa_decode_paged(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                    num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                    indptr, last_page_len, o, lse, workspace, stream=None):
    """k_data, v_data [pages, Hkv, P, D] (heads-major)."""
    _paged("fa_decode_paged", dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
           num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices, indptr,
           last_page_len, o, lse, workspace, stream)


def fa_decode_paged_noalloc(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                            num_total_pages, total_used_pages, sm_scale, q, k_data, v_data,
                            indices, indptr, last_page_len, o, lse, stream=None):
    """fa_decode_paged without a workspace: the library's static scratch array
    (FA_NOALLOC_SCRATCH_BYTES per GPU) holds the split partials."""
    lib = load_library()
    fn = "fa_decode_paged_noalloc"
    tdt = CODE_TORCH_DTYPES.get(dtype)
    if tdt is None:
        _check(fn, lib.fa_decode_paged_noalloc(dtype, batch, num_qo_heads, num_kv_heads,
                                               head_dim, page_size, num_total_pages,
                                               total_used_pages, sm_scale, *([None] * 8),
                                               None))
    pool = num_total_pages * num_kv_heads * page_size * head_dim
    args = (
        _dev_buf(q, "q", batch * num_qo_heads * head_dim, tdt),
        _dev_buf(k_data, "k_data", pool, tdt),
        _dev_buf(v_data, "v_data", pool, tdt),
        _dev_buf(indices, "indices", total_used_pages, torch.int32,
                 allow_none=total_used_pages == 0),
        _dev_buf(indptr, "indptr", batch + 1, torch.int32),
        _dev_buf(last_page_len, "last_page_len", batch, torch.int32),
        _dev_buf(o, "o", batch * num_qo_heads * head_dim, tdt),
        _dev_buf(lse, "lse", batch * num_qo_heads, torch.float32),
    )
    _check(fn, lib.fa_decode_paged_noalloc(dtype, batch, num_qo_heads, num_kv_heads, head_dim,
                                           page_size, num_total_pages, total_used_pages,
                                           float(sm_scale), *args, _stream(stream)))


def fa_decode_paged_opts(opts, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                         num_total_pages, total_used_pages, sm_scale, q, k_data, v_data,
                         indices, indptr, last_page_len, o, lse, workspace, stream=None):
    """opts: DecodeOptions (layout, window, soft-cap)."""
    _paged("fa_decode_paged_opts", dtype, batch, num_qo_heads, num_kv_heads, head_dim,
           page_size, num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
           indptr, last_page_len, o, lse, workspace, stream, opts=opts)


def fa_decode_contig_opts(opts, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
                          valid_kv_len, scale, q, k_cache, v_cache, o, lse, workspace,
                          stream=None):
    """opts: DecodeOptions (layout, window, soft-cap)."""
    _contig("fa_decode_contig_opts", dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len,
            valid_kv_len, scale, q, k_cache, v_cache, o, lse, workspace, stream, opts=opts)


def fa_decode_paged_nhd(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                        num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices,
                        indptr, last_page_len, o, lse, workspace, stream=None):
    """k_data, v_data [pages, P, Hkv, D] (token-major)."""
    _paged("fa_decode_paged_nhd", dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
           num_total_pages, total_used_pages, sm_scale, q, k_data, v_data, indices, indptr,
           last_page_len, o, lse, workspace, stream)


def fa_debug_gather_paged(dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                          total_used_pages, data, indices, indptr, last_page_len, out,
                          out_rows, workspace, stream=None, layout="hnd"):
    """layout "nhd" calls fa_debug_gather_paged_nhd (data [pages, P, Hkv, D])."""
    lib = load_library()
    fn = "fa_debug_gather_paged_nhd" if layout == "nhd" else "fa_debug_gather_paged"
    tdt = CODE_TORCH_DTYPES[dtype]
    args = (
        _dev_buf(data, "data", num_total_pages * num_kv_heads * page_size * head_dim, tdt),
        _dev_buf(indices, "indices", total_used_pages, torch.int32,
                 allow_none=total_used_pages == 0),
        _dev_buf(indptr, "indptr", batch + 1, torch.int32),
        _dev_buf(last_page_len, "last_page_len", batch, torch.int32),
        _dev_buf(out, "out", out_rows * num_kv_heads * head_dim, tdt),
    )
    ws_ptr, ws_bytes = _workspace(workspace, None)
    _check(fn, getattr(lib, fn)(
        dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages, total_used_pages,
        *args, int(out_rows), ws_ptr, ws_bytes, _stream(stream)))


def fa_debug_timing_enable(enable):
    _check("fa_debug_timing_enable", load_library().fa_debug_timing_enable(int(bool(enable))))


def fa_debug_timing_read():
    """(main kernel ms, whole call ms, calls) summed since the last read."""
    a, b, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    _check("fa_debug_timing_read", load_library().fa_debug_timing_read(
        ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, n.value


def fa_debug_plan(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                  total_used_pages):
    """(chunk rows, units bound, heads per unit, kernel kind) of a call's plan."""
    out = [ctypes.c_int() for _ in range(4)]
    _check("fa_debug_plan", load_library().fa_debug_plan(
        dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_used_pages,
        *[ctypes.byref(x) for x in out]))
    return tuple(x.value for x in out)


def fa_debug_schedule(dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                      total_used_pages, indptr, last_page_len, out, stream=None):
    """Fills out (device int32, 8 per work index) with the split-unit schedule."""
    lib = load_library()
    if not isinstance(out, torch.Tensor) or out.device.type != "cuda" or \
            out.dtype != torch.int32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 device tensor")
    _check("fa_debug_schedule", lib.fa_debug_schedule(
        dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_used_pages,
        _dev_buf(indptr, "indptr", batch + 1, torch.int32),
        _dev_buf(last_page_len, "last_page_len", batch, torch.int32),
        out.data_ptr(), out.numel(), _stream(stream)))


def fa_debug_counters_in_use(batch, num_qo_heads, num_kv_heads, head_dim, page_size,
                             total_used_pages, workspace, stream=None):
    """How many of the workspace's counters a paged call of these dimensions
    uses were left part counted (synchronises the stream to read the answer)."""
    lib = load_library()
    ws_ptr, ws_bytes = _workspace(workspace, None)
    out = torch.zeros(1, dtype=torch.int32, device=workspace.device)
    _check("fa_debug_counters_in_use", lib.fa_debug_counters_in_use(
        batch, num_qo_heads, num_kv_heads, head_dim, page_size, total_used_pages, ws_ptr,
        ws_bytes, out.data_ptr(), _stream(stream)))
    return int(out.item())


def fa_debug_read_probe(buf, sink, stream=None):
    """Streams every byte of buf (a contiguous device tensor) once."""
    lib = load_library()
    for t, name in ((buf, "buf"), (sink, "sink")):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if sink.dtype != torch.int32 or sink.numel() < 1:
        raise ValueError("sink must be an int32 device tensor")
    _check("fa_debug_read_probe", lib.fa_debug_read_probe(
        buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), _stream(stream)))


def _append(fn, dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
            total_used_pages, k_new, v_new, indices, indptr, last_page_len, k_data, v_data,
            stream):
    lib = load_library()
    call = getattr(lib, fn)
    tdt = CODE_TORCH_DTYPES.get(dtype)
    if tdt is None:
        _check(fn, call(dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                        total_used_pages, *([None] * 7), None))
    rows = batch * num_kv_heads * head_dim
    pool = num_total_pages * num_kv_heads * page_size * head_dim
    args = (
        _dev_buf(k_new, "k_new", rows, tdt),
        _dev_buf(v_new, "v_new", rows, tdt),
        _dev_buf(indices, "indices", total_used_pages, torch.int32,
                 allow_none=total_used_pages == 0),
        _dev_buf(indptr, "indptr", batch + 1, torch.int32),
        _dev_buf(last_page_len, "last_page_len", batch, torch.int32),
        _dev_buf(k_data, "k_data", pool, tdt),
        _dev_buf(v_data, "v_data", pool, tdt),
    )
    _check(fn, call(dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                    total_used_pages, *args, _stream(stream)))


def fa_append_paged(dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                    total_used_pages, k_new, v_new, indices, indptr, last_page_len, k_data,
                    v_data, stream=None):
    """k_data, v_data [pages, Hkv, P, D] (heads-major), updated in place."""
    _append("fa_append_paged", dtype, batch, num_kv_heads, head_dim, page_size,
            num_total_pages, total_used_pages, k_new, v_new, indices, indptr, last_page_len,
            k_data, v_data, stream)


def fa_append_paged_nhd(dtype, batch, num_kv_heads, head_dim, page_size, num_total_pages,
                        total_used_pages, k_new, v_new, indices, indptr, last_page_len, k_data,
                        v_data, stream=None):
    """k_data, v_data [pages, P, Hkv, D] (token-major), updated in place."""
    _append("fa_append_paged_nhd", dtype, batch, num_kv_heads, head_dim, page_size,
            num_total_pages, total_used_pages, k_new, v_new, indices, indptr, last_page_len,
            k_data, v_data, stream)


def fa_merge_states(dtype, num_rows, num_parts, head_dim, o_parts, lse_parts, o, lse=None,
                    stream=None):
    """o_parts [num_parts, num_rows, D] f32, lse_parts [num_parts, num_rows] f32 ->
    o [num_rows, D] in dtype, lse [num_rows] f32 (None: not written)."""
    lib = load_library()
    tdt = CODE_TORCH_DTYPES.get(dtype)
    if tdt is None or num_rows <= 0 or num_parts <= 0:
        # the library reports the problem with the arguments (or, for no rows,
        # accepts the call without looking at the buffers)
        _check("fa_merge_states", lib.fa_merge_states(dtype, num_rows, num_parts, head_dim,
                                                      None, None, None, None, _stream(stream)))
        return
    args = (
        _dev_buf(o_parts, "o_parts", num_parts * num_rows * head_dim, torch.float32),
        _dev_buf(lse_parts, "lse_parts", num_parts * num_rows, torch.float32),
        _dev_buf(o, "o", num_rows * head_dim, tdt),
        _dev_buf(lse, "lse", num_rows, torch.float32, allow_none=True),
    )
    _check("fa_merge_states", lib.fa_merge_states(dtype, num_rows, num_parts, head_dim, *args,
                                                  _stream(stream)))


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()
