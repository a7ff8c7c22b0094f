"""Float64 CPU oracle for single-query GQA decode attention.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP
library (decode_attention_query_amd) and imports nothing from it.

The arithmetic lives in decode_ref.c (plain C, f64, two-pass softmax); this
module only marshals numpy arrays into it.  Element arrays are passed as raw
bits: float32 arrays as-is, f16 and bf16 as their 16-bit patterns (uint16 /
int16 / float16 numpy arrays; numpy has no bf16, so bf16 is always bits).

Functions and what they follow:
  decode_contig  -- contiguous [Hkv, max_kv_len, D] cache masked to valid_kv_len
                    (ferrum-kernels 0.7.7 src/backend/cuda/decode_attention.rs,
                    decode_attention argument list and module doc); layout="nhd":
                    token-major [max_kv_len, Hkv, D] (ferrox-cuda 0.15.2
                    src/attn.rs, gqa_decode kernel source)
  decode_paged   -- paged [pages, Hkv, P, D] store via indptr/indices/last_page_len
                    (baracuda-kernels 0.0.1-alpha.68 src/attention/batch_paged_decode.rs,
                    module doc "Layout" and "Query / output"); layout="nhd":
                    [pages, P, Hkv, D] (reading: the page-level token-major form)
  gather_paged   -- the page-table-resolved rows, raw bits (same page, "Layout")
  append_paged   -- decode-time append of one new K/V row per request (same page,
                    "Companion plans"; reading: the table already counts the row)
  seq_lens       -- L_b from the page table (reading: all pages but the last are full)
  validate_table -- the device-side page-table contract (same page, "Layout")
  attend_f64     -- one query row over explicit f64 rows (a split's partial)
  merge          -- combine partials over a partition of the rows via their lse
Both decode functions take window= (sliding window, the last `window` rows),
softcap= (scores c * tanh(x / c)) and alibi= (per-head slopes of a linear
distance penalty), the variants the baracuda-kernels page lists as unsupported
by its plan (module doc "Constraints"); 0 / None turns each off.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
LAYOUTS = {"hnd": 0, "nhd": 1}

STATUS = {0: "OK", 1: "BAD_ARG", 2: "BAD_INDPTR", 3: "BAD_INDEX",
          4: "BAD_LAST_PAGE_LEN", 5: "NO_MEMORY"}

_P = ctypes.c_void_p
_I = ctypes.c_int
_D = ctypes.c_double
_I64 = ctypes.c_int64


class _Lib:
    """A loaded build of decode_ref.c (the default one, or a test's variant)."""

    def __init__(self, path):
        lib = ctypes.CDLL(path)
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_to_f64.restype = _D
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = _D
        lib.oracle_validate_table.argtypes = [_I, _I, _I, _I, _P, _P, _P]
        lib.oracle_validate_table.restype = _I
        lib.oracle_seq_lens.argtypes = [_I, _I, _P, _P, _P]
        lib.oracle_seq_lens.restype = None
        lib.oracle_gather_paged.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I]
        lib.oracle_gather_paged.restype = _I
        lib.oracle_decode_paged.argtypes = [_I, _I, _I, _I, _I, _I, _D, _P, _P, _P, _P, _P,
                                            _P, _I, _P, _P, _P, _P, _I, _I, _I, _D, _P, _P]
        lib.oracle_decode_paged.restype = _I
        lib.oracle_decode_contig.argtypes = [_I, _I, _I, _I, _I, _I, _D, _P, _P, _P, _P, _P,
                                             _I, _I, _I, _D, _P, _P]
        lib.oracle_decode_contig.restype = _I
        lib.oracle_attend_f64.argtypes = [_I, _I64, _D, _P, _P, _P, _P, _P]
        lib.oracle_attend_f64.restype = None
        lib.oracle_merge.argtypes = [_I, _I, _P, _P, _P, _P]
        lib.oracle_merge.restype = None
        lib.oracle_append_paged.argtypes = [_I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I]
        lib.oracle_append_paged.restype = _I
        self.lib = lib


_variant = None  # set by use_library() to test a variant build


def use_library(path):
    """Route every function of this module through another build of
    decode_ref.c (None restores the default).  Used by the tests that plant a
    mistake in a copy of the oracle and check that a pin catches it."""
    global _variant
    _variant = None if path is None else _Lib(path)


def _load():
    global _lib
    if _variant is not None:
        return _variant.lib
    if _lib is not None:
        return _lib.lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "decode_ref.c"))):
        from . import build as _build
        _build.build()
    _lib = _Lib(_LIB_PATH)
    return _lib.lib


def _bits(a, dtype):
    """Raw element storage for the C side (C-contiguous)."""
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError(f"f32 data must be float32, got {a.dtype}")
    else:
        if a.dtype.itemsize != 2:
            raise TypeError(f"{dtype} data must be 16-bit patterns, got {a.dtype}")
    return a


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


_keep = []
_keep_mask = []


def _slopes(alibi, hq):
    """Pointer to the ALiBi slopes as f64 [Hq], or NULL."""
    if alibi is None:
        return None
    a = np.ascontiguousarray(np.asarray(alibi, dtype=np.float64))
    assert a.shape == (hq,)
    _keep[:] = [a]  # alive for the duration of the call
    return _ptr(a)


def _mask(mask, total_rows):
    """Pointer to a packed custom mask (uint8, bit i at byte i // 8, bit i % 8,
    at least total_rows bits), or NULL."""
    if mask is None:
        return None
    m = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(-1))
    assert m.size * 8 >= total_rows, "custom mask shorter than the rows it covers"
    _keep_mask[:] = [m]  # alive for the duration of the call
    return _ptr(m)


def f16_to_f64(bits: int) -> float:
    return _load().oracle_f16_to_f64(int(bits) & 0xFFFF)


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def validate_table(batch, page_size, num_total_pages, indices, indptr, last_page_len):
    indices, indptr, lpl = _i32(indices), _i32(indptr), _i32(last_page_len)
    if indptr.shape != (batch + 1,) or lpl.shape != (batch,):
        return "BAD_ARG"
    r = _load().oracle_validate_table(batch, page_size, num_total_pages, int(indices.size),
                                      _ptr(indices), _ptr(indptr), _ptr(lpl))
    return STATUS[r]


def seq_lens(page_size, indptr, last_page_len):
    indptr, lpl = _i32(indptr), _i32(last_page_len)
    out = np.zeros(lpl.size, dtype=np.int64)
    _load().oracle_seq_lens(int(lpl.size), page_size, _ptr(indptr), _ptr(lpl), _ptr(out))
    return out


def _paged_dims(shape, layout):
    """(Hkv, P, D) of a paged store's shape in the given layout."""
    if layout == "nhd":
        _, page_size, hkv, head_dim = shape
    elif layout == "hnd":
        _, hkv, page_size, head_dim = shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return hkv, page_size, head_dim


def gather_paged(dtype, data, indices, indptr, last_page_len, layout="hnd"):
    """Resolved rows of a paged store `data` ([pages, Hkv, P, D], or
    [pages, P, Hkv, D] for layout="nhd"), raw bits, as [sum L_b, Hkv, D]."""
    data = _bits(data, dtype)
    hkv, page_size, head_dim = _paged_dims(data.shape, layout)
    indices, indptr, lpl = _i32(indices), _i32(indptr), _i32(last_page_len)
    total = int(seq_lens(page_size, indptr, lpl).sum())
    out = np.empty((total, hkv, head_dim), dtype=data.dtype)
    r = _load().oracle_gather_paged(DTYPES[dtype], int(lpl.size), hkv, head_dim, page_size,
                                    _ptr(data), _ptr(indices), _ptr(indptr), _ptr(lpl),
                                    _ptr(out), LAYOUTS[layout])
    if r != 0:
        raise RuntimeError(f"oracle_gather_paged: {STATUS[r]}")
    return out


def append_paged(dtype, data, indices, indptr, last_page_len, new_rows, layout="hnd"):
    """A copy of the paged store `data` with request b's new row new_rows[b]
    ([batch, Hkv, D]) written at its last valid row L_b - 1 (none if L_b = 0)."""
    out = np.array(_bits(data, dtype), copy=True)
    new_rows = _bits(new_rows, dtype)
    hkv, page_size, head_dim = _paged_dims(out.shape, layout)
    indices, indptr, lpl = _i32(indices), _i32(indptr), _i32(last_page_len)
    assert new_rows.shape == (lpl.size, hkv, head_dim)
    r = _load().oracle_append_paged(DTYPES[dtype], int(lpl.size), hkv, head_dim, page_size,
                                    _ptr(out), _ptr(indices), _ptr(indptr), _ptr(lpl),
                                    _ptr(new_rows), LAYOUTS[layout])
    if r != 0:
        raise RuntimeError(f"oracle_append_paged: {STATUS[r]}")
    return out


def decode_paged(dtype, q, k_data, v_data, indices, indptr, last_page_len, scale,
                 samples=None, threads=0, layout="hnd", window=0, softcap=0.0, alibi=None,
                 mask=None):
    """q [B, Hq, D]; k_data/v_data [pages, Hkv, P, D] (layout="nhd":
    [pages, P, Hkv, D]).  Returns (o, lse) in f64: o [B, Hq, D], lse [B, Hq];
    with samples=[(b, h), ...] returns o [n, D], lse [n].  window > 0: only the
    last `window` rows of each request; softcap > 0: scores capped with tanh;
    alibi: per query head slopes [Hq] (None: off); mask: packed custom mask,
    one bit per row of every request, requests back to back (None: off)."""
    q, k_data, v_data = _bits(q, dtype), _bits(k_data, dtype), _bits(v_data, dtype)
    batch, hq, head_dim = q.shape
    hkv, page_size, d2 = _paged_dims(k_data.shape, layout)
    assert d2 == head_dim and v_data.shape == k_data.shape
    indices, indptr, lpl = _i32(indices), _i32(indptr), _i32(last_page_len)
    if samples is None:
        n_sample = 0
        sb = sh = np.zeros(1, dtype=np.int32)
        o = np.empty((batch, hq, head_dim), dtype=np.float64)
        lse = np.empty((batch, hq), dtype=np.float64)
    else:
        samples = np.asarray(samples, dtype=np.int32).reshape(-1, 2)
        n_sample = samples.shape[0]
        sb = np.ascontiguousarray(samples[:, 0])
        sh = np.ascontiguousarray(samples[:, 1])
        o = np.empty((n_sample, head_dim), dtype=np.float64)
        lse = np.empty((n_sample,), dtype=np.float64)
    r = _load().oracle_decode_paged(DTYPES[dtype], batch, hq, hkv, head_dim, page_size,
                                    float(scale), _ptr(q), _ptr(k_data), _ptr(v_data),
                                    _ptr(indices), _ptr(indptr), _ptr(lpl), n_sample,
                                    _ptr(sb), _ptr(sh), _ptr(o), _ptr(lse), int(threads),
                                    LAYOUTS[layout], int(window), float(softcap), _slopes(alibi, hq),
                                    _mask(mask, int(seq_lens(page_size, indptr, lpl).sum())))
    if r != 0:
        raise RuntimeError(f"oracle_decode_paged: {STATUS[r]}")
    return o, lse


def decode_contig(dtype, q, k_cache, v_cache, valid_kv_len, scale, threads=0, layout="hnd",
                  window=0, softcap=0.0, alibi=None, mask=None):
    """q [Hq, D]; k_cache/v_cache [Hkv, max_kv_len, D] (layout="nhd":
    [max_kv_len, Hkv, D]).  Returns (o [Hq, D], lse [Hq]) f64.  mask: packed
    custom mask, bit j for row j (None: off)."""
    q, k_cache, v_cache = _bits(q, dtype), _bits(k_cache, dtype), _bits(v_cache, dtype)
    hq, head_dim = q.shape
    if layout == "nhd":
        max_kv_len, hkv, d2 = k_cache.shape
    elif layout == "hnd":
        hkv, max_kv_len, d2 = k_cache.shape
    else:
        raise ValueError(f"unknown layout {layout!r}")
    assert d2 == head_dim and v_cache.shape == k_cache.shape
    o = np.empty((hq, head_dim), dtype=np.float64)
    lse = np.empty((hq,), dtype=np.float64)
    r = _load().oracle_decode_contig(DTYPES[dtype], hq, hkv, head_dim, max_kv_len,
                                     int(valid_kv_len), float(scale), _ptr(q), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(o), _ptr(lse), int(threads),
                                     LAYOUTS[layout], int(window), float(softcap),
                                     _slopes(alibi, hq), _mask(mask, int(valid_kv_len)))
    if r != 0:
        raise RuntimeError(f"oracle_decode_contig: {STATUS[r]}")
    return o, lse


def attend_f64(q, k, v, scale):
    """One f64 query row q [D] against rows k, v [L, D] (f64)."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64).reshape(-1, q.size)
    v = np.ascontiguousarray(v, dtype=np.float64).reshape(-1, q.size)
    o = np.empty(q.size, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    _load().oracle_attend_f64(q.size, k.shape[0], float(scale), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(o), _ptr(lse))
    return o, float(lse[0])


def merge(o_parts, lse_parts):
    """Merge partials o_parts [S, D] (each normalised over its rows), lse_parts [S]."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64).reshape(-1)
    s, head_dim = o_parts.shape
    o = np.empty(head_dim, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    _load().oracle_merge(head_dim, s, _ptr(o_parts), _ptr(lse_parts), _ptr(o), _ptr(lse))
    return o, float(lse[0])
