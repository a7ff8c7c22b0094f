"""Test-side helpers: build paged and contiguous layouts from *logical* rows.

The page-table scatter here is written independently of the oracle's gather (it
is the inverse operation), so a test can start from the logical rows of each
request, lay them out in a paged store, and check what the oracle (or the HIP
library) reads back.
"""
import math

import numpy as np
import torch

import workloads as W


def rand_t(rng, shape, dtype, std=1.0):
    """float32 N(0, std) rounded to dtype (RNE) as a torch CPU tensor."""
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(std)
    return torch.from_numpy(x).to(W.TORCH_DTYPES[dtype])


def f64(t):
    """Exact float64 values of a CPU tensor (a library conversion, not the oracle's)."""
    return t.to(torch.float64).numpy()


def scatter_paged(rows, page_size, rng, pool_extra=0, empty_last_page=(), fill=None,
                  permute=True, layout="hnd"):
    """Lays logical rows out in a paged store.

    rows: list over requests of tensors [L_b, Hkv, D] (one dtype).
    empty_last_page: requests that get one more, empty page (last_page_len 0);
      their L_b must be a multiple of page_size.
    Returns (data [pool, Hkv, P, D] -- [pool, P, Hkv, D] for layout "nhd" --,
    indices, indptr, last_page_len) where unused memory holds `fill` (default
    NaN)."""
    batch = len(rows)
    hkv, d = rows[0].shape[1], rows[0].shape[2]
    dtype = rows[0].dtype
    n_pages, lpl = [], []
    for b, r in enumerate(rows):
        L = r.shape[0]
        n = math.ceil(L / page_size)
        last = L - (n - 1) * page_size if n else 0
        if b in empty_last_page:
            assert L % page_size == 0
            n += 1
            last = 0
        n_pages.append(n)
        lpl.append(last)
    used = sum(n_pages)
    pool = max(1, used + pool_extra)
    perm = rng.permutation(pool) if permute else np.arange(pool)
    shape = (pool, page_size, hkv, d) if layout == "nhd" else (pool, hkv, page_size, d)
    data = torch.full(shape, float("nan") if fill is None else fill, dtype=dtype)
    indices = np.zeros(used, dtype=np.int32)
    indptr = np.zeros(batch + 1, dtype=np.int32)
    k = 0
    for b, r in enumerate(rows):
        indptr[b] = k
        for p in range(n_pages[b]):
            page = int(perm[k])
            indices[k] = page
            lo = p * page_size
            hi = min(r.shape[0], lo + page_size)
            if hi > lo and layout == "nhd":
                # a page is [P, Hkv, D], like the logical rows [L, Hkv, D]
                data[page, : hi - lo] = r[lo:hi]
            elif hi > lo:
                # a page is [Hkv, P, D]; logical rows are [L, Hkv, D]
                data[page, :, : hi - lo, :] = r[lo:hi].permute(1, 0, 2)
            k += 1
    indptr[batch] = k
    return data, indices, indptr, np.asarray(lpl, dtype=np.int32)


def contig_from_rows(rows, max_kv_len, fill=1.0e4, layout="hnd"):
    """[L, Hkv, D] logical rows -> [Hkv, max_kv_len, D] cache ([max_kv_len, Hkv, D]
    for layout "nhd"); slack holds fill."""
    L, hkv, d = rows.shape
    if layout == "nhd":
        cache = torch.full((max_kv_len, hkv, d), fill, dtype=rows.dtype)
        cache[:L] = rows
        return cache
    cache = torch.full((hkv, max_kv_len, d), fill, dtype=rows.dtype)
    cache[:, :L, :] = rows.permute(1, 0, 2)
    return cache
