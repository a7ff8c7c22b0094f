"""Seeded synthetic inputs for single-query GQA decode attention.

Shared by the tests, the benchmark and the smoke check, on both sides of a
parity comparison (the HIP library and the float64 oracle).  This module holds
none of the attention arithmetic: it only draws values and builds page tables.

Recipe (every config):
  * numpy SeedSequence(seed) is split into five child streams, used for, in
    order: request lengths, the physical page permutation, q, K, V.
  * K and V pools are drawn in blocks of PAGE_BLOCK pages, block i from child i
    of the K (or V) stream, so blocks can be drawn in parallel threads and the
    result does not depend on the thread count.
  * Values are drawn as float32 N(0, 1), multiplied by the config's standard
    deviation (a power of two, so exactly), and cast to the element type with
    round-to-nearest-even (torch CPU .to()).
  * Poison: K/V rows that exist in memory but lie outside a request's valid
    range (tail rows of its last page, contiguous slots past valid_kv_len) hold
    1e4; pool pages that no request references hold NaN.  Neither may change any
    output bit.
  * Paged requests take consecutive ids from the permuted pool; indptr is their
    prefix sum; last_page_len = ((L - 1) % P) + 1 for L >= 1.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
PAGE_BLOCK = 256          # pages per independently seeded draw block
POISON_ROW = 1.0e4        # excluded-but-present rows
POISON_PAGE = float("nan")  # pages nobody references
_THREADS = 8


@dataclass
class ContigProblem:
    name: str
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    max_kv_len: int
    valid_kv_len: int
    scale: float
    q: torch.Tensor          # [Hq, D]
    k_cache: torch.Tensor    # [Hkv, max_kv_len, D]; [max_kv_len, Hkv, D] if token-major
    v_cache: torch.Tensor    # same
    layout: str = "hnd"      # "hnd" heads-major, "nhd" token-major

    @property
    def group(self):
        return self.num_qo_heads // self.num_kv_heads


@dataclass
class PagedProblem:
    name: str
    dtype: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_total_pages: int
    scale: float
    q: torch.Tensor          # [B, Hq, D]
    k_data: torch.Tensor     # [pages, Hkv, P, D]; [pages, P, Hkv, D] if token-major
    v_data: torch.Tensor     # same
    indices: torch.Tensor    # [total_used_pages] int32
    indptr: torch.Tensor     # [B + 1] int32
    last_page_len: torch.Tensor  # [B] int32
    kv_lens: np.ndarray = field(default=None)  # lengths the recipe drew (int64)
    layout: str = "hnd"      # "hnd" heads-major, "nhd" token-major

    @property
    def total_used_pages(self):
        return int(self.indices.numel())

    @property
    def group(self):
        return self.num_qo_heads // self.num_kv_heads


def token_major(p):
    """The same problem with K and V stored token-major: contiguous
    [max_kv_len, Hkv, D], paged [pages, P, Hkv, D] (same values, same page
    table)."""
    import dataclasses
    assert p.layout == "hnd"
    if isinstance(p, ContigProblem):
        return dataclasses.replace(p, name=p.name + "_nhd", layout="nhd",
                                   k_cache=p.k_cache.permute(1, 0, 2).contiguous(),
                                   v_cache=p.v_cache.permute(1, 0, 2).contiguous())
    return dataclasses.replace(p, name=p.name + "_nhd", layout="nhd",
                               k_data=p.k_data.permute(0, 2, 1, 3).contiguous(),
                               v_data=p.v_data.permute(0, 2, 1, 3).contiguous())


def pack_mask(keep) -> np.ndarray:
    """A custom mask in the packed form the library and the oracle read: the
    flattened booleans (row i of the concatenated per-request rows) at byte
    i // 8, bit i % 8; a set bit keeps the row."""
    return np.packbits(np.asarray(keep, dtype=bool).reshape(-1), bitorder="little")


def random_mask(seed, lens, keep=0.5, blocks=False) -> np.ndarray:
    """Seeded keep-booleans for requests of the given lengths, concatenated in
    request order: independent rows kept with probability `keep`; with
    blocks=True, runs of 1-40 rows kept or dropped together; with an integer
    blocks=R, runs of R rows (a block-sparse mask) kept or dropped together."""
    rng = np.random.default_rng(seed)
    total = int(np.sum(lens))
    if blocks is False:
        return rng.random(total) < keep
    if blocks is not True:
        run = int(blocks)
        assert run > 0
        flags = rng.random((total + run - 1) // run) < keep
        return np.repeat(flags, run)[:total]
    out = np.empty(total, dtype=bool)
    i = 0
    while i < total:
        n = int(rng.integers(1, 41))
        out[i:i + n] = rng.random() < keep
        i += n
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw element storage of a CPU tensor as numpy (float32, or uint16 patterns)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_scale(x: float) -> float:
    """The float32 value nearest to x, as a Python float."""
    return float(np.float32(x))


def _draw_pool(ss: np.random.SeedSequence, shape, std: float, dtype: str) -> torch.Tensor:
    """[pages, ...] pool drawn blockwise from children of ss, cast to dtype."""
    pages = shape[0]
    per_page = int(np.prod(shape[1:]))
    n_blocks = max(1, math.ceil(pages / PAGE_BLOCK))
    kids = ss.spawn(n_blocks)
    out = torch.empty(shape, dtype=TORCH_DTYPES[dtype])
    flat = out.view(pages, per_page)

    def fill(i):
        p0 = i * PAGE_BLOCK
        p1 = min(pages, p0 + PAGE_BLOCK)
        buf = np.random.default_rng(kids[i]).standard_normal((p1 - p0) * per_page,
                                                               dtype=np.float32)
        if std != 1.0:
            buf *= np.float32(std)
        flat[p0:p1] = torch.from_numpy(buf.reshape(p1 - p0, per_page)).to(out.dtype)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, range(n_blocks)))
    return out


def pages_for_lens(lens, page_size):
    """Page counts and last_page_len for requests of the given lengths."""
    lens = np.asarray(lens, dtype=np.int64)
    n_pages = (lens + page_size - 1) // page_size
    lpl = np.where(lens > 0, (lens - 1) % page_size + 1, 0)
    return n_pages.astype(np.int64), lpl.astype(np.int64)


def make_paged(name, dtype, batch, num_qo_heads, num_kv_heads, head_dim, page_size,
               seed, lens=None, lens_fn=None, n_pages=None, last_page_len=None,
               pool_pages=None, pool_slack=0.0, q_std=1.0, kv_std=1.0, scale=None,
               poison=True, permute=True) -> PagedProblem:
    """Builds a paged problem.

    Lengths come from `lens`, or from lens_fn(rng) drawn on the length stream, or
    as explicit (n_pages, last_page_len).  The pool holds pool_pages pages (or the
    used pages plus pool_slack of them), permuted unless permute=False."""
    ss = np.random.SeedSequence(seed)
    s_len, s_perm, s_q, s_k, s_v = ss.spawn(5)
    if n_pages is None:
        if lens is None:
            lens = lens_fn(np.random.default_rng(s_len))
        lens = np.asarray(lens, dtype=np.int64)
        assert lens.shape == (batch,)
        n_pages, last_page_len = pages_for_lens(lens, page_size)
    n_pages = np.asarray(n_pages, dtype=np.int64)
    last_page_len = np.asarray(last_page_len, dtype=np.int64)
    if lens is None:
        lens = np.where(n_pages > 0, (n_pages - 1) * page_size + last_page_len, 0)
    used = int(n_pages.sum())
    if pool_pages is None:
        pool_pages = max(1, used + int(math.ceil(used * pool_slack)))
    assert pool_pages >= used and pool_pages >= 1
    if permute:
        perm = np.random.default_rng(s_perm).permutation(pool_pages).astype(np.int32)
    else:
        perm = np.arange(pool_pages, dtype=np.int32)
    indices = perm[:used].copy()
    indptr = np.zeros(batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(n_pages)
    if scale is None:
        scale = f32_scale(1.0 / math.sqrt(head_dim))
    tdt = TORCH_DTYPES[dtype]
    qn = np.random.default_rng(s_q).standard_normal((batch, num_qo_heads, head_dim),
                                                    dtype=np.float32)
    if q_std != 1.0:
        qn *= np.float32(q_std)
    q = torch.from_numpy(qn).to(tdt)
    shape = (pool_pages, num_kv_heads, page_size, head_dim)
    k = _draw_pool(s_k, shape, kv_std, dtype)
    v = _draw_pool(s_v, shape, kv_std, dtype)
    if poison:
        referenced = np.zeros(pool_pages, dtype=bool)
        referenced[indices] = True
        unref = torch.from_numpy(np.nonzero(~referenced)[0])
        if unref.numel():
            k[unref] = POISON_PAGE
            v[unref] = POISON_PAGE
        for b in range(batch):
            if n_pages[b] == 0:
                continue
            last = int(indices[indptr[b + 1] - 1])
            r0 = int(last_page_len[b])
            if r0 < page_size:
                k[last, :, r0:, :] = POISON_ROW
                v[last, :, r0:, :] = POISON_ROW
    return PagedProblem(name=name, dtype=dtype, batch=batch, num_qo_heads=num_qo_heads,
                        num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
                        num_total_pages=pool_pages, scale=float(scale), q=q, k_data=k,
                        v_data=v, indices=torch.from_numpy(indices),
                        indptr=torch.from_numpy(indptr),
                        last_page_len=torch.from_numpy(last_page_len.astype(np.int32)),
                        kv_lens=np.asarray(lens, dtype=np.int64))


def make_contig(name, dtype, num_qo_heads, num_kv_heads, head_dim, max_kv_len, valid_kv_len,
                seed, q_std=1.0, kv_std=1.0, scale=None, poison=True) -> ContigProblem:
    ss = np.random.SeedSequence(seed)
    _, _, s_q, s_k, s_v = ss.spawn(5)
    if scale is None:
        scale = f32_scale(1.0 / math.sqrt(head_dim))
    tdt = TORCH_DTYPES[dtype]
    qn = np.random.default_rng(s_q).standard_normal((num_qo_heads, head_dim), dtype=np.float32)
    if q_std != 1.0:
        qn *= np.float32(q_std)
    q = torch.from_numpy(qn).to(tdt)
    # The cache is drawn as a pool of "pages" of one KV row per head, i.e. as
    # [max_kv_len, Hkv, D], and then laid out heads-major [Hkv, max_kv_len, D].
    k = _draw_pool(s_k, (max(max_kv_len, 1), num_kv_heads, head_dim), kv_std, dtype)
    v = _draw_pool(s_v, (max(max_kv_len, 1), num_kv_heads, head_dim), kv_std, dtype)
    k = k[:max_kv_len].permute(1, 0, 2).contiguous()
    v = v[:max_kv_len].permute(1, 0, 2).contiguous()
    if poison and valid_kv_len < max_kv_len:
        k[:, valid_kv_len:, :] = POISON_ROW
        v[:, valid_kv_len:, :] = POISON_ROW
    return ContigProblem(name=name, dtype=dtype, num_qo_heads=num_qo_heads,
                         num_kv_heads=num_kv_heads, head_dim=head_dim, max_kv_len=max_kv_len,
                         valid_kv_len=valid_kv_len, scale=float(scale), q=q, k_cache=k,
                         v_cache=v)


# --------------------------------------------------------------- the configs
#
# c1..c5 are the five synthetic workloads at full size; the *_small variants
# keep each config's dtype, heads, head_dim and page size but shrink batch and
# lengths so the float64 oracle finishes in seconds while still spanning many
# tiles and ragged tails.

def _c5_lens(rng, batch, mu, sigma, hi):
    return np.clip(np.rint(rng.lognormal(mu, sigma, size=batch)), 1, hi).astype(np.int64)


def _c5_tables(lens, page_size):
    """Skew-config edge requests: request 0 keeps its length rounded up to a whole
    number of pages and gets one more, empty page (last_page_len 0); request 1
    has a single row."""
    lens = lens.copy()
    lens[0] = max(page_size, int(math.ceil(lens[0] / page_size)) * page_size)
    lens[1] = 1
    n_pages, lpl = pages_for_lens(lens, page_size)
    n_pages[0] += 1
    lpl[0] = 0
    return n_pages, lpl


# The five configurations.  dtype, if given, stores the same shapes and
# draws in another element type (the name gains a suffix); None keeps the
# configuration's own.
def _named(name, own, dtype):
    return (name, own) if dtype in (None, own) else (f"{name}_as_{dtype}", dtype)


def c1(seed=1001, dtype=None):
    name, dt = _named("c1_contig_f32", "f32", dtype)
    return make_contig(name, dt, 8, 2, 64, 256, 128, seed)


def c2(seed=1002, dtype=None):
    name, dt = _named("c2_contig_f16", "f16", dtype)
    return make_contig(name, dt, 32, 8, 128, 8192, 4096, seed, kv_std=0.5)


def _heads(name, own, qo_heads):
    """qo_heads, if given, replaces the number of query heads (the KV heads and
    every draw of K, V and the page table stay; q is drawn at the new shape)."""
    return (name, own) if qo_heads in (None, own) else (f"{name}_hq{qo_heads}", qo_heads)


def c3(seed=1003, dtype=None, qo_heads=None):
    name, dt = _named("c3_paged_bf16", "bf16", dtype)
    name, hq = _heads(name, 32, qo_heads)
    return make_paged(name, dt, 64, hq, 8, 128, 16, seed,
                      lens_fn=lambda r: r.integers(512, 8192, size=64, endpoint=True),
                      pool_pages=40000)


def c4(seed=1004, dtype=None, qo_heads=None):
    name, dt = _named("c4_paged_bf16_g8", "bf16", dtype)
    name, hq = _heads(name, 64, qo_heads)
    return make_paged(name, dt, 32, hq, 8, 128, 32, seed,
                      lens=np.full(32, 32768), pool_pages=32768)


def c5(seed=1005, dtype=None, qo_heads=None):
    name, dt = _named("c5_paged_f16_skew", "f16", dtype)
    name, hq = _heads(name, 16, qo_heads)
    ss = np.random.SeedSequence(seed)
    lens = _c5_lens(np.random.default_rng(ss.spawn(1)[0]), 128, 7.0, 1.5, 131072)
    n_pages, lpl = _c5_tables(lens, 16)
    return make_paged(name, dt, 128, hq, 4, 256, 16, seed,
                      n_pages=n_pages, last_page_len=lpl, pool_slack=0.25)


def c1_small(seed=2001):
    return make_contig("c1_small", "f32", 8, 2, 64, 256, 128, seed)


def c2_small(seed=2002):
    return make_contig("c2_small", "f16", 32, 8, 128, 1024, 777, seed, kv_std=0.5)


def c3_small(seed=2003):
    return make_paged("c3_small", "bf16", 6, 32, 8, 128, 16, seed,
                      lens_fn=lambda r: r.integers(1, 700, size=6, endpoint=True),
                      pool_pages=400)


def c4_small(seed=2004):
    return make_paged("c4_small", "bf16", 3, 64, 8, 128, 32, seed,
                      lens=np.array([2000, 1025, 33]), pool_slack=0.1)


def c5_small(seed=2005):
    ss = np.random.SeedSequence(seed)
    lens = _c5_lens(np.random.default_rng(ss.spawn(1)[0]), 12, 4.0, 1.5, 3000)
    n_pages, lpl = _c5_tables(lens, 16)
    return make_paged("c5_small", "f16", 12, 16, 4, 256, 16, seed, n_pages=n_pages,
                      last_page_len=lpl, pool_slack=0.25)


FULL = {"c1": c1, "c2": c2, "c3": c3, "c4": c4, "c5": c5}
SMALL = {"c1": c1_small, "c2": c2_small, "c3": c3_small, "c4": c4_small, "c5": c5_small}
