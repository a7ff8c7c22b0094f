"""Seeded random problems on the GPU against the oracle.

Each case draws an element type, head dim, KV head count, group size (up to
32, so some groups span several 16-head workgroups), page size, a batch whose
lengths mix empty, one-row, short, split-boundary (multiples of 128 and their
neighbours) and long requests, sometimes empty trailing pages, a K/V layout,
and, at random, a sliding window, a soft-cap, ALiBi slopes and a custom mask.
The outputs are compared element by element with the float64 oracle under the
same tolerances as every other parity test.  The point is coverage of
combinations that no hand-picked case names; each case prints its draw before
it runs, so a failure names its problem.
"""
import math

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import contig_from_rows, rand_t, scatter_paged
from gpu_util import announce, compare, device, to_dev
from test_gpu_variants import _oracle, _run, alibi_slopes

pytestmark = pytest.mark.gpu

N_PAGED = 40
N_CONTIG = 16
MAX_ELEMS = 12_000_000    # K (and V) elements generated per case
MAX_WORK = 150_000_000    # rows x query heads x head dim the oracle evaluates


@pytest.fixture(scope="module")
def dev():
    return device()


def _length(rng, page_size):
    kind = rng.choice(["empty", "one", "short", "edge", "mid", "long", "pages"],
                      p=[0.06, 0.06, 0.18, 0.2, 0.25, 0.15, 0.1])
    if kind == "empty":
        return 0
    if kind == "one":
        return 1
    if kind == "short":
        return int(rng.integers(2, 65))
    if kind == "edge":  # around the split quantum
        return max(0, 128 * int(rng.integers(1, 40)) + int(rng.integers(-1, 2)))
    if kind == "mid":
        return int(rng.integers(65, 3000))
    if kind == "long":
        return int(rng.integers(3000, 20000))
    return page_size * int(rng.integers(1, 60))  # whole pages


def _draw(rng):
    c = dict(dtype=str(rng.choice(["f32", "f16", "bf16"])),
             d=int(rng.choice([64, 128, 256])),
             hkv=int(rng.choice([1, 2, 3, 4, 8])),
             group=int(rng.choice([1, 2, 3, 4, 5, 6, 8, 16, 20, 32])),
             page_size=int(rng.choice([1, 2, 5, 16, 32, 48, 64, 128, 256])),
             layout=str(rng.choice(["hnd", "nhd"])),
             window=int(rng.integers(1, 3000)) if rng.random() < 0.25 else 0,
             softcap=float(rng.uniform(5.0, 50.0)) if rng.random() < 0.2 else 0.0,
             alibi=bool(rng.random() < 0.2),
             mask=(float(rng.choice([0.2, 0.5, 0.9])), bool(rng.random() < 0.5))
             if rng.random() < 0.25 else None)
    if c["hkv"] * c["group"] > 64:
        c["group"] = max(1, 64 // c["hkv"])
    batch = int(rng.integers(1, 13))
    lens = [_length(rng, c["page_size"]) for _ in range(batch)]
    # keep the case small enough for the oracle and the generator
    while (sum(lens) * c["hkv"] * c["d"] > MAX_ELEMS
           or sum(lens) * c["hkv"] * c["group"] * c["d"] > MAX_WORK):
        i = int(np.argmax(lens))
        lens[i] //= 2
    c["lens"] = lens
    c["empty_last"] = tuple(b for b, L in enumerate(lens)
                            if L > 0 and L % c["page_size"] == 0 and rng.random() < 0.3)
    return c


def _mask_for(c, lens, seed):
    if c["mask"] is None:
        return None
    keep, blocks = c["mask"]
    return W.pack_mask(W.random_mask(seed, lens, keep=keep, blocks=blocks))


@pytest.mark.parametrize("case", range(N_PAGED))
def test_random_paged(dev, case):
    rng = np.random.default_rng(7000 + case)
    c = _draw(rng)
    announce(f"random paged {case}: {c}")
    dtype, d, hkv, lens = c["dtype"], c["d"], c["hkv"], c["lens"]
    hq = hkv * c["group"]
    k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    pool_seed, extra = int(rng.integers(1 << 31)), int(rng.integers(0, 5))
    kd, ind, ptr, lpl = scatter_paged(k_rows, c["page_size"], np.random.default_rng(pool_seed),
                                      extra, c["empty_last"], fill=1.0e4, layout=c["layout"])
    vd, ind_v, _, _ = scatter_paged(v_rows, c["page_size"], np.random.default_rng(pool_seed),
                                    extra, c["empty_last"], fill=1.0e4, layout=c["layout"])
    assert np.array_equal(ind, ind_v)
    q = rand_t(rng, (len(lens), hq, d), dtype)
    p = W.PagedProblem(name="random", dtype=dtype, batch=len(lens), num_qo_heads=hq,
                       num_kv_heads=hkv, head_dim=d, page_size=c["page_size"],
                       num_total_pages=kd.shape[0], scale=float(np.float32(1 / math.sqrt(d))),
                       q=q, k_data=kd, v_data=vd, indices=torch.from_numpy(ind),
                       indptr=torch.from_numpy(ptr), last_page_len=torch.from_numpy(lpl),
                       layout=c["layout"])
    slopes = alibi_slopes(hq) if c["alibi"] else None
    mask = _mask_for(c, lens, 8000 + case)
    o, lse = _run(p, to_dev(p, dev), c["window"], c["softcap"], slopes, mask=mask)
    torch.cuda.synchronize()
    ro, rl = _oracle(p, c["window"], c["softcap"], alibi=slopes, mask=mask)
    compare(dtype, o, lse, ro, rl, f"random paged {case}")


@pytest.mark.parametrize("case", range(N_CONTIG))
def test_random_contig(dev, case):
    rng = np.random.default_rng(9000 + case)
    c = _draw(rng)
    valid = c["lens"][0]
    max_len = valid + int(rng.integers(0, 300))
    if max_len == 0:
        max_len = 1
    announce(f"random contig {case}: valid {valid}, max {max_len}, {c}")
    dtype, d, hkv = c["dtype"], c["d"], c["hkv"]
    hq = hkv * c["group"]
    rows_k = rand_t(rng, (valid, hkv, d), dtype)
    rows_v = rand_t(rng, (valid, hkv, d), dtype)
    p = W.ContigProblem(name="random", dtype=dtype, num_qo_heads=hq, num_kv_heads=hkv,
                        head_dim=d, max_kv_len=max_len, valid_kv_len=valid,
                        scale=float(np.float32(1 / math.sqrt(d))),
                        q=rand_t(rng, (hq, d), dtype),
                        k_cache=contig_from_rows(rows_k, max_len, layout=c["layout"]),
                        v_cache=contig_from_rows(rows_v, max_len, layout=c["layout"]),
                        layout=c["layout"])
    slopes = alibi_slopes(hq) if c["alibi"] else None
    mask = _mask_for(c, [valid], 10000 + case)
    o, lse = _run(p, to_dev(p, dev), c["window"], c["softcap"], slopes, mask=mask)
    torch.cuda.synchronize()
    ro, rl = _oracle(p, c["window"], c["softcap"], alibi=slopes, mask=mask)
    compare(dtype, o, lse, ro, rl, f"random contig {case}")
