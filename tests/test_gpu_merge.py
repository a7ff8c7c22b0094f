"""The standalone merge of split partials on the GPU (fa_merge_states).

Two kinds of check against the float64 oracle:
  * random partials (o_s ~ N(0, 1), lse_s spread over several units, empty
    parts with lse_s = -inf whose o_s rows hold NaN, rows whose parts are all
    empty), element by element against oracle.merge row by row;
  * context-parallel decode: each request's pages are dealt out in S
    contiguous shares, every share is decoded on its own (fa_decode_paged over
    a page table of that share), and merging the S results must give the
    oracle's decode over the whole problem.
"""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from gpu_util import announce, compare, device, oracle_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _partials(rng, s, rows, d, empty_frac, all_empty_rows):
    o = rng.standard_normal((s, rows, d)).astype(np.float32)
    lse = (rng.standard_normal((s, rows)) * 3.0).astype(np.float32)
    empty = rng.random((s, rows)) < empty_frac
    for r in all_empty_rows:
        empty[:, r] = True
    lse[empty] = -np.inf
    o[empty] = np.nan  # an empty part's output must not reach the result
    return o, lse


def _oracle_rows(o, lse):
    s, rows, d = o.shape
    ro = np.empty((rows, d))
    rl = np.empty(rows)
    for r in range(rows):
        ro[r], rl[r] = oracle.merge(o[:, r, :].astype(np.float64), lse[:, r].astype(np.float64))
    return ro, rl


CASES = [
    # dtype, head_dim, parts, rows, fraction of empty parts
    ("f32", 128, 2, 5, 0.0),
    ("f32", 64, 1, 33, 0.0),
    ("f32", 256, 8, 17, 0.2),
    ("bf16", 128, 3, 257, 0.1),
    ("f16", 256, 9, 63, 0.3),
    ("bf16", 64, 17, 100, 0.5),
    ("f32", 128, 70, 9, 0.25),
    ("f16", 64, 4, 1, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-S{c[2]}-R{c[3]}")
def test_merge_matches_oracle(dev, case):
    dtype, d, s, rows, frac = case
    announce(f"merge {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    all_empty = [rows // 2] if rows > 2 else []
    o_p, l_p = _partials(rng, s, rows, d, frac, all_empty)
    o, lse = fad.merge_states(torch.from_numpy(o_p).to(dev), torch.from_numpy(l_p).to(dev),
                              out_dtype=W.TORCH_DTYPES[dtype])
    torch.cuda.synchronize()
    ro, rl = _oracle_rows(o_p, l_p)
    compare(dtype, o, lse, ro, rl, what=f"merge {case}")
    # run to run: bit-identical
    o2, lse2 = fad.merge_states(torch.from_numpy(o_p).to(dev), torch.from_numpy(l_p).to(dev),
                                out_dtype=W.TORCH_DTYPES[dtype])
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.uint8) if o.dtype != torch.float32 else o.view(torch.int32),
                       o2.view(torch.uint8) if o2.dtype != torch.float32 else o2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def test_merge_without_lse_output(dev):
    announce("merge lse=NULL")
    rng = np.random.default_rng(5)
    o_p, l_p = _partials(rng, 3, 40, 128, 0.2, [7])
    o = torch.empty((40, 128), dtype=torch.float32, device=dev)
    fad.fa_merge_states(fad.FA_DTYPE_F32, 40, 3, 128, torch.from_numpy(o_p).to(dev),
                        torch.from_numpy(l_p).to(dev), o, None)
    torch.cuda.synchronize()
    ro, rl = _oracle_rows(o_p, l_p)
    compare("f32", o, torch.from_numpy(rl.astype(np.float32)), ro, rl, what="merge lse=NULL")


def _share_tables(p, s):
    """Page tables of S shares of every request: request b's n_b pages are cut
    into S contiguous runs; a run that does not end the request ends on a full
    page, the last keeps the request's last_page_len."""
    ind = p.indices.numpy()
    ptr = p.indptr.numpy()
    lpl = p.last_page_len.numpy()
    out = []
    for k in range(s):
        sel, iptr, l = [], [0], []
        for b in range(p.batch):
            n = int(ptr[b + 1] - ptr[b])
            a, e = (k * n) // s, ((k + 1) * n) // s
            sel.append(ind[ptr[b] + a:ptr[b] + e])
            iptr.append(iptr[-1] + (e - a))
            l.append(int(lpl[b]) if e == n and e > a else (p.page_size if e > a else 0))
        out.append((np.concatenate(sel).astype(np.int32), np.array(iptr, dtype=np.int32),
                    np.array(l, dtype=np.int32)))
    return out


@pytest.mark.parametrize("parts", [2, 3, 5])
def test_context_parallel_decode(dev, parts):
    """Shares decoded separately, then merged, equal the decode of the whole."""
    announce(f"context-parallel decode, {parts} shares")
    lens = [0, 1, 16, 100, 777, 2048, 4096, 40]
    n_pages, lpl = W.pages_for_lens(lens, 16)
    n_pages[6] += 1      # one request with an empty trailing page
    lpl[6] = 0
    p = W.make_paged("cp", "f32", len(lens), 16, 4, 128, 16, seed=77, n_pages=n_pages,
                     last_page_len=lpl, pool_slack=0.2)
    q, k, v = p.q.to(dev), p.k_data.to(dev), p.v_data.to(dev)
    o_parts, l_parts = [], []
    for ind, ptr, l in _share_tables(p, parts):
        o, lse = fad.decode_paged(q, k, v, torch.from_numpy(ind).to(dev),
                                  torch.from_numpy(ptr).to(dev), torch.from_numpy(l).to(dev),
                                  p.scale)
        o_parts.append(o)
        l_parts.append(lse)
    o, lse = fad.merge_states(torch.stack(o_parts), torch.stack(l_parts),
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle_of(p)
    compare("f32", o, lse, ro, rl, what=f"context-parallel {parts}")


def test_merge_many_rows(dev):
    """600,000 rows x 2 parts at D = 128: 75,000 workgroups, so the launch and
    the kernel's 64-bit row offsets go well past 16-bit grid sizes; sampled
    rows against the oracle, every row finite."""
    announce("merge 600k rows")
    rows, s_, d = 600_000, 2, 128
    g = torch.Generator(device="cpu").manual_seed(31)
    o_p = torch.randn((s_, rows, d), generator=g).to(dev)
    l_p = (torch.randn((s_, rows), generator=g) * 3.0).to(dev)
    l_p[1, ::5] = -float("inf")
    o, lse = fad.merge_states(o_p, l_p, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    pick = np.unique(np.concatenate([np.arange(4), rows - 1 - np.arange(4),
                                     np.random.default_rng(3).integers(0, rows, 200)]))
    idx = torch.from_numpy(pick).to(dev)
    op = o_p[:, idx, :].cpu().numpy()
    lp = l_p[:, idx].cpu().numpy()
    ro, rl = _oracle_rows(op, lp)
    compare("f32", o[idx], lse[idx], ro, rl, what="merge 600k rows")
    del o_p, l_p, o, lse
    torch.cuda.empty_cache()
