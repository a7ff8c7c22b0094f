"""Token-major K/V layouts on the GPU: fa_decode_contig_nhd ([max_kv_len, Hkv, D],
the ferrox-cuda gqa_decode layout) and fa_decode_paged_nhd ([pages, P, Hkv, D]).

Each case is checked against the oracle's token-major path element by element
(same tolerances as the heads-major tests), and against the heads-major entry
point on the same logical rows, which must give bit-identical outputs: the two
layouts change addresses only, never the order of the arithmetic.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from _helpers import rand_t, scatter_paged
from gpu_util import announce, compare, compare_all, device, oracle_of, run, to_dev
from test_gpu_parity import CONTIG_EDGE, EDGE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _both(p, dev):
    """(o, lse) of p as given (heads-major) and of its token-major copy."""
    pn = W.token_major(p)
    o, lse = run(p, to_dev(p, dev))
    on, ln = run(pn, to_dev(pn, dev))
    torch.cuda.synchronize()
    return pn, (o, lse), (on, ln)


def _assert_same(a, b, what):
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), \
        f"{what}: token-major outputs differ from heads-major"


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_token_major_small_configs(dev, name):
    p = W.SMALL[name]()
    announce(f"token-major small {name}")
    pn, hnd, nhd = _both(p, dev)
    ro, rl = oracle_of(pn)
    compare(p.dtype, nhd[0], nhd[1], ro, rl, pn.name)
    _assert_same(hnd, nhd, pn.name)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-P{c[4]}")
def test_token_major_paged_edge_cases(dev, case):
    dtype, d, hkv, group, page_size, lens, empty = case
    announce(f"token-major edge paged {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()) ^ 0x5A5A)
    k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    kd, ind, ptr, lpl = scatter_paged(k_rows, page_size, np.random.default_rng(2), 3, empty,
                                      fill=1.0e4)
    vd, _, _, _ = scatter_paged(v_rows, page_size, np.random.default_rng(2), 3, empty,
                                fill=1.0e4)
    q = rand_t(rng, (len(lens), hkv * group, d), dtype)
    p = W.PagedProblem(name="edge", dtype=dtype, batch=len(lens), num_qo_heads=hkv * group,
                       num_kv_heads=hkv, head_dim=d, page_size=page_size,
                       num_total_pages=kd.shape[0], scale=float(np.float32(1 / math.sqrt(d))),
                       q=q, k_data=kd, v_data=vd, indices=torch.from_numpy(ind),
                       indptr=torch.from_numpy(ptr), last_page_len=torch.from_numpy(lpl))
    pn, hnd, nhd = _both(p, dev)
    ro, rl = oracle_of(pn)
    compare(dtype, nhd[0], nhd[1], ro, rl, str(case))
    _assert_same(hnd, nhd, str(case))


@pytest.mark.parametrize("case", CONTIG_EDGE, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-L{c[5]}")
def test_token_major_contig_edge_cases(dev, case):
    dtype, d, hkv, group, max_len, valid = case
    announce(f"token-major edge contig {case}")
    p = W.make_contig("edge", dtype, hkv * group, hkv, d, max_len, valid,
                      seed=zlib.crc32(str(case).encode()) ^ 0x5A5A)
    pn, hnd, nhd = _both(p, dev)
    ro, rl = oracle_of(pn)
    compare(dtype, nhd[0], nhd[1], ro, rl, str(case))
    _assert_same(hnd, nhd, str(case))


def test_token_major_gather_bit_exact(dev):
    for name in ("c3", "c4", "c5"):
        p = W.token_major(W.SMALL[name]())
        announce(f"token-major gather {p.name}")
        total = int(oracle.seq_lens(p.page_size, p.indptr.numpy(),
                                    p.last_page_len.numpy()).sum())
        ws = fad.workspace_paged(p.batch, p.num_kv_heads, p.num_kv_heads, p.head_dim,
                                 p.page_size, p.total_used_pages, dev)
        for which, data in (("k", p.k_data), ("v", p.v_data)):
            out = torch.zeros((total, p.num_kv_heads, p.head_dim), dtype=data.dtype, device=dev)
            fad.fa_debug_gather_paged(fad.DTYPE_CODES[p.dtype], p.batch, p.num_kv_heads,
                                      p.head_dim, p.page_size, p.num_total_pages,
                                      p.total_used_pages, data.to(dev), p.indices.to(dev),
                                      p.indptr.to(dev), p.last_page_len.to(dev), out, total, ws,
                                      layout="nhd")
            torch.cuda.synchronize()
            want = oracle.gather_paged(p.dtype, W.bits(data), p.indices.numpy(),
                                       p.indptr.numpy(), p.last_page_len.numpy(), layout="nhd")
            got = W.bits(out.cpu())
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (p.name, which)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_token_major_full(dev, name):
    """The full workloads stored token-major, in the benchmark's launch
    configuration: bit-identical to heads-major, and every output against the
    oracle's token-major path."""
    p = W.FULL[name]()
    announce(f"token-major full {name}")
    pn, hnd, nhd = _both(p, dev)
    _assert_same(hnd, nhd, pn.name)
    eo, el = compare_all(pn, nhd[0], nhd[1])
    announce(f"  every output: max|do|={eo:.2e} max|dlse|={el:.2e}")
    del hnd, nhd
    torch.cuda.empty_cache()