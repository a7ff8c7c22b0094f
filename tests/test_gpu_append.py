"""Decode-time paged KV append on the GPU (fa_append_paged, fa_append_paged_nhd),
bit-exact against the oracle's append over the whole pool, then decode over
the appended store against the oracle."""
import math
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from _helpers import rand_t, scatter_paged
from gpu_util import announce, compare, device, oracle_of, run, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


CASES = [
    # dtype, head_dim, num_kv_heads, page_size, lens, empty_last_page
    ("bf16", 128, 8, 16, [1, 0, 16, 17, 300, 4096], (2,)),
    ("f16", 256, 4, 16, [0, 5, 1024, 33], ()),
    ("f32", 64, 2, 7, [1, 2, 49, 50], ()),
    ("bf16", 64, 1, 1, [3, 1, 0], ()),
    ("f16", 128, 2, 32, [64, 65, 31], (0,)),
]


def _store(case, layout, rng):
    dtype, d, hkv, page_size, lens, empty = case
    rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    seed = int(rng.integers(1 << 30))
    pool, ind, ptr, lpl = scatter_paged(rows, page_size, np.random.default_rng(seed), 5, empty,
                                        fill=1.0e4, layout=layout)
    new = rand_t(rng, (len(lens), hkv, d), dtype)
    return pool, ind, ptr, lpl, new


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-H{c[2]}-P{c[3]}")
def test_append_bit_exact(dev, case, layout):
    announce(f"append {layout} {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    kp, ind, ptr, lpl, k_new = _store(case, layout, rng)
    vp, _, _, _, v_new = _store(case, layout, np.random.default_rng(7))
    dk, dv = kp.to(dev), vp.to(dev)
    fad.append_paged(k_new.to(dev), v_new.to(dev), dk, dv, torch.from_numpy(ind).to(dev),
                     torch.from_numpy(ptr).to(dev), torch.from_numpy(lpl).to(dev), layout=layout)
    torch.cuda.synchronize()
    dtype = case[0]
    for got, pool, new in ((dk, kp, k_new), (dv, vp, v_new)):
        want = oracle.append_paged(dtype, W.bits(pool), ind, ptr, lpl, W.bits(new), layout=layout)
        assert np.array_equal(W.bits(got.cpu()).view(np.uint8), want.view(np.uint8)), layout


def test_append_then_decode_c3_small(dev):
    """A decode step: append the new token's K/V, then decode over the store."""
    p = W.SMALL["c3"]()
    rng = np.random.default_rng(11)
    k_new = rand_t(rng, (p.batch, p.num_kv_heads, p.head_dim), p.dtype)
    v_new = rand_t(rng, (p.batch, p.num_kv_heads, p.head_dim), p.dtype)
    d = to_dev(p, dev)
    fad.append_paged(k_new.to(dev), v_new.to(dev), d["k"], d["v"], d["indices"], d["indptr"],
                     d["lpl"])
    o, lse = run(p, d)
    torch.cuda.synchronize()
    args = (p.indices.numpy(), p.indptr.numpy(), p.last_page_len.numpy())
    k2 = oracle.append_paged(p.dtype, W.bits(p.k_data), *args, W.bits(k_new))
    v2 = oracle.append_paged(p.dtype, W.bits(p.v_data), *args, W.bits(v_new))
    ro, rl = oracle.decode_paged(p.dtype, W.bits(p.q), k2, v2, *args, p.scale)
    compare(p.dtype, o, lse, ro, rl, "append+decode")


def test_append_full_c3(dev):
    """The full C3 store: one append for all 64 requests, bit-exact."""
    p = W.FULL["c3"]()
    announce("append full c3")
    rng = np.random.default_rng(12)
    k_new = rand_t(rng, (p.batch, p.num_kv_heads, p.head_dim), p.dtype)
    dk = p.k_data.to(dev)
    dv = p.v_data.to(dev)
    fad.append_paged(k_new.to(dev), k_new.to(dev), dk, dv, p.indices.to(dev), p.indptr.to(dev),
                     p.last_page_len.to(dev))
    torch.cuda.synchronize()
    want = oracle.append_paged(p.dtype, W.bits(p.k_data), p.indices.numpy(), p.indptr.numpy(),
                               p.last_page_len.numpy(), W.bits(k_new))
    assert np.array_equal(W.bits(dk.cpu()).view(np.uint8), want.view(np.uint8))
    del dk, dv
    torch.cuda.empty_cache()


def test_append_rejects_bad_shapes(dev):
    k = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device=dev)
    pool = torch.zeros((4, 2, 16, 128), dtype=torch.bfloat16, device=dev)
    ind = torch.zeros(2, dtype=torch.int32, device=dev)
    ptr = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev)
    lpl = torch.ones(2, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        fad.append_paged(k[:1], k, pool, pool, ind, ptr, lpl)
    with pytest.raises(ValueError):
        fad.fa_append_paged(fad.FA_DTYPE_BF16, 2, 2, 128, 16, 4, 2, k, k, ind, ptr, lpl[:1],
                            pool, pool)
