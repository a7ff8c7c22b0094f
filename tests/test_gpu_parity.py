"""Parity of the HIP decode library with the float64 oracle, on the GPU.

Every call goes through the C ABI (libfadecode.so via the ctypes binding).
Tolerances: o within 1e-5 (f32) or 4e-3 (f16, bf16) absolute, lse within 1e-4
absolute, empty requests exactly o = 0 and lse = -inf, the page-table gather
bit-exact.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from _helpers import contig_from_rows, rand_t, scatter_paged
from gpu_util import (announce, check_gather, compare, compare_all, device, oracle_of, run,
                      to_dev)

pytestmark = pytest.mark.gpu

_FULL = {}


def full(name):
    if name not in _FULL:
        announce(f"generating full workload {name}")
        _FULL[name] = W.FULL[name]()
    return _FULL[name]


@pytest.fixture(scope="module")
def dev():
    return device()


# ------------------------------------------------------------------ configs

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_small_config_parity(dev, name):
    p = W.SMALL[name]()
    announce(f"small {name}: {p.name}")
    d = to_dev(p, dev)
    o, lse = run(p, d)
    torch.cuda.synchronize()
    ro, rl = oracle_of(p)
    eo, el = compare(p.dtype, o, lse, ro, rl, p.name)
    announce(f"  max|do|={eo:.2e} max|dlse|={el:.2e}")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_full_config_parity(dev, name):
    """Full-size workloads in the benchmark's launch configuration: every
    (request, head) output against the oracle's whole call, at the stated
    tolerances alone (no ulp allowance)."""
    p = full(name)
    announce(f"full {name}: {p.name}")
    d = to_dev(p, dev)
    o, lse = run(p, d)
    eo, el = compare_all(p, o, lse)
    announce(f"  every output: max|do|={eo:.2e} max|dlse|={el:.2e}")
    del d, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,dtype", [("c3", "f32"), ("c2", "f32"), ("c3", "f16"),
                                        ("c4", "f16"), ("c5", "bf16")])
def test_full_shapes_other_dtype(dev, name, dtype):
    """Full-size shapes stored in another element type (f32 runs the matrix-core
    kernel with k = 4 products at these head dims): every output against the
    oracle at that type's tolerance."""
    p = W.FULL[name](dtype=dtype)
    announce(f"full {name} as {dtype}: {p.name}")
    d = to_dev(p, dev)
    o, lse = run(p, d)
    eo, el = compare_all(p, o, lse)
    announce(f"  every output: max|do|={eo:.2e} max|dlse|={el:.2e}")
    del d, o, lse
    torch.cuda.empty_cache()


# --------------------------------------------------------------- edge cases

EDGE = [
    # dtype, head_dim, num_kv_heads, group, page_size, lens, empty_last_page
    ("f32", 64, 2, 4, 16, [0, 1, 15, 16, 17, 300], ()),
    ("f16", 128, 2, 1, 1, [1, 2, 257, 513], ()),
    ("bf16", 256, 1, 2, 3, [5, 256, 257, 700], ()),
    ("bf16", 128, 1, 8, 32, [1023, 1024, 1025], ()),
    ("f16", 64, 2, 3, 7, [0, 49, 260], ()),
    ("bf16", 128, 1, 16, 16, [300, 1], ()),
    ("f32", 256, 1, 6, 5, [33, 512], ()),
    ("bf16", 128, 2, 4, 16, [32, 0, 48, 3], (0, 1)),
    ("f16", 128, 2, 4, 1024, [1000, 5], ()),
    ("bf16", 64, 4, 4, 16, [0, 0, 0], ()),
    ("f32", 128, 3, 5, 8, [64, 129, 2], ()),
    ("f16", 256, 2, 8, 64, [4096, 64, 65], ()),
    # groups wider than one 16-head block: a KV head's query heads span workgroups
    ("bf16", 128, 1, 32, 16, [700, 1, 3000], ()),
    ("f16", 64, 2, 24, 16, [0, 100, 2500], ()),
    ("f32", 128, 1, 64, 32, [513, 40], ()),
    ("f16", 256, 1, 17, 16, [300, 2], ()),
    # an even number of 16-head blocks: two blocks per workgroup share each
    # K/V tile (G = 32: one workgroup per KV head and unit; G = 64: two)
    ("f16", 256, 2, 32, 16, [0, 1, 31, 33, 2049], ()),
    ("bf16", 64, 3, 32, 8, [7, 96, 1500], ()),
    ("f32", 64, 1, 32, 16, [100, 16, 1], ()),
    ("f32", 256, 1, 32, 5, [77, 3000], ()),
    ("bf16", 128, 2, 64, 16, [5000, 16, 0], (1,)),
    ("f16", 128, 1, 96, 32, [31, 640], ()),
    # groups that are not powers of two: one block of the whole group up to
    # 16 heads, else blocks of 16 with a shorter last one (G = 48: the last
    # workgroup's second block is empty; G = 71: 16 + 16 | 16 + 16 | 7)
    ("bf16", 128, 4, 7, 16, [0, 1, 700, 2500], ()),
    ("f16", 64, 2, 6, 8, [33, 900], ()),
    ("f32", 256, 1, 13, 16, [17, 1300], ()),
    ("bf16", 128, 1, 48, 16, [600, 2, 3100], ()),
    ("f16", 128, 1, 71, 16, [1, 1030], ()),
    ("bf16", 64, 2, 24, 32, [2048, 5], (0,)),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-P{c[4]}")
def test_paged_edge_cases(dev, case):
    dtype, d, hkv, group, page_size, lens, empty = case
    announce(f"edge paged {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    kd, ind, ptr, lpl = scatter_paged(k_rows, page_size, np.random.default_rng(1), 3, empty,
                                      fill=1.0e4)
    vd, _, _, _ = scatter_paged(v_rows, page_size, np.random.default_rng(1), 3, empty,
                                fill=1.0e4)
    q = rand_t(rng, (len(lens), hkv * group, d), dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    p = W.PagedProblem(name="edge", dtype=dtype, batch=len(lens), num_qo_heads=hkv * group,
                       num_kv_heads=hkv, head_dim=d, page_size=page_size,
                       num_total_pages=kd.shape[0], scale=scale, q=q, k_data=kd, v_data=vd,
                       indices=torch.from_numpy(ind), indptr=torch.from_numpy(ptr),
                       last_page_len=torch.from_numpy(lpl))
    o, lse = run(p, to_dev(p, dev))
    torch.cuda.synchronize()
    ro, rl = oracle_of(p)
    compare(dtype, o, lse, ro, rl, str(case))


CONTIG_EDGE = [
    ("f32", 64, 2, 4, 256, 0),
    ("f32", 64, 2, 4, 256, 1),
    ("f16", 128, 8, 4, 300, 300),
    ("bf16", 256, 1, 8, 1000, 257),
    ("bf16", 128, 4, 2, 5000, 4999),
    ("f16", 64, 1, 1, 64, 63),
    ("f32", 128, 2, 3, 700, 513),
    ("bf16", 128, 1, 32, 4096, 4000),
    ("f32", 64, 1, 20, 300, 299),
    ("f16", 256, 2, 64, 2000, 1999),
    ("f32", 64, 1, 32, 100, 0),
    ("bf16", 128, 4, 7, 4096, 4096),
    ("f16", 256, 1, 40, 700, 699),
]


@pytest.mark.parametrize("case", CONTIG_EDGE, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-L{c[5]}")
def test_contig_edge_cases(dev, case):
    dtype, d, hkv, group, max_len, valid = case
    announce(f"edge contig {case}")
    p = W.make_contig("edge", dtype, hkv * group, hkv, d, max_len, valid,
                      seed=zlib.crc32(str(case).encode()))
    o, lse = run(p, to_dev(p, dev))
    torch.cuda.synchronize()
    ro, rl = oracle_of(p)
    compare(dtype, o, lse, ro, rl, str(case))


def test_worked_example(dev):
    """The ferrox-cuda page's hardware test (every q 0.01, k 0.02, v 0.03,
    three rows), widened to head_dim 64: o is the V row, lse = score + ln 3."""
    hq, hkv, d, L = 4, 2, 64, 3
    qv, kv, vv = np.float32(0.01), np.float32(0.02), np.float32(0.03)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q = torch.full((hq, d), float(qv), device=dev)
    k = torch.full((hkv, L, d), float(kv), device=dev)
    v = torch.full((hkv, L, d), float(vv), device=dev)
    o, lse = fad.decode_contig(q, k, v, L, scale)
    torch.cuda.synchronize()
    assert np.allclose(o.cpu().numpy(), float(vv), rtol=0, atol=1e-7)
    want = d * float(qv) * float(kv) * scale + math.log(3.0)
    assert np.allclose(lse.cpu().numpy(), want, rtol=0, atol=1e-5)


# ------------------------------------------------------------ invariants

def test_gather_bit_exact_small(dev):
    for name in ("c3", "c4", "c5"):
        p = W.SMALL[name]()
        announce(f"gather {p.name}")
        check_gather(p, dev)


def test_deterministic_full_c3(dev):
    p = full("c3")
    d = to_dev(p, dev)
    o1, l1 = run(p, d)
    o2, l2 = run(p, d)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_page_permutation_bit_identical(dev):
    """Moving pages to other physical slots (same logical rows, rewritten
    indices) leaves every output bit unchanged."""
    p = W.SMALL["c3"]()
    o1, l1 = run(p, to_dev(p, dev))
    perm = torch.from_numpy(np.random.default_rng(3).permutation(p.num_total_pages))
    inv = torch.argsort(perm)
    # new slot perm[i] holds old page i
    k2 = torch.empty_like(p.k_data)
    v2 = torch.empty_like(p.v_data)
    k2[perm] = p.k_data
    v2[perm] = p.v_data
    p2 = W.PagedProblem(**{**p.__dict__, "k_data": k2, "v_data": v2,
                           "indices": perm[p.indices.long()].to(torch.int32)})
    o2, l2 = run(p2, to_dev(p2, dev))
    torch.cuda.synchronize()
    del inv
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_poison_does_not_leak(dev):
    """Excluded rows and unreferenced pages never change an output bit."""
    p = W.SMALL["c5"]()
    o1, l1 = run(p, to_dev(p, dev))
    used = torch.zeros(p.num_total_pages, dtype=torch.bool)
    used[p.indices.long()] = True
    for poison in (float("nan"), -3.0e4, 6.0e4):
        k2, v2 = p.k_data.clone(), p.v_data.clone()
        k2[~used] = poison
        v2[~used] = poison
        for b in range(p.batch):
            n = int(p.indptr[b + 1] - p.indptr[b])
            if n == 0:
                continue
            last = int(p.indices[p.indptr[b + 1] - 1])
            r0 = int(p.last_page_len[b])
            k2[last, :, r0:, :] = poison
            v2[last, :, r0:, :] = poison
        p2 = W.PagedProblem(**{**p.__dict__, "k_data": k2, "v_data": v2})
        o2, l2 = run(p2, to_dev(p2, dev))
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), poison
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), poison


def test_contig_matches_paged(dev):
    """The same logical rows in a contiguous cache and in pages agree (within
    tolerance: the two layouts may split the rows differently)."""
    rng = np.random.default_rng(9)
    for dtype in ("f32", "f16", "bf16"):
        hkv, group, d, L = 4, 4, 128, 3000
        q = rand_t(rng, (hkv * group, d), dtype)
        rows_k, rows_v = rand_t(rng, (L, hkv, d), dtype), rand_t(rng, (L, hkv, d), dtype)
        kc = contig_from_rows(rows_k, 4096).to(dev)
        vc = contig_from_rows(rows_v, 4096).to(dev)
        oc, lc = fad.decode_contig(q.to(dev), kc, vc, L, 0.0884)
        kd, ind, ptr, lpl = scatter_paged([rows_k], 16, np.random.default_rng(2), 5)
        vd, _, _, _ = scatter_paged([rows_v], 16, np.random.default_rng(2), 5)
        op, lp = fad.decode_paged(q[None].to(dev), kd.to(dev), vd.to(dev),
                                  torch.from_numpy(ind).to(dev), torch.from_numpy(ptr).to(dev),
                                  torch.from_numpy(lpl).to(dev), 0.0884)
        torch.cuda.synchronize()
        tol = 1e-5 if dtype == "f32" else 4e-3
        assert (oc.float() - op[0].float()).abs().max().item() <= tol
        assert (lc - lp[0]).abs().max().item() <= 1e-4


def test_side_stream(dev):
    """A call on a non-default stream gives the same bits as on the default one."""
    p = W.SMALL["c4"]()
    d = to_dev(p, dev)
    o1, l1 = run(p, d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o2, l2 = run(p, d)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_binding_checks_shapes(dev):
    """Host checks refuse operands smaller than the dimensions passed."""
    p = W.SMALL["c3"]()
    d = to_dev(p, dev)
    o = torch.empty_like(d["q"])
    lse = torch.empty((p.batch, p.num_qo_heads), dtype=torch.float32, device=dev)
    ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim, p.page_size,
                             p.total_used_pages, dev)
    with pytest.raises(ValueError):
        fad.fa_decode_paged(fad.FA_DTYPE_BF16, p.batch + 1, p.num_qo_heads, p.num_kv_heads,
                            p.head_dim, p.page_size, p.num_total_pages, p.total_used_pages,
                            p.scale, d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"],
                            o, lse, ws)
    with pytest.raises(fad.FaError):
        fad.fa_decode_paged(fad.FA_DTYPE_BF16, p.batch, p.num_qo_heads, p.num_kv_heads,
                            p.head_dim, p.page_size, p.num_total_pages, p.total_used_pages,
                            p.scale, d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"],
                            o, lse, ws[:16])


@pytest.mark.parametrize("name,qo_heads", [("c3", 8), ("c3", 16), ("c3", 56), ("c3", 128),
                                            ("c3", 192), ("c3", 256), ("c3", 384), ("c5", 4)])
def test_full_shapes_other_group(dev, name, qo_heads):
    """Full-size K/V and page tables with another number of query heads per KV
    head (G = 1, 2, 7, 16, 24, 32 and 48 on C3's store, G = 1 on C5's), as
    bench.py --qo-heads times them: every output against the oracle."""
    p = W.FULL[name](qo_heads=qo_heads)
    announce(f"full {name} with {qo_heads} query heads: {p.name}")
    d = to_dev(p, dev)
    o, lse = run(p, d)
    eo, el = compare_all(p, o, lse)
    announce(f"  every output: max|do|={eo:.2e} max|dlse|={el:.2e}")
    del d, o, lse
    torch.cuda.empty_cache()
