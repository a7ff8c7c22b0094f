"""Sliding window and logits soft-cap on the GPU (fa_decode_paged_opts,
fa_decode_contig_opts) against the oracle's window= / softcap= paths, element
by element with the same tolerances as the plain entry points."""
import math
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from _helpers import rand_t, scatter_paged
from gpu_util import announce, compare, device, sample_pairs, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _oracle(p, window, softcap, samples=None, alibi=None):
    if isinstance(p, W.PagedProblem):
        return oracle.decode_paged(p.dtype, W.bits(p.q), W.bits(p.k_data), W.bits(p.v_data),
                                   p.indices.numpy(), p.indptr.numpy(), p.last_page_len.numpy(),
                                   p.scale, samples=samples, layout=p.layout, window=window,
                                   softcap=softcap, alibi=alibi)
    return oracle.decode_contig(p.dtype, W.bits(p.q), W.bits(p.k_cache), W.bits(p.v_cache),
                                p.valid_kv_len, p.scale, layout=p.layout, window=window,
                                softcap=softcap, alibi=alibi)


def _run(p, d, window, softcap, alibi=None):
    dev_alibi = None
    if alibi is not None:
        dev_alibi = torch.tensor(alibi, dtype=torch.float32, device=d["q"].device)
    if isinstance(p, W.PagedProblem):
        return fad.decode_paged(d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"],
                                p.scale, layout=p.layout, window=window, softcap=softcap,
                                alibi=dev_alibi)
    return fad.decode_contig(d["q"], d["k"], d["v"], p.valid_kv_len, p.scale, layout=p.layout,
                             window=window, softcap=softcap, alibi=dev_alibi)


def alibi_slopes(hq, max_bias=8.0):
    """The usual geometric ALiBi slopes 2^(-max_bias (h + 1) / Hq), rounded to f32."""
    return [float(np.float32(2.0 ** (-max_bias * (h + 1) / hq))) for h in range(hq)]


CASES = [
    # dtype, head_dim, num_kv_heads, group, page_size, lens
    ("bf16", 128, 2, 4, 16, [0, 1, 15, 16, 17, 300, 5000]),
    ("f16", 64, 2, 3, 7, [1, 49, 260, 700]),
    ("f32", 64, 2, 4, 16, [2, 33, 513]),
    ("f16", 256, 1, 8, 32, [1023, 1025, 64]),
    ("bf16", 128, 1, 16, 1, [40, 3]),
]
VARIANTS = [(1, 0.0, False), (5, 0.0, False), (16, 0.0, False), (17, 0.0, False),
            (257, 0.0, False), (0, 1.0, False), (0, 30.0, False), (100, 5.0, False),
            (0, 0.0, True), (33, 0.0, True), (0, 20.0, True)]


@pytest.mark.parametrize("variant", VARIANTS,
                         ids=lambda v: f"w{v[0]}-cap{v[1]:g}" + ("-alibi" if v[2] else ""))
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-P{c[4]}")
def test_paged_variants(dev, case, variant):
    dtype, d, hkv, group, page_size, lens = case
    window, cap, with_alibi = variant
    slopes = alibi_slopes(hkv * group) if with_alibi else None
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    kd, ind, ptr, lpl = scatter_paged(k_rows, page_size, np.random.default_rng(3), 3, (),
                                      fill=1.0e4)
    vd, _, _, _ = scatter_paged(v_rows, page_size, np.random.default_rng(3), 3, (), fill=1.0e4)
    # a larger q so that the cap binds
    q = rand_t(rng, (len(lens), hkv * group, d), dtype, std=4.0)
    p = W.PagedProblem(name="variant", dtype=dtype, batch=len(lens), num_qo_heads=hkv * group,
                       num_kv_heads=hkv, head_dim=d, page_size=page_size,
                       num_total_pages=kd.shape[0], scale=float(np.float32(1 / math.sqrt(d))),
                       q=q, k_data=kd, v_data=vd, indices=torch.from_numpy(ind),
                       indptr=torch.from_numpy(ptr), last_page_len=torch.from_numpy(lpl))
    for layout in ("hnd", "nhd"):
        pp = p if layout == "hnd" else W.token_major(p)
        o, lse = _run(pp, to_dev(pp, dev), window, cap, slopes)
        torch.cuda.synchronize()
        ro, rl = _oracle(pp, window, cap, alibi=slopes)
        compare(dtype, o, lse, ro, rl, f"{case} {variant} {layout}")


@pytest.mark.parametrize("variant", [(1, 0.0, False), (100, 0.0, False), (4000, 0.0, False),
                                     (0, 20.0, False), (64, 10.0, False), (0, 0.0, True),
                                     (300, 5.0, True)],
                         ids=lambda v: f"w{v[0]}-cap{v[1]:g}" + ("-alibi" if v[2] else ""))
def test_contig_variants(dev, variant):
    window, cap, with_alibi = variant
    slopes = alibi_slopes(16) if with_alibi else None
    p = W.make_contig("variant", "f16", 16, 4, 128, 5000, 4999, seed=77, q_std=4.0)
    o, lse = _run(p, to_dev(p, dev), window, cap, slopes)
    torch.cuda.synchronize()
    ro, rl = _oracle(p, window, cap, alibi=slopes)
    compare("f16", o, lse, ro, rl, f"contig {variant}")


def test_variants_full_c3(dev):
    """The full C3 workload with a 1000-row window and a soft-cap of 30,
    sampled against the oracle; no window and a cap far beyond every score
    match the plain call within the tolerance."""
    p = W.FULL["c3"]()
    announce("variants full c3")
    d = to_dev(p, dev)
    o, lse = _run(p, d, 1000, 30.0)
    torch.cuda.synchronize()
    pairs = sample_pairs(p, 64, np.random.default_rng(8))
    ro, rl = _oracle(p, 1000, 30.0, samples=pairs)
    idx = (torch.from_numpy(pairs[:, 0].astype(np.int64)),
           torch.from_numpy(pairs[:, 1].astype(np.int64)))
    compare(p.dtype, o.cpu()[idx], lse.cpu()[idx], ro, rl, "c3 w1000 cap30", strict=True)
    o0, l0 = _run(p, d, 0, 0.0)
    o1, l1 = _run(p, d, 0, 1.0e6)
    torch.cuda.synchronize()
    assert torch.allclose(o1.float(), o0.float(), atol=4e-3, rtol=0)
    assert torch.allclose(l1, l0, atol=1e-4, rtol=0)
