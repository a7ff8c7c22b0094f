"""Sliding window, logits soft-cap, ALiBi and the custom mask on the GPU
(fa_decode_paged_opts, fa_decode_contig_opts) against the oracle's window= /
softcap= / alibi= / mask= paths, element by element with the same tolerances
as the plain entry points."""
import math
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from _helpers import rand_t, scatter_paged
from gpu_util import announce, compare, compare_all, device, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _oracle(p, window, softcap, samples=None, alibi=None, mask=None):
    if isinstance(p, W.PagedProblem):
        return oracle.decode_paged(p.dtype, W.bits(p.q), W.bits(p.k_data), W.bits(p.v_data),
                                   p.indices.numpy(), p.indptr.numpy(), p.last_page_len.numpy(),
                                   p.scale, samples=samples, layout=p.layout, window=window,
                                   softcap=softcap, alibi=alibi, mask=mask)
    return oracle.decode_contig(p.dtype, W.bits(p.q), W.bits(p.k_cache), W.bits(p.v_cache),
                                p.valid_kv_len, p.scale, layout=p.layout, window=window,
                                softcap=softcap, alibi=alibi, mask=mask)


def _run(p, d, window, softcap, alibi=None, mask=None):
    dev_alibi = dev_mask = None
    if alibi is not None:
        dev_alibi = torch.tensor(alibi, dtype=torch.float32, device=d["q"].device)
    if mask is not None:
        dev_mask = torch.from_numpy(np.ascontiguousarray(mask)).to(d["q"].device)
    if isinstance(p, W.PagedProblem):
        return fad.decode_paged(d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"],
                                p.scale, layout=p.layout, window=window, softcap=softcap,
                                alibi=dev_alibi, mask=dev_mask)
    return fad.decode_contig(d["q"], d["k"], d["v"], p.valid_kv_len, p.scale, layout=p.layout,
                             window=window, softcap=softcap, alibi=dev_alibi, mask=dev_mask)


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
    ("f32", 128, 2, 8, 32, [1, 300, 1500]),
    ("f32", 256, 1, 4, 16, [3, 700, 2049]),
    ("bf16", 128, 1, 32, 16, [5, 900, 2100]),
    # two 16-head blocks per workgroup (an even number of blocks)
    ("f16", 256, 2, 32, 16, [1, 48, 1500]),
    ("f32", 64, 1, 64, 8, [7, 600, 1100]),
    ("f32", 128, 1, 32, 16, [77, 1200]),  # shared tiles with the per-score options
    # a group that is not a power of two, and a ragged last head block
    ("bf16", 128, 2, 7, 16, [3, 800]),
    ("f16", 128, 1, 40, 16, [300, 1700]),
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
    """The full C3 workload with a 1000-row window and a soft-cap of 30, every
    output against the oracle; no window and a cap far beyond every score
    match the plain call within the tolerance."""
    p = W.FULL["c3"]()
    announce("variants full c3")
    d = to_dev(p, dev)
    o, lse = _run(p, d, 1000, 30.0)
    torch.cuda.synchronize()
    compare_all(p, o, lse, "c3 w1000 cap30", window=1000, softcap=30.0)
    o0, l0 = _run(p, d, 0, 0.0)
    o1, l1 = _run(p, d, 0, 1.0e6)
    torch.cuda.synchronize()
    assert torch.allclose(o1.float(), o0.float(), atol=4e-3, rtol=0)
    assert torch.allclose(l1, l0, atol=1e-4, rtol=0)


# ------------------------------------------------------------ custom mask

MASKS = [  # keep probability, blocks of rows, window, cap, alibi
    (0.5, False, 0, 0.0, False),
    (0.9, False, 0, 0.0, False),
    (0.05, False, 0, 0.0, False),
    (0.5, True, 0, 0.0, False),
    (0.7, False, 40, 0.0, True),
    (0.5, True, 0, 10.0, True),
    # block-sparse masks: whole 32-row tiles dropped, whose loads are skipped
    (0.3, 64, 0, 0.0, False),
    (0.5, 256, 0, 0.0, False),
    (0.4, 96, 40, 10.0, True),
]


@pytest.mark.parametrize("mvar", MASKS, ids=lambda m: f"keep{m[0]}"
                         + ("" if m[1] is False else "-blocks" if m[1] is True else f"-runs{m[1]}")
                         + (f"-w{m[2]}" if m[2] else "") + (f"-cap{m[3]:g}" if m[3] else "")
                         + ("-alibi" if m[4] else ""))
@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-D{c[1]}-G{c[3]}-P{c[4]}")
def test_paged_mask(dev, case, mvar):
    """Random and block masks over requests of ragged lengths (empty, one row,
    page edges, split requests), one request with every row dropped, alone
    and with a window, a cap and ALiBi; both K/V layouts."""
    dtype, d, hkv, group, page_size, lens = case
    keep_p, blocks, window, cap, with_alibi = mvar
    slopes = alibi_slopes(hkv * group) if with_alibi else None
    rng = np.random.default_rng(zlib.crc32(str(case).encode()) + 1)
    k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    kd, ind, ptr, lpl = scatter_paged(k_rows, page_size, np.random.default_rng(4), 3, (),
                                      fill=1.0e4)
    vd, _, _, _ = scatter_paged(v_rows, page_size, np.random.default_rng(4), 3, (), fill=1.0e4)
    q = rand_t(rng, (len(lens), hkv * group, d), dtype, std=2.0)
    p = W.PagedProblem(name="mask", dtype=dtype, batch=len(lens), num_qo_heads=hkv * group,
                       num_kv_heads=hkv, head_dim=d, page_size=page_size,
                       num_total_pages=kd.shape[0], scale=float(np.float32(1 / math.sqrt(d))),
                       q=q, k_data=kd, v_data=vd, indices=torch.from_numpy(ind),
                       indptr=torch.from_numpy(ptr), last_page_len=torch.from_numpy(lpl))
    keep = W.random_mask(zlib.crc32(str(mvar).encode()), lens, keep=keep_p, blocks=blocks)
    starts = np.concatenate([[0], np.cumsum(lens)])
    mid = len(lens) // 2
    keep[starts[mid]:starts[mid + 1]] = False  # a request left with no row
    packed = W.pack_mask(keep)
    for layout in ("hnd", "nhd"):
        pp = p if layout == "hnd" else W.token_major(p)
        o, lse = _run(pp, to_dev(pp, dev), window, cap, slopes, mask=packed)
        torch.cuda.synchronize()
        ro, rl = _oracle(pp, window, cap, alibi=slopes, mask=packed)
        compare(dtype, o, lse, ro, rl, f"{case} {mvar} {layout}")


def test_mask_all_ones_and_short(dev):
    """An all-ones mask gives the plain call's output bit for bit; a mask
    shorter than the rows drops the rows past its end (and reads nothing past
    it), which equals an explicit mask with those bits cleared."""
    p = W.make_paged("mask-short", "bf16", 6, 16, 4, 128, 16, 91,
                     lens=np.array([700, 3000, 1, 0, 2500, 40]), pool_slack=0.1)
    lens = oracle.seq_lens(p.page_size, p.indptr.numpy(), p.last_page_len.numpy())
    total = int(lens.sum())
    d = to_dev(p, dev)
    plain = _run(p, d, 0, 0.0)
    ones = _run(p, d, 0, 0.0, mask=W.pack_mask(np.ones(total, bool)))
    torch.cuda.synchronize()
    assert torch.equal(plain[0], ones[0]) and torch.equal(plain[1], ones[1])
    keep = W.random_mask(5, lens, keep=0.6)
    full = W.pack_mask(keep)
    cut = full[: full.size // 2]  # the second half of the rows read as dropped
    keep_cut = keep.copy()
    keep_cut[cut.size * 8:] = False
    got = _run(p, d, 0, 0.0, mask=cut)
    want = _run(p, d, 0, 0.0, mask=W.pack_mask(keep_cut))
    torch.cuda.synchronize()
    assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1])
    ro, rl = _oracle(p, 0, 0.0, mask=W.pack_mask(keep_cut))
    compare(p.dtype, got[0], got[1], ro, rl, "short mask")


@pytest.mark.parametrize("keep_p,blocks", [(0.5, False), (0.3, True), (0.3, 128), (0.6, 33)])
def test_contig_mask(dev, keep_p, blocks):
    p = W.make_contig("mask", "f16", 16, 4, 128, 5000, 4999, seed=78, q_std=2.0)
    keep = W.random_mask(12, [p.valid_kv_len], keep=keep_p, blocks=blocks)
    o, lse = _run(p, to_dev(p, dev), 0, 0.0, mask=W.pack_mask(keep))
    torch.cuda.synchronize()
    ro, rl = _oracle(p, 0, 0.0, mask=W.pack_mask(keep))
    compare("f16", o, lse, ro, rl, f"contig mask {keep_p} {blocks}")


@pytest.mark.parametrize("blocks", [False, 256])
def test_mask_full_c3(dev, blocks):
    """The full C3 workload under a random half mask (rows one by one, or
    256-row runs, whose dropped tiles are not loaded), every output against
    the oracle."""
    p = W.FULL["c3"]()
    announce(f"mask full c3 blocks={blocks}")
    lens = oracle.seq_lens(p.page_size, p.indptr.numpy(), p.last_page_len.numpy())
    packed = W.pack_mask(W.random_mask(13, lens, keep=0.5, blocks=blocks))
    o, lse = _run(p, to_dev(p, dev), 0, 0.0, mask=packed)
    torch.cuda.synchronize()
    compare_all(p, o, lse, "c3 mask", mask=packed)


def test_mask_long_units(dev):
    """Block-sparse mask over split units of more than 64 tiles per wave, so
    each wave looks up which of its tiles hold a kept row in more than one
    64-tile window (a contiguous cache of 9M rows, D = 64: units of ~8,800
    rows against 64 x 128 = 8,192 rows per window); every output against the
    oracle, and against the same call without the mask's dropped runs cut
    out of the rows (an all-ones mask) for the plain path."""
    n = 9_000_000
    chunk, _, _, _ = fad.fa_debug_plan(fad.FA_DTYPE_BF16, 1, 2, 1, 64, n, 1)
    assert chunk > 64 * 128, chunk
    p = W.make_contig("long-mask", "bf16", 2, 1, 64, n, n - 1, seed=515, q_std=2.0)
    announce(f"mask long units: chunk {chunk}")
    keep = W.random_mask(16, [p.valid_kv_len], keep=0.3, blocks=512)
    packed = W.pack_mask(keep)
    d = to_dev(p, dev)
    o, lse = _run(p, d, 0, 0.0, mask=packed)
    torch.cuda.synchronize()
    ro, rl = _oracle(p, 0, 0.0, mask=packed)
    compare("bf16", o, lse, ro, rl, "long units, block-sparse mask")
    ones = _run(p, d, 0, 0.0, mask=W.pack_mask(np.ones(p.valid_kv_len, bool)))
    plain = _run(p, d, 0, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(ones[0], plain[0]) and torch.equal(ones[1], plain[1])
    del d
    torch.cuda.empty_cache()
