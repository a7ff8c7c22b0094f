"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each pin_* function raises AssertionError when the oracle (whichever build the
`oracle` module currently routes through) disagrees with:
  * library routines: numpy's float16 and torch's bfloat16 widening, scipy's
    logsumexp, torch's float64 scaled_dot_product_attention with GQA;
  * closed forms: identical V rows, identical K rows, a single row, scale 0,
    the worked example printed on the ferrox-cuda page, the merge of two
    partials with equal lse;
  * brute force: a 50-digit mpmath evaluation of the definition on tiny inputs,
    without the max shift, over logical rows the test lays out in pages itself;
  * invariants: row permutation, poisoned excluded rows, paged vs contiguous,
    the page-table gather as the inverse of the test's own scatter.
The same functions run against deliberately broken copies of the oracle
(test_oracle_mutants.py) to show each plausible mistake fails at least one pin.
"""
import json
import math
import os

import mpmath
import numpy as np
import scipy.special
import torch

import oracle as O
import workloads as W
from _helpers import contig_from_rows, f64, rand_t, scatter_paged

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = ("f32", "f16", "bf16")


def _paged_problem(rng, dtype, lens, hkv, group, d, page_size, pool_extra=3,
                   empty_last_page=(), k_rows=None, v_rows=None, q=None, layout="hnd"):
    """Random logical rows -> paged layout.  Returns a dict with both views."""
    hq = hkv * group
    batch = len(lens)
    if k_rows is None:
        k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    if v_rows is None:
        v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
    if q is None:
        q = rand_t(rng, (batch, hq, d), dtype)
    seed = int(rng.integers(1 << 30))
    kd, ind, ptr, lpl = scatter_paged(k_rows, page_size, np.random.default_rng(seed),
                                      pool_extra, empty_last_page, fill=1.0e4, layout=layout)
    vd, ind2, ptr2, lpl2 = scatter_paged(v_rows, page_size, np.random.default_rng(seed),
                                         pool_extra, empty_last_page, fill=1.0e4,
                                         layout=layout)
    assert np.array_equal(ind, ind2) and np.array_equal(lpl, lpl2)
    return dict(dtype=dtype, q=q, k_rows=k_rows, v_rows=v_rows, k_data=kd, v_data=vd,
                indices=ind, indptr=ptr, last_page_len=lpl, hq=hq, hkv=hkv, group=group,
                d=d, page_size=page_size, layout=layout)


def _oracle_paged(p, scale):
    return O.decode_paged(p["dtype"], W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]),
                          p["indices"], p["indptr"], p["last_page_len"], scale,
                          layout=p["layout"])


# ------------------------------------------------------------------ decoders

def pin_f16_decoder():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([O.f16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)), "f16 NaN patterns"
    assert np.array_equal(ref[~nan], got[~nan]), "f16 values"
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan])), "f16 signs"


def pin_bf16_decoder():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.bf16_to_f64(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got)), "bf16 NaN patterns"
    assert np.array_equal(ref[~nan], got[~nan]), "bf16 values"
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan])), "bf16 signs"


# ------------------------------------------------------------- worked example

def pin_worked_example():
    """The ferrox-cuda page's hardware test inputs; closed-form outputs."""
    g = json.load(open(os.path.join(GOLDEN, "ferrox_gqa_decode_hw_example.json")))
    hq, hkv, d, L = g["n_heads"], g["n_kv_heads"], g["head_dim"], g["seq_len"]
    qv, kv, vv = (np.float32(g["q_fill_f32"]), np.float32(g["k_fill_f32"]),
                  np.float32(g["v_fill_f32"]))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q = np.full((hq, d), qv, dtype=np.float32)
    k = np.full((hkv, L, d), kv, dtype=np.float32)
    v = np.full((hkv, L, d), vv, dtype=np.float32)
    o, lse = O.decode_contig("f32", q, k, v, L, scale)
    score = d * float(qv) * float(kv) * scale
    assert np.all(o == float(vv)), "worked example: o must equal the V row"
    assert np.allclose(lse, score + math.log(3.0), rtol=0, atol=1e-15), "worked example lse"
    # the same rows through a paged store with a ragged last page
    rng = np.random.default_rng(7)
    rows_k = torch.full((L, hkv, d), float(kv), dtype=torch.float32)
    rows_v = torch.full((L, hkv, d), float(vv), dtype=torch.float32)
    p = _paged_problem(rng, "f32", [L], hkv, hq // hkv, d, 2, k_rows=[rows_k],
                       v_rows=[rows_v], q=torch.from_numpy(q[None].copy()))
    o2, lse2 = _oracle_paged(p, scale)
    assert np.all(o2 == float(vv)) and np.allclose(lse2, score + math.log(3.0), atol=1e-15)


# ----------------------------------------------------------------- closed forms

def pin_identical_v_rows():
    rng = np.random.default_rng(11)
    for dtype in DTYPES:
        lens = [5, 17, 1, 33]
        vstar = rand_t(rng, (1, 2, 64), dtype)
        v_rows = [vstar.expand(L, 2, 64).contiguous() for L in lens]
        p = _paged_problem(rng, dtype, lens, 2, 3, 64, 4, v_rows=v_rows)
        o, _ = _oracle_paged(p, 0.125)
        want = f64(vstar)[0]
        for b in range(len(lens)):
            for h in range(p["hq"]):
                np.testing.assert_allclose(o[b, h], want[h // 3], rtol=1e-14, atol=0)


def pin_identical_k_rows():
    rng = np.random.default_rng(12)
    for dtype in DTYPES:
        lens = [3, 16, 40]
        kstar = rand_t(rng, (1, 2, 32), dtype)
        k_rows = [kstar.expand(L, 2, 32).contiguous() for L in lens]
        p = _paged_problem(rng, dtype, lens, 2, 2, 32, 5, k_rows=k_rows)
        scale = 0.3
        o, lse = _oracle_paged(p, scale)
        qf, kf = f64(p["q"]), f64(kstar)[0]
        for b, L in enumerate(lens):
            vmean = f64(p["v_rows"][b]).mean(axis=0)
            for h in range(p["hq"]):
                g = h // 2
                np.testing.assert_allclose(o[b, h], vmean[g], rtol=1e-12, atol=1e-14)
                x = scale * float(np.dot(qf[b, h], kf[g]))
                assert abs(lse[b, h] - (x + math.log(L))) < 1e-12


def pin_single_row():
    rng = np.random.default_rng(13)
    for dtype in DTYPES:
        p = _paged_problem(rng, dtype, [1, 1], 2, 4, 128, 16)
        scale = 0.0884
        o, lse = _oracle_paged(p, scale)
        qf = f64(p["q"])
        for b in range(2):
            v0, k0 = f64(p["v_rows"][b])[0], f64(p["k_rows"][b])[0]
            for h in range(p["hq"]):
                assert np.array_equal(o[b, h], v0[h // 4]), "L=1 must return V[0]"
                assert abs(lse[b, h] - scale * float(np.dot(qf[b, h], k0[h // 4]))) < 1e-12


def pin_scale_zero():
    rng = np.random.default_rng(14)
    lens = [7, 64, 2]
    p = _paged_problem(rng, "bf16", lens, 1, 4, 64, 8)
    o, lse = _oracle_paged(p, 0.0)
    for b, L in enumerate(lens):
        vmean = f64(p["v_rows"][b]).mean(axis=0)[0]
        for h in range(4):
            np.testing.assert_allclose(o[b, h], vmean, rtol=1e-12, atol=1e-14)
            assert abs(lse[b, h] - math.log(L)) < 1e-13


def pin_empty_requests():
    """n_b = 0, and a single allocated page with last_page_len 0: o = 0, lse = -inf."""
    rng = np.random.default_rng(15)
    k_rows = [rand_t(rng, (L, 2, 64), "f16") for L in (0, 0, 9)]
    v_rows = [rand_t(rng, (L, 2, 64), "f16") for L in (0, 0, 9)]
    p = _paged_problem(rng, "f16", [0, 0, 9], 2, 2, 64, 4, empty_last_page=(1,),
                       k_rows=k_rows, v_rows=v_rows)
    assert list(np.diff(p["indptr"])) == [0, 1, 3] and p["last_page_len"][1] == 0
    o, lse = _oracle_paged(p, 0.125)
    for b in (0, 1):
        assert np.all(o[b] == 0.0) and np.all(np.isneginf(lse[b]))
    assert np.all(np.isfinite(lse[2]))
    qc = rand_t(rng, (4, 64), "f32")
    kc = rand_t(rng, (2, 8, 64), "f32")
    o, lse = O.decode_contig("f32", W.bits(qc), W.bits(kc), W.bits(kc), 0, 0.125)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


# -------------------------------------------------------- library routines

def pin_lse_logsumexp():
    rng = np.random.default_rng(16)
    lens = [100, 1, 37, 256]
    p = _paged_problem(rng, "f32", lens, 4, 2, 64, 16)
    scale = 0.125
    _, lse = _oracle_paged(p, scale)
    qf = f64(p["q"])
    for b in range(len(lens)):
        kf = f64(p["k_rows"][b])  # [L, Hkv, D]
        for h in range(p["hq"]):
            x = scale * (kf[:, h // 2, :] @ qf[b, h])
            assert abs(lse[b, h] - scipy.special.logsumexp(x)) < 1e-12


def pin_sdpa_float64():
    rng = np.random.default_rng(17)
    for dtype, (hq, hkv, d, L, maxlen) in [("f32", (8, 2, 64, 128, 256)),
                                           ("f16", (12, 4, 128, 300, 301)),
                                           ("bf16", (6, 1, 256, 77, 80))]:
        q = rand_t(rng, (hq, d), dtype)
        rows_k = rand_t(rng, (L, hkv, d), dtype)
        rows_v = rand_t(rng, (L, hkv, d), dtype)
        kc, vc = contig_from_rows(rows_k, maxlen), contig_from_rows(rows_v, maxlen)
        scale = float(np.float32(1.0 / math.sqrt(d)))
        o, _ = O.decode_contig(dtype, W.bits(q), W.bits(kc), W.bits(vc), L, scale)
        tq = torch.from_numpy(f64(q))[None, :, None, :]
        tk = torch.from_numpy(f64(rows_k)).permute(1, 0, 2)[None].contiguous()
        tv = torch.from_numpy(f64(rows_v)).permute(1, 0, 2)[None].contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale,
                                                               enable_gqa=True)
        np.testing.assert_allclose(o, ref[0, :, 0, :].numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------------ brute force

def _mp_attend(qrow, krows, vrows, scale):
    """50-digit evaluation of the definition, one pass, no max shift."""
    mpmath.mp.dps = 50
    L = len(krows)
    if L == 0:
        return [mpmath.mpf(0)] * len(qrow), -mpmath.inf
    w = []
    for j in range(L):
        x = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                            for a, b in zip(qrow, krows[j]))
        w.append(mpmath.e ** x)
    z = mpmath.fsum(w)
    o = [mpmath.fsum(w[j] * mpmath.mpf(vrows[j][d]) for j in range(L)) / z
         for d in range(len(qrow))]
    return o, mpmath.log(z)


def pin_bruteforce_mpmath():
    _bruteforce(np.random.default_rng(18), "hnd", (1, 2, 4), (1, 2, 3, 4))


def pin_bruteforce_mpmath_token_major():
    """The same brute force over token-major pages [pages, P, Hkv, D]."""
    _bruteforce(np.random.default_rng(28), "nhd", (1, 3), (1, 2, 4))


def _bruteforce(rng, layout, dims, page_sizes):
    for d in dims:
        for page_size in page_sizes:
            for group in (1, 2, 3):
                hkv = 1 + int(rng.integers(2))
                dtype = DTYPES[int(rng.integers(3))]
                lens = [int(x) for x in rng.integers(0, 7, size=3)]
                empty = tuple(b for b in range(3) if lens[b] % page_size == 0
                              and rng.random() < 0.5)
                p = _paged_problem(rng, dtype, lens, hkv, group, d, page_size,
                                   pool_extra=int(rng.integers(4)), empty_last_page=empty,
                                   layout=layout)
                scale = float(rng.uniform(0.1, 2.0))
                o, lse = _oracle_paged(p, scale)
                qf = f64(p["q"])
                for b, L in enumerate(lens):
                    kf, vf = f64(p["k_rows"][b]), f64(p["v_rows"][b])
                    for h in range(p["hq"]):
                        g = h // group
                        mo, ml = _mp_attend(qf[b, h], kf[:, g, :], vf[:, g, :], scale)
                        if L == 0:
                            assert np.all(o[b, h] == 0) and np.isneginf(lse[b, h])
                            continue
                        for dd in range(d):
                            ref = float(mo[dd])
                            assert abs(o[b, h, dd] - ref) <= 1e-13 * max(1.0, abs(ref)), \
                                (d, page_size, group, b, h, dd)
                        assert abs(lse[b, h] - float(ml)) <= 1e-13 * max(1.0, abs(float(ml)))


def pin_attend_f64_mpmath():
    """The oracle's attention over explicit f64 rows (what a split's partial
    is) against the 50-digit evaluation of the definition, on random
    double-precision rows of assorted lengths, head dims and scales; no rows
    gives o = 0 and lse = -inf."""
    rng = np.random.default_rng(29)
    for trial in range(40):
        d = int(rng.choice([1, 2, 3, 8, 16]))
        L = int(rng.integers(1, 9))
        q = rng.standard_normal(d) * 1.5
        k = rng.standard_normal((L, d)) * 1.5
        v = rng.standard_normal((L, d)) * float(rng.choice([0.25, 1.0, 4.0]))
        scale = float(rng.uniform(0.05, 2.0))
        o, lse = O.attend_f64(q, k, v, scale)
        mo, ml = _mp_attend(q.tolist(), k.tolist(), v.tolist(), scale)
        for dd in range(d):
            ref = float(mo[dd])
            assert abs(o[dd] - ref) <= 1e-13 * max(1.0, abs(ref)), (trial, dd)
        assert abs(lse - float(ml)) <= 1e-13 * max(1.0, abs(float(ml))), trial
    o, lse = O.attend_f64(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 0.5)
    assert np.all(o == 0.0) and np.isneginf(lse)


# ------------------------------------------------------------- head mapping

def pin_head_mapping():
    """Distinct constant V per KV head: query head h must see KV head h // G."""
    rng = np.random.default_rng(19)
    hkv, group, d = 3, 4, 64
    lens = [6, 21]
    consts = [0.25, -1.5, 3.0]
    v_rows = []
    for L in lens:
        t = torch.empty((L, hkv, d), dtype=torch.float16)
        for g in range(hkv):
            t[:, g, :] = consts[g]
        v_rows.append(t)
    p = _paged_problem(rng, "f16", lens, hkv, group, d, 4, v_rows=v_rows)
    o, _ = _oracle_paged(p, 0.125)
    for b in range(len(lens)):
        for h in range(hkv * group):
            np.testing.assert_allclose(o[b, h], consts[h // group], rtol=1e-14, atol=0)


# -------------------------------------------------------------- split / merge

def pin_merge_closed_form():
    """Two parts with equal lse: weights 1/2 each, lse grows by ln 2."""
    rng = np.random.default_rng(20)
    o1, o2 = rng.standard_normal(16), rng.standard_normal(16)
    o, lse = O.merge(np.stack([o1, o2]), np.array([0.7, 0.7]))
    np.testing.assert_allclose(o, 0.5 * (o1 + o2), rtol=1e-15, atol=1e-15)
    assert abs(lse - (0.7 + math.log(2.0))) < 1e-15
    # an empty part (lse = -inf) changes nothing; all parts empty gives 0 / -inf
    o, lse = O.merge(np.stack([o1, np.full(16, np.nan)]), np.array([1.25, -np.inf]))
    assert np.array_equal(o, o1) and lse == 1.25
    o, lse = O.merge(np.zeros((3, 16)), np.full(3, -np.inf))
    assert np.all(o == 0) and np.isneginf(lse)


def pin_merge_partition():
    """Merging the partials of any partition of the rows gives the whole."""
    rng = np.random.default_rng(21)
    for trial in range(20):
        L = int(rng.integers(1, 200))
        d = 32
        q = rng.standard_normal(d)
        k = rng.standard_normal((L, d)) * 2.0
        v = rng.standard_normal((L, d))
        scale = float(rng.uniform(0.05, 1.0))
        o_all, lse_all = O.attend_f64(q, k, v, scale)
        cuts = np.sort(rng.integers(0, L + 1, size=int(rng.integers(0, 6))))
        bounds = [0, *cuts.tolist(), L]
        parts = [O.attend_f64(q, k[a:b], v[a:b], scale) for a, b in zip(bounds, bounds[1:])]
        o, lse = O.merge(np.stack([p[0] for p in parts]), np.array([p[1] for p in parts]))
        np.testing.assert_allclose(o, o_all, rtol=0, atol=1e-12)
        assert abs(lse - lse_all) < 1e-12


# -------------------------------------------------------------- invariants

def pin_permutation_invariance():
    rng = np.random.default_rng(22)
    lens = [50, 129]
    p = _paged_problem(rng, "bf16", lens, 2, 4, 128, 16)
    o, lse = _oracle_paged(p, 0.0884)
    perms = [rng.permutation(L) for L in lens]
    p2 = _paged_problem(rng, "bf16", lens, 2, 4, 128, 16, q=p["q"],
                        k_rows=[r[pp] for r, pp in zip(p["k_rows"], perms)],
                        v_rows=[r[pp] for r, pp in zip(p["v_rows"], perms)])
    o2, lse2 = _oracle_paged(p2, 0.0884)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)


def pin_masking_poison():
    """Rows outside [0, L_b) and unreferenced pages never change a bit."""
    rng = np.random.default_rng(23)
    lens = [13, 31, 8]
    p = _paged_problem(rng, "f16", lens, 2, 2, 64, 8, pool_extra=5)
    o, lse = _oracle_paged(p, 0.125)
    used = np.zeros(p["k_data"].shape[0], dtype=bool)
    used[p["indices"]] = True
    for poison in (float("nan"), -1.0e4, 6.0e4):
        kd, vd = p["k_data"].clone(), p["v_data"].clone()
        kd[torch.from_numpy(~used)] = poison
        vd[torch.from_numpy(~used)] = poison
        for b in range(len(lens)):
            last = int(p["indices"][p["indptr"][b + 1] - 1])
            r0 = int(p["last_page_len"][b])
            kd[last, :, r0:, :] = poison
            vd[last, :, r0:, :] = poison
        o2, lse2 = O.decode_paged("f16", W.bits(p["q"]), W.bits(kd), W.bits(vd), p["indices"],
                                  p["indptr"], p["last_page_len"], 0.125)
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # contiguous: slots past valid_kv_len
    q = rand_t(rng, (8, 64), "f32")
    rows_k, rows_v = rand_t(rng, (40, 2, 64), "f32"), rand_t(rng, (40, 2, 64), "f32")
    ref = O.decode_contig("f32", W.bits(q), W.bits(contig_from_rows(rows_k, 64)),
                          W.bits(contig_from_rows(rows_v, 64)), 40, 0.125)
    for poison in (float("nan"), 1.0e4):
        got = O.decode_contig("f32", W.bits(q), W.bits(contig_from_rows(rows_k, 64, poison)),
                              W.bits(contig_from_rows(rows_v, 64, poison)), 40, 0.125)
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def pin_paged_equals_contig():
    rng = np.random.default_rng(24)
    for dtype in DTYPES:
        L, hkv, group, d = 97, 2, 4, 128
        q = rand_t(rng, (hkv * group, d), dtype)
        rows_k, rows_v = rand_t(rng, (L, hkv, d), dtype), rand_t(rng, (L, hkv, d), dtype)
        oc, lc = O.decode_contig(dtype, W.bits(q), W.bits(contig_from_rows(rows_k, 128)),
                                 W.bits(contig_from_rows(rows_v, 128)), L, 0.0884)
        for page_size in (1, 16, 97, 128):
            p = _paged_problem(rng, dtype, [L], hkv, group, d, page_size, k_rows=[rows_k],
                               v_rows=[rows_v], q=q[None].contiguous())
            op, lp = _oracle_paged(p, 0.0884)
            assert np.array_equal(op[0], oc) and np.array_equal(lp[0], lc), (dtype, page_size)


def pin_token_major_equals_heads_major():
    """The same logical rows laid out token-major (contiguous [L, Hkv, D] as on
    the ferrox-cuda page, paged [pages, P, Hkv, D]) give bit-identical results
    to the heads-major layouts, and gather back to the same rows."""
    rng = np.random.default_rng(27)
    for dtype in DTYPES:
        L, hkv, group, d = 53, 3, 2, 64
        q = rand_t(rng, (hkv * group, d), dtype)
        rows_k, rows_v = rand_t(rng, (L, hkv, d), dtype), rand_t(rng, (L, hkv, d), dtype)
        ref = O.decode_contig(dtype, W.bits(q), W.bits(contig_from_rows(rows_k, 60)),
                              W.bits(contig_from_rows(rows_v, 60)), L, 0.125)
        got = O.decode_contig(dtype, W.bits(q),
                              W.bits(contig_from_rows(rows_k, 60, layout="nhd")),
                              W.bits(contig_from_rows(rows_v, 60, layout="nhd")), L, 0.125,
                              layout="nhd")
        assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1]), dtype
        lens = [L, 0, 16, 7]
        k_rows = [rows_k] + [rand_t(rng, (n, hkv, d), dtype) for n in lens[1:]]
        v_rows = [rows_v] + [rand_t(rng, (n, hkv, d), dtype) for n in lens[1:]]
        qb = rand_t(rng, (len(lens), hkv * group, d), dtype)
        seed = int(rng.integers(1 << 30))
        out = {}
        for layout in ("hnd", "nhd"):
            p = _paged_problem(np.random.default_rng(seed), dtype, lens, hkv, group, d, 8,
                               empty_last_page=(2,), k_rows=k_rows, v_rows=v_rows, q=qb,
                               layout=layout)
            out[layout] = _oracle_paged(p, 0.125)
            got = O.gather_paged(dtype, W.bits(p["k_data"]), p["indices"], p["indptr"],
                                 p["last_page_len"], layout=layout)
            want = np.concatenate([W.bits(r) for r in k_rows if r.shape[0]])
            assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), (dtype, layout)
        assert np.array_equal(out["hnd"][0], out["nhd"][0]), dtype
        assert np.array_equal(out["hnd"][1], out["nhd"][1]), dtype


def pin_gather_inverse():
    rng = np.random.default_rng(25)
    for dtype in DTYPES:
        lens = [0, 1, 16, 17, 45]
        p = _paged_problem(rng, dtype, lens, 3, 1, 64, 16, pool_extra=4,
                           empty_last_page=(2,))
        for which in ("k", "v"):
            got = O.gather_paged(dtype, W.bits(p[which + "_data"]), p["indices"], p["indptr"],
                                 p["last_page_len"])
            want = np.concatenate([W.bits(r) for r in p[which + "_rows"] if r.shape[0]])
            assert got.shape == want.shape and np.array_equal(got.view(np.uint8),
                                                              want.view(np.uint8))


def pin_append_completes_the_scatter():
    """Appending each request's last logical row into a store that holds all
    but that row gives, bit for bit, the store holding every row (the test's
    own scatter), in both layouts; empty requests and every other byte of the
    pool are left alone."""
    rng = np.random.default_rng(29)
    for layout in ("hnd", "nhd"):
        for dtype in DTYPES:
            page_size, hkv, d = 4, 3, 8
            lens = [1, 0, 4, 5, 9, 8]           # request 5 also gets an empty last page
            rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
            seed = int(rng.integers(1 << 30))
            full, ind, ptr, lpl = scatter_paged(rows, page_size, np.random.default_rng(seed), 3,
                                                (5,), fill=7.0, layout=layout)
            # the same table, but each request's last row still holds stale values
            stale = [r.clone() for r in rows]
            for r in stale:
                if r.shape[0]:
                    r[-1] = -3.0
            before, ind2, _, _ = scatter_paged(stale, page_size, np.random.default_rng(seed), 3,
                                               (5,), fill=7.0, layout=layout)
            assert np.array_equal(ind, ind2)
            new = torch.zeros((len(lens), hkv, d), dtype=rows[0].dtype)
            for b, r in enumerate(rows):
                new[b] = r[-1] if r.shape[0] else 99.0   # ignored for the empty request
            got = O.append_paged(dtype, W.bits(before), ind, ptr, lpl, W.bits(new),
                                 layout=layout)
            assert np.array_equal(got.view(np.uint8), W.bits(full).view(np.uint8)), \
                (layout, dtype)


# ------------------------------------------------- sliding window, soft-cap

def pin_window_is_truncation():
    """A sliding window of W rows equals plain attention over each request's
    last W rows, laid out by the test itself, bit for bit (paged and
    contiguous); W = 0 and W >= L change nothing; W = 1 gives the newest row."""
    rng = np.random.default_rng(32)
    for dtype in DTYPES:
        hkv, group, d, page_size = 2, 3, 16, 4
        lens = [0, 1, 5, 13, 31]
        k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
        v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
        q = rand_t(rng, (len(lens), hkv * group, d), dtype)
        p = _paged_problem(rng, dtype, lens, hkv, group, d, page_size, k_rows=k_rows,
                           v_rows=v_rows, q=q)
        full = _oracle_paged(p, 0.3)
        args = (dtype, W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]), p["indices"],
                p["indptr"], p["last_page_len"], 0.3)
        for win in (0, 1, 4, 13, 40):
            got = O.decode_paged(*args, window=win)
            cut = [(r[max(0, r.shape[0] - win):] if win else r) for r in k_rows]
            cutv = [(r[max(0, r.shape[0] - win):] if win else r) for r in v_rows]
            pt = _paged_problem(rng, dtype, [r.shape[0] for r in cut], hkv, group, d, page_size,
                                k_rows=cut, v_rows=cutv, q=q)
            want = _oracle_paged(pt, 0.3)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), \
                (dtype, win)
            if win == 0 or win >= max(lens):
                assert np.array_equal(got[0], full[0]) and np.array_equal(got[1], full[1])
            if win == 1:
                for b, L in enumerate(lens):
                    if L:
                        for h in range(hkv * group):
                            assert np.array_equal(got[0][b, h], f64(v_rows[b][L - 1, h // group]))
        # contiguous: the window of a cache equals the cache of the window
        L, win = 29, 7
        rk, rv = rand_t(rng, (L, hkv, d), dtype), rand_t(rng, (L, hkv, d), dtype)
        qc = rand_t(rng, (hkv * group, d), dtype)
        got = O.decode_contig(dtype, W.bits(qc), W.bits(contig_from_rows(rk, 40)),
                              W.bits(contig_from_rows(rv, 40)), L, 0.3, window=win)
        want = O.decode_contig(dtype, W.bits(qc), W.bits(contig_from_rows(rk[L - win:], 40)),
                               W.bits(contig_from_rows(rv[L - win:], 40)), win, 0.3)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), dtype


def _mp_attend_capped(qrow, krows, vrows, scale, cap):
    """50-digit evaluation with capped scores cap * tanh(x / cap)."""
    mpmath.mp.dps = 50
    w = []
    for j in range(len(krows)):
        x = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                            for a, b in zip(qrow, krows[j]))
        w.append(mpmath.e ** (mpmath.mpf(cap) * mpmath.tanh(x / mpmath.mpf(cap))))
    z = mpmath.fsum(w)
    o = [mpmath.fsum(w[j] * mpmath.mpf(vrows[j][d]) for j in range(len(krows))) / z
         for d in range(len(qrow))]
    return o, mpmath.log(z)


def pin_softcap_mpmath():
    """Capped scores against a 50-digit evaluation, on tiny requests, for caps
    that bind hard (0.5), moderately (3) and barely (50)."""
    rng = np.random.default_rng(33)
    for cap in (0.5, 3.0, 50.0):
        for dtype in DTYPES:
            hkv, group, d = 2, 2, 4
            lens = [1, 3, 6]
            p = _paged_problem(rng, dtype, lens, hkv, group, d, 2)
            scale = 1.7
            o, lse = O.decode_paged(dtype, W.bits(p["q"]), W.bits(p["k_data"]),
                                    W.bits(p["v_data"]), p["indices"], p["indptr"],
                                    p["last_page_len"], scale, softcap=cap)
            qf = f64(p["q"])
            for b in range(len(lens)):
                kf, vf = f64(p["k_rows"][b]), f64(p["v_rows"][b])
                for h in range(hkv * group):
                    mo, ml = _mp_attend_capped(qf[b, h], kf[:, h // group], vf[:, h // group],
                                               scale, cap)
                    for dd in range(d):
                        assert abs(o[b, h, dd] - float(mo[dd])) <= 1e-13 * max(1, abs(float(mo[dd])))
                    assert abs(lse[b, h] - float(ml)) <= 1e-13 * max(1.0, abs(float(ml)))


def pin_softcap_identical_k_rows():
    """Identical K rows stay equally weighted under the cap: o is the mean of
    V and lse = cap * tanh(x / cap) + ln L."""
    rng = np.random.default_rng(34)
    hkv, group, d, L, cap = 1, 2, 32, 9, 2.0
    k_row = rand_t(rng, (1, hkv, d), "f32")
    k_rows = [k_row.expand(L, hkv, d).contiguous()]
    p = _paged_problem(rng, "f32", [L], hkv, group, d, 4, k_rows=k_rows)
    o, lse = O.decode_paged("f32", W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]),
                            p["indices"], p["indptr"], p["last_page_len"], 0.5, softcap=cap)
    vf = f64(p["v_rows"][0])
    qf, kf = f64(p["q"]), f64(k_row)
    for h in range(group):
        np.testing.assert_allclose(o[0, h], vf[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15)
        x = 0.5 * float(mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b)
                                    for a, b in zip(qf[0, h], kf[0, 0])))
        want = cap * math.tanh(x / cap) + math.log(L)
        assert abs(lse[0, h] - want) <= 1e-13 * max(1.0, abs(want))


def _slopes(hq):
    return [2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)]


def pin_alibi_mpmath():
    """ALiBi scores against a 50-digit evaluation of scale * q.k + m_h * (j - (L - 1))
    (also under a cap, where the bias comes first)."""
    rng = np.random.default_rng(35)
    for cap in (0.0, 4.0):
        for dtype in DTYPES:
            hkv, group, d = 2, 2, 4
            lens = [1, 4, 7]
            p = _paged_problem(rng, dtype, lens, hkv, group, d, 3)
            slopes = _slopes(hkv * group)
            scale = 0.9
            o, lse = O.decode_paged(dtype, W.bits(p["q"]), W.bits(p["k_data"]),
                                    W.bits(p["v_data"]), p["indices"], p["indptr"],
                                    p["last_page_len"], scale, softcap=cap, alibi=slopes)
            mpmath.mp.dps = 50
            qf = f64(p["q"])
            for b, L in enumerate(lens):
                kf, vf = f64(p["k_rows"][b]), f64(p["v_rows"][b])
                for h in range(hkv * group):
                    g = h // group
                    xs = []
                    for j in range(L):
                        x = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                                            for a, c in zip(qf[b, h], kf[j, g]))
                        x += mpmath.mpf(slopes[h]) * (j - (L - 1))
                        if cap:
                            x = mpmath.mpf(cap) * mpmath.tanh(x / cap)
                        xs.append(mpmath.e ** x)
                    z = mpmath.fsum(xs)
                    for dd in range(d):
                        ref = float(mpmath.fsum(xs[j] * mpmath.mpf(vf[j, g, dd])
                                                for j in range(L)) / z)
                        assert abs(o[b, h, dd] - ref) <= 1e-13 * max(1.0, abs(ref))
                    assert abs(lse[b, h] - float(mpmath.log(z))) <= 1e-13 * max(1.0, abs(float(mpmath.log(z))))


def pin_alibi_geometric_weights():
    """Identical K rows under ALiBi: row j weighs exp(m (j - L + 1)), a geometric
    sequence, so o is the geometric mean-weighted V and lse = x + ln sum_k e^(-m k).
    Zero slopes change nothing, bit for bit."""
    rng = np.random.default_rng(36)
    hkv, group, d, L = 1, 4, 16, 11
    k_row = rand_t(rng, (1, hkv, d), "f32")
    p = _paged_problem(rng, "f32", [L], hkv, group, d, 4,
                       k_rows=[k_row.expand(L, hkv, d).contiguous()])
    args = ("f32", W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]), p["indices"],
            p["indptr"], p["last_page_len"], 0.25)
    plain = O.decode_paged(*args)
    zero = O.decode_paged(*args, alibi=[0.0] * group)
    assert np.array_equal(plain[0], zero[0]) and np.array_equal(plain[1], zero[1])
    slopes = _slopes(group)
    o, lse = O.decode_paged(*args, alibi=slopes)
    vf = f64(p["v_rows"][0])[:, 0, :]
    qf, kf = f64(p["q"])[0], f64(k_row)[0, 0]
    for h in range(group):
        w = np.exp(slopes[h] * (np.arange(L) - (L - 1)))
        np.testing.assert_allclose(o[0, h], (w[:, None] * vf).sum(0) / w.sum(), rtol=1e-12,
                                   atol=1e-14)
        x = 0.25 * float(np.dot(qf[h], kf))
        assert abs(lse[0, h] - (x + math.log(w.sum()))) <= 1e-12


def pin_alibi_window_is_truncation():
    """Distances count back from the query, so a window of W rows under ALiBi
    equals the truncated request with the same slopes, bit for bit."""
    rng = np.random.default_rng(37)
    hkv, group, d, L, win = 2, 2, 8, 23, 9
    rows_k, rows_v = rand_t(rng, (L, hkv, d), "bf16"), rand_t(rng, (L, hkv, d), "bf16")
    q = rand_t(rng, (1, hkv * group, d), "bf16")
    slopes = _slopes(hkv * group)
    p = _paged_problem(rng, "bf16", [L], hkv, group, d, 4, k_rows=[rows_k], v_rows=[rows_v], q=q)
    got = O.decode_paged("bf16", W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]),
                         p["indices"], p["indptr"], p["last_page_len"], 0.3, window=win,
                         alibi=slopes)
    pt = _paged_problem(rng, "bf16", [win], hkv, group, d, 4, k_rows=[rows_k[L - win:]],
                        v_rows=[rows_v[L - win:]], q=q)
    want = O.decode_paged("bf16", W.bits(pt["q"]), W.bits(pt["k_data"]), W.bits(pt["v_data"]),
                          pt["indices"], pt["indptr"], pt["last_page_len"], 0.3, alibi=slopes)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def _masked_rows(rows, keep):
    return rows[torch.from_numpy(np.asarray(keep, dtype=bool))]


def pin_mask_is_compaction():
    """A custom mask equals plain attention over the kept rows, laid out by the
    test itself, bit for bit: random and all-ones masks, requests whose rows
    are all dropped (o = 0, lse = -inf), and a window on top (a row must pass
    both).  Several requests, so each request's bits must start at its own
    offset; paged and contiguous."""
    rng = np.random.default_rng(38)
    for dtype in DTYPES:
        hkv, group, d, page_size = 2, 2, 8, 4
        lens = [6, 0, 13, 1, 22, 9]
        k_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
        v_rows = [rand_t(rng, (L, hkv, d), dtype) for L in lens]
        q = rand_t(rng, (len(lens), hkv * group, d), dtype)
        p = _paged_problem(rng, dtype, lens, hkv, group, d, page_size, k_rows=k_rows,
                           v_rows=v_rows, q=q)
        args = (dtype, W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]), p["indices"],
                p["indptr"], p["last_page_len"], 0.4)
        starts = np.concatenate([[0], np.cumsum(lens)])
        plain = O.decode_paged(*args)
        for trial, win in ((0, 0), (1, 0), (2, 0), (3, 5)):
            keep = W.random_mask(100 + trial, lens, keep=0.5) if trial else np.ones(sum(lens), bool)
            if trial == 2:
                keep[starts[4]:starts[5]] = False  # a request with every row dropped
            got = O.decode_paged(*args, window=win, mask=W.pack_mask(keep))
            per = []
            for b, L in enumerate(lens):
                kb = keep[starts[b]:starts[b + 1]].copy()
                if win:
                    kb[:max(0, L - win)] = False
                per.append(kb)
            pt = _paged_problem(rng, dtype, [int(m.sum()) for m in per], hkv, group, d, page_size,
                                k_rows=[_masked_rows(r, m) for r, m in zip(k_rows, per)],
                                v_rows=[_masked_rows(r, m) for r, m in zip(v_rows, per)], q=q)
            want = _oracle_paged(pt, 0.4)
            assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), \
                (dtype, trial)
            if trial == 0:
                assert np.array_equal(got[0], plain[0]) and np.array_equal(got[1], plain[1])
            if trial == 2:
                assert np.all(got[0][4] == 0.0) and np.all(np.isneginf(got[1][4]))
        # contiguous: bit j for row j
        L = 27
        rk, rv = rand_t(rng, (L, hkv, d), dtype), rand_t(rng, (L, hkv, d), dtype)
        qc = rand_t(rng, (hkv * group, d), dtype)
        keep = W.random_mask(7, [L], keep=0.4, blocks=True)
        got = O.decode_contig(dtype, W.bits(qc), W.bits(contig_from_rows(rk, 32)),
                              W.bits(contig_from_rows(rv, 32)), L, 0.4, mask=W.pack_mask(keep))
        n = int(keep.sum())
        want = O.decode_contig(dtype, W.bits(qc), W.bits(contig_from_rows(_masked_rows(rk, keep), 32)),
                               W.bits(contig_from_rows(_masked_rows(rv, keep), 32)), n, 0.4)
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), dtype


def pin_mask_alibi_mpmath():
    """Under a mask, ALiBi still measures each kept row's distance from the
    query at its original position: a 50-digit evaluation over the kept rows
    with m_h * (j - (L - 1))."""
    rng = np.random.default_rng(39)
    hkv, group, d = 1, 2, 4
    lens = [9, 5]
    p = _paged_problem(rng, "f32", lens, hkv, group, d, 3)
    keep = W.random_mask(11, lens, keep=0.6)
    slopes = [0.5, 0.125]
    o, lse = O.decode_paged("f32", W.bits(p["q"]), W.bits(p["k_data"]), W.bits(p["v_data"]),
                            p["indices"], p["indptr"], p["last_page_len"], 0.7, alibi=slopes,
                            mask=W.pack_mask(keep))
    mpmath.mp.dps = 50
    qf = f64(p["q"])
    start = 0
    for b, L in enumerate(lens):
        kf, vf = f64(p["k_rows"][b]), f64(p["v_rows"][b])
        rows = [j for j in range(L) if keep[start + j]]
        start += L
        for h in range(group):
            xs = {}
            for j in rows:
                x = mpmath.mpf(0.7) * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(c)
                                                  for a, c in zip(qf[b, h], kf[j, 0]))
                xs[j] = mpmath.e ** (x + mpmath.mpf(slopes[h]) * (j - (L - 1)))
            z = mpmath.fsum(xs.values())
            for dd in range(d):
                ref = float(mpmath.fsum(xs[j] * mpmath.mpf(vf[j, 0, dd]) for j in rows) / z)
                assert abs(o[b, h, dd] - ref) <= 1e-13 * max(1.0, abs(ref))
            assert abs(lse[b, h] - float(mpmath.log(z))) <= 1e-13


def pin_seq_lens():
    """The oracle's L_b equals the row count the test scattered."""
    rng = np.random.default_rng(26)
    for page_size in (1, 5, 16):
        lens = [int(x) for x in rng.integers(0, 80, size=9)]
        empty = tuple(b for b, L in enumerate(lens) if L % page_size == 0)
        p = _paged_problem(rng, "bf16", lens, 1, 1, 64, page_size, empty_last_page=empty)
        assert list(O.seq_lens(page_size, p["indptr"], p["last_page_len"])) == lens


def pin_validate_table():
    ind = np.array([3, 0, 2], dtype=np.int32)
    ptr = np.array([0, 2, 3], dtype=np.int32)
    lpl = np.array([4, 1], dtype=np.int32)
    assert O.validate_table(2, 4, 4, ind, ptr, lpl) == "OK"
    assert O.validate_table(2, 4, 3, ind, ptr, lpl) == "BAD_INDEX"
    assert O.validate_table(2, 4, 4, np.array([3, -1, 2]), ptr, lpl) == "BAD_INDEX"
    assert O.validate_table(2, 4, 4, ind, np.array([1, 2, 3]), lpl) == "BAD_INDPTR"
    assert O.validate_table(2, 4, 4, ind, np.array([0, 3, 2]), lpl) == "BAD_INDPTR"
    assert O.validate_table(2, 4, 4, ind, np.array([0, 2, 4]), lpl) == "BAD_INDPTR"
    assert O.validate_table(2, 4, 4, ind, ptr, np.array([5, 1])) == "BAD_LAST_PAGE_LEN"
    assert O.validate_table(2, 4, 4, ind, ptr, np.array([4, -1])) == "BAD_LAST_PAGE_LEN"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
