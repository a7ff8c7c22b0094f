"""Helpers of the GPU tests: run the HIP library on a workload and compare
its outputs with the float64 oracle element by element."""
import sys

import numpy as np
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W

# tolerances (absolute): o per element type, lse always f32 against f64
O_TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3}
LSE_TOL = 1e-4
MANT_BITS = {"f32": 23, "f16": 10, "bf16": 7}


# relative error of the f32 arithmetic before o is rounded to a 16-bit type
# (scores, exponentials and the P.V sums in f32, bf16 probabilities split into
# two parts): well under 2^-12 of |o|
F32_MARGIN = 2.0 ** -12


def o_tolerance(dtype, o_ref):
    """Per-element bound on |o - o_ref|: the stated tolerance, or, for a 16-bit
    output where it is larger, half an ulp of the element type at |o_ref| (the
    error of rounding even the exact result to nearest) plus the f32 margin.
    That takes over at |o| >= 1 for bf16 (half an ulp on [1, 2) is 3.9e-3) and
    |o| >= 8 for f16; below, the bound is the stated tolerance itself, as for
    every output of the five configured workloads."""
    if dtype == "f32":
        return np.full(np.shape(o_ref), O_TOL[dtype])
    mag = np.maximum(np.abs(o_ref), np.finfo(np.float64).tiny)
    half_ulp = np.exp2(np.floor(np.log2(mag)) - MANT_BITS[dtype] - 1)
    return np.maximum(O_TOL[dtype], half_ulp + F32_MARGIN * mag)


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU (run with -m 'not gpu' on a CPU-only host)")
    fad.load_library()
    return torch.device("cuda:0")


def announce(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(p, dev):
    """Device copies of a problem's tensors (dict)."""
    if isinstance(p, W.PagedProblem):
        return dict(q=p.q.to(dev), k=p.k_data.to(dev), v=p.v_data.to(dev),
                    indices=p.indices.to(dev), indptr=p.indptr.to(dev),
                    lpl=p.last_page_len.to(dev))
    return dict(q=p.q.to(dev), k=p.k_cache.to(dev), v=p.v_cache.to(dev))


def run(p, d, o=None, lse=None, workspace=None):
    """The library's o and lse for problem p (device tensors d)."""
    if isinstance(p, W.PagedProblem):
        return fad.decode_paged(d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"],
                                p.scale, o=o, lse=lse, workspace=workspace, layout=p.layout)
    return fad.decode_contig(d["q"], d["k"], d["v"], p.valid_kv_len, p.scale, o=o, lse=lse,
                             workspace=workspace, layout=p.layout)


def oracle_of(p, samples=None):
    if isinstance(p, W.PagedProblem):
        return oracle.decode_paged(p.dtype, W.bits(p.q), W.bits(p.k_data), W.bits(p.v_data),
                                   p.indices.numpy(), p.indptr.numpy(),
                                   p.last_page_len.numpy(), p.scale, samples=samples,
                                   layout=p.layout)
    return oracle.decode_contig(p.dtype, W.bits(p.q), W.bits(p.k_cache), W.bits(p.v_cache),
                                p.valid_kv_len, p.scale, layout=p.layout)


def compare(dtype, o_gpu, lse_gpu, o_ref, lse_ref, what="", strict=False):
    """Element-by-element check; returns (max |do|, max |dlse|).  strict: the
    stated tolerance alone, with no one-ulp allowance for |o| >= 1."""
    go = o_gpu.float().cpu().numpy().astype(np.float64).reshape(o_ref.shape)
    gl = lse_gpu.cpu().numpy().astype(np.float64).reshape(lse_ref.shape)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(gl), empty), f"{what}: -inf lse pattern differs"
    assert np.all(go[empty] == 0.0), f"{what}: empty rows must give o = 0"
    assert np.all(np.isfinite(go)), f"{what}: non-finite o"
    diff = np.abs(go - o_ref)
    err_o = float(np.max(diff)) if go.size else 0.0
    fin = ~empty
    err_l = float(np.max(np.abs(gl[fin] - lse_ref[fin]))) if fin.any() else 0.0
    tol = O_TOL[dtype] if strict else o_tolerance(dtype, o_ref)
    worst = float(np.max(diff - tol)) if go.size else -1.0
    assert worst <= 0.0, f"{what}: max |o - oracle| = {err_o:.3e} exceeds its bound by {worst:.3e}"
    assert err_l <= LSE_TOL, f"{what}: max |lse - oracle| = {err_l:.3e} > {LSE_TOL}"
    return err_o, err_l


def compare_all(p, o, lse, what=None, strict=True, **oracle_kw):
    """Every (request, head) output of a call against the oracle's whole call
    (on every host core); returns (max |do|, max |dlse|)."""
    torch.cuda.synchronize()
    if isinstance(p, W.PagedProblem):
        ro, rl = oracle.decode_paged(p.dtype, W.bits(p.q), W.bits(p.k_data), W.bits(p.v_data),
                                     p.indices.numpy(), p.indptr.numpy(),
                                     p.last_page_len.numpy(), p.scale, layout=p.layout,
                                     **oracle_kw)
    else:
        ro, rl = oracle.decode_contig(p.dtype, W.bits(p.q), W.bits(p.k_cache),
                                      W.bits(p.v_cache), p.valid_kv_len, p.scale,
                                      layout=p.layout, **oracle_kw)
    return compare(p.dtype, o, lse, ro, rl, what or p.name, strict=strict)


def check_gather(p, dev):
    """The decode kernel's own loads of the page-table-resolved K and V rows
    (fa_debug_gather_paged runs its split units, LDS page staging and tile
    loads) against the oracle's gather, byte for byte."""
    import oracle as O
    lens = O.seq_lens(p.page_size, p.indptr.numpy(), p.last_page_len.numpy())
    rows = int(lens.sum())
    ws = fad.workspace_paged(p.batch, p.num_kv_heads, p.num_kv_heads, p.head_dim, p.page_size,
                             p.total_used_pages, dev)
    ind, ptr, lpl = p.indices.to(dev), p.indptr.to(dev), p.last_page_len.to(dev)
    for which, data in (("k", p.k_data), ("v", p.v_data)):
        out = torch.zeros((rows, p.num_kv_heads, p.head_dim), dtype=data.dtype, device=dev)
        dd = data.to(dev)
        fad.fa_debug_gather_paged(fad.DTYPE_CODES[p.dtype], p.batch, p.num_kv_heads,
                                  p.head_dim, p.page_size, p.num_total_pages,
                                  p.total_used_pages, dd, ind if p.total_used_pages else None,
                                  ptr, lpl, out, rows, ws, layout=p.layout)
        torch.cuda.synchronize()
        del dd
        want = O.gather_paged(p.dtype, W.bits(data), p.indices.numpy(), p.indptr.numpy(),
                              p.last_page_len.numpy(), layout=p.layout)
        got = W.bits(out.cpu())
        del out
        assert got.shape == want.shape, (p.name, which)
        same = got.view(np.uint8).reshape(rows, -1) == want.view(np.uint8).reshape(rows, -1)
        bad = np.nonzero(~same.all(axis=1))[0]
        assert bad.size == 0, (f"{p.name} {which}: {bad.size} of {rows} gathered rows differ, "
                               f"first at row {bad[0]}")
