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


def o_tolerance(dtype, o_ref):
    """Per-element bound on |o - o_ref|: the stated tolerance, or one unit in
    the last place of the element type at |o_ref| where that is larger.  Even
    the correctly rounded exact result is half an ulp away from o_ref, and for
    |o| >= 1 half a bf16 ulp already exceeds 4e-3; below 1 (every configured
    workload) the bound is the stated tolerance itself."""
    mag = np.maximum(np.abs(o_ref), np.finfo(np.float64).tiny)
    ulp = np.exp2(np.floor(np.log2(mag)) - MANT_BITS[dtype])
    return np.maximum(O_TOL[dtype], ulp)


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


def sample_pairs(p, n, rng):
    """(b, h) pairs: every head of the first two requests and of the longest one,
    then random pairs, n in total at least."""
    lens = oracle.seq_lens(p.page_size, p.indptr.numpy(), p.last_page_len.numpy())
    picks = []
    for b in sorted({0, min(1, p.batch - 1), int(np.argmax(lens)), p.batch - 1}):
        picks += [(b, h) for h in range(p.num_qo_heads)]
    while len(picks) < n:
        picks.append((int(rng.integers(p.batch)), int(rng.integers(p.num_qo_heads))))
    return np.array(picks, dtype=np.int32)
