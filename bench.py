"""Benchmark: batched paged bf16 GQA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c4|c5|c2|c1]

One step is one call of the library's decode entry point over the whole batch
(split plan, attention kernel and split merge), with inputs resident in HBM.
Prints one JSON line.  value = algorithmic bytes per call / wall time per call
(GB/s, 1e9 B/s), where the algorithmic bytes are the valid K and V rows, q, o,
lse and the page table, counted once each.  roofline.achieved divides the same
bytes by the attention kernel's own average duration, timed with HIP events the
library records on its stream during a second run of the same steps.
per_call gives p10 / median / p90 of single calls, each in its own event pair
(--flush: with the caches flushed before each call).  cpu_baseline runs the
float64 oracle on the host over the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import decode_attention_query_amd as fad  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) + µs/call, batched paged bf16 GQA decode"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def kept_rows(lens, window=0, keep=None):
    """K/V rows that take part, per request: the last `window` rows under a
    sliding window, and of those the ones a custom mask keeps."""
    lens = np.asarray(lens, dtype=np.int64)
    if keep is None:
        return np.minimum(lens, window) if window else lens
    out = np.zeros_like(lens)
    start = 0
    for b, L in enumerate(lens):
        lo = max(0, L - window) if window else 0
        out[b] = int(np.count_nonzero(keep[start + lo:start + L]))
        start += L
    return out


def algorithmic_bytes(p, window=0, keep=None):
    """K/V rows that take part (valid rows; under a sliding window the last
    `window` of each request; under a custom mask the kept ones) + q + o + lse
    + page table, each counted once."""
    es = W.ELEM_BYTES[p.dtype]
    if isinstance(p, W.ContigProblem):
        rows = int(kept_rows([p.valid_kv_len], window, keep)[0])
        kv = rows * p.num_kv_heads * p.head_dim * es * 2
        return kv + 2 * p.num_qo_heads * p.head_dim * es + 4 * p.num_qo_heads
    lens = kept_rows(p.kv_lens, window, keep)
    kv = int(lens.sum()) * p.num_kv_heads * p.head_dim * es * 2
    qo = 2 * p.batch * p.num_qo_heads * p.head_dim * es
    lse = 4 * p.batch * p.num_qo_heads
    table = 4 * (p.total_used_pages + 2 * p.batch + 1)
    return kv + qo + lse + table


def kernel_source_sha():
    """Hash of the HIP sources with comments and whitespace removed: a traffic
    figure holds only for the code it was taken on."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "decode_attention_query_amd", "csrc", "*"))):
        if f.endswith((".hpp", ".hip")):
            text = open(f).read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(os.path.basename(f).encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload_name):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary (profiles/hbm_traffic_<workload>.md), or None if there is none or
    the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("kernel_source_sha") == kernel_source_sha():
                return rec
    return None


def describe(p):
    if isinstance(p, W.ContigProblem):
        return {"workload": p.name, "layout": "contiguous", "kv_order": p.layout,
                "num_qo_heads": p.num_qo_heads,
                "num_kv_heads": p.num_kv_heads, "head_dim": p.head_dim,
                "max_kv_len": p.max_kv_len, "valid_kv_len": p.valid_kv_len}
    lens = np.asarray(p.kv_lens)
    return {"workload": p.name, "layout": "paged", "kv_order": p.layout, "batch": p.batch,
            "num_qo_heads": p.num_qo_heads, "num_kv_heads": p.num_kv_heads,
            "head_dim": p.head_dim, "page_size": p.page_size,
            "num_total_pages": p.num_total_pages, "total_used_pages": p.total_used_pages,
            "sum_kv_len": int(lens.sum()), "max_kv_len": int(lens.max())}


def cpu_baseline(p, nbytes, window=0, softcap=0.0, mask=None, min_seconds=2.0, max_runs=5):
    """The float64 oracle over the whole workload on this host's cores: whole
    calls repeated until min_seconds have passed (at most max_runs), median."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    times = []
    while len(times) < max_runs and (len(times) < 1 or sum(times) < min_seconds):
        t0 = time.perf_counter()
        if isinstance(p, W.ContigProblem):
            oracle.decode_contig(p.dtype, W.bits(p.q), W.bits(p.k_cache), W.bits(p.v_cache),
                                 p.valid_kv_len, p.scale, threads=threads, layout=p.layout,
                                 window=window, softcap=softcap, mask=mask)
        else:
            oracle.decode_paged(p.dtype, W.bits(p.q), W.bits(p.k_data), W.bits(p.v_data),
                                p.indices.numpy(), p.indptr.numpy(), p.last_page_len.numpy(),
                                p.scale, threads=threads, layout=p.layout, window=window,
                                softcap=softcap, mask=mask)
        times.append(time.perf_counter() - t0)
    dt = float(np.median(times))
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_call": round(dt, 3),
            "sample": f"the whole {p.name} call (every request and head), "
                      f"median of {len(times)} runs"}


def hbm_probe(dev, nbytes=4 << 30, reps=10):
    """Bandwidth context on this GPU: the library's read probe (the attention
    kernels' load shape over nbytes) and the runtime's device copy (reads and
    writes nbytes // 2 each; also the calibration kernel of the HBM counters)."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    half = buf[: nbytes // 2]
    dst = torch.empty_like(half)
    out = {}
    for name, fn, moved in (("read_probe", lambda: fad.fa_debug_read_probe(buf, sink), nbytes),
                            ("copy", lambda: dst.copy_(half), nbytes)):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name + "_GBps"] = round(moved * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del buf, dst
    torch.cuda.empty_cache()
    return out


def per_call_times(step, n, dev, flush):
    """p10 / median / p90 of single calls, each bracketed by its own event pair
    on the library's stream; with flush, a 512 MiB buffer is written before
    every call (outside the bracket) so the 256 MiB last-level cache and the
    L2s hold none of the call's inputs."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush else None
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in pairs:
        if flush:
            scratch.fill_(1)
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])
    out = {"p10_us": round(float(np.percentile(t, 10)), 2),
           "median_us": round(float(np.median(t)), 2),
           "p90_us": round(float(np.percentile(t, 90)), 2)}
    del scratch
    return out


def time_append(p, d, dev, steps, warmup):
    """The decode-time KV append of one new token per request, in place in the
    device store d: µs per call and algorithmic GB/s (new rows read and
    written, page-table words read)."""
    es = W.ELEM_BYTES[p.dtype]
    g = torch.Generator(device="cpu").manual_seed(5)
    shape = (p.batch, p.num_kv_heads, p.head_dim)
    k_new = torch.randn(shape, generator=g).to(W.TORCH_DTYPES[p.dtype]).to(dev)
    v_new = torch.randn(shape, generator=g).to(W.TORCH_DTYPES[p.dtype]).to(dev)

    def call():
        fad.append_paged(k_new, v_new, d["k"], d["v"], d["ind"], d["ptr"], d["lpl"],
                         layout=p.layout)

    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    nbytes = 2 * 2 * p.batch * p.num_kv_heads * p.head_dim * es + 4 * (3 * p.batch + 1)
    return {"us_per_call": round(us, 2), "GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
            "algorithmic_bytes_per_call": nbytes}


def time_merge(p, dev, parts, steps, warmup):
    """The standalone merge of `parts` split partials per output row of the
    workload (rows = B * Hq, f32 partials, o in the workload's element type):
    µs per call back to back and captured 16 calls to a graph, and GB/s over
    its algorithmic bytes (partials and their lse read once, o and lse
    written)."""
    es = W.ELEM_BYTES[p.dtype]
    batch = 1 if isinstance(p, W.ContigProblem) else p.batch
    rows, d = batch * p.num_qo_heads, p.head_dim
    g = torch.Generator(device="cpu").manual_seed(9)
    o_parts = torch.randn((parts, rows, d), generator=g).to(dev)
    lse_parts = (torch.randn((parts, rows), generator=g) * 3.0).to(dev)
    o = torch.empty((rows, d), dtype=W.TORCH_DTYPES[p.dtype], device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)

    def call():
        fad.fa_merge_states(fad.DTYPE_CODES[p.dtype], rows, parts, d, o_parts, lse_parts, o, lse)

    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / steps
    us_graph = graph_call_time(call, 16, max(1, steps // 16) + 4)
    nbytes = parts * rows * (d + 1) * 4 + rows * (d * es + 4)
    return {"parts": parts, "rows": rows, "us_per_call": round(us, 2),
            "graph_us_per_call": round(us_graph, 2),
            "GBps_graph": round(nbytes / (us_graph * 1e-6) / 1e9, 2),
            "algorithmic_bytes_per_call": nbytes}


def graph_call_time(step, n_calls, reps):
    """Mean µs per call when n_calls calls are captured in one HIP graph and
    the graph is replayed reps times (what a serving loop that captures its
    decode step sees)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_calls):
            step()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * n_calls)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c3", choices=sorted(W.FULL))
    ap.add_argument("--dtype", default=None, choices=["f32", "f16", "bf16"],
                    help="store the workload's shapes in this element type instead of its own")
    ap.add_argument("--qo-heads", type=int, default=None,
                    help="paged workloads: this many query heads over the same KV heads and "
                         "K/V (another GQA group size)")
    ap.add_argument("--layout", default="hnd", choices=["hnd", "nhd"],
                    help="K/V storage: heads-major (default) or token-major")
    ap.add_argument("--graph-calls", type=int, default=0,
                    help="also time N calls captured in one HIP graph (no host or launch "
                         "overhead between calls)")
    ap.add_argument("--append", action="store_true",
                    help="also time the decode-time KV append (paged workloads)")
    ap.add_argument("--merge-parts", type=int, default=0,
                    help="also time the standalone merge of this many split partials per "
                         "output row of the workload (0: off)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window: attend only each request's last W rows (0: all)")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="logits soft-cap c: scores -> c * tanh(x / c) (0: off)")
    ap.add_argument("--mask-keep", type=float, default=0.0,
                    help="custom mask: keep each K/V row with this probability (seeded; "
                         "0: no mask); bytes count the kept rows only")
    ap.add_argument("--rotate", type=int, default=1,
                    help="cycle the calls over this many distinct device copies of the K/V "
                         "store (paged), as successive layers of a model would, so no call "
                         "finds the previous call's rows in the 256 MB last-level cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe", action="store_true",
                    help="also measure the read probe and a device copy for context")
    ap.add_argument("--flush", action="store_true",
                    help="per-call timings with the caches flushed before each call")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requests and KV heads shard across GPUs with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fad.load_library()
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    if args.qo_heads is not None:
        if args.workload not in ("c3", "c4", "c5"):
            sys.exit("--qo-heads applies to the paged workloads c3, c4 and c5")
        p = W.FULL[args.workload](dtype=args.dtype, qo_heads=args.qo_heads)
    else:
        p = W.FULL[args.workload](dtype=args.dtype)
    if args.layout == "nhd":
        p = W.token_major(p)
    print(f"[bench] generated {p.name} in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
          flush=True)
    keep = mask = dev_mask = None
    if args.mask_keep > 0.0:
        lens = [p.valid_kv_len] if isinstance(p, W.ContigProblem) else p.kv_lens
        keep = W.random_mask(4242, lens, keep=args.mask_keep)
        mask = W.pack_mask(keep)
        dev_mask = torch.from_numpy(mask).to(dev)
    nbytes = algorithmic_bytes(p, args.window, keep)

    if isinstance(p, W.ContigProblem):
        q, k, v = p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty(p.num_qo_heads, dtype=torch.float32, device=dev)
        ws = fad.workspace_paged(1, p.num_qo_heads, p.num_kv_heads, p.head_dim, p.max_kv_len, 1,
                                 dev)

        def step():
            fad.decode_contig(q, k, v, p.valid_kv_len, p.scale, o=o, lse=lse, workspace=ws,
                              layout=p.layout, window=args.window, softcap=args.softcap,
                              mask=dev_mask)
    else:
        q, k, v = p.q.to(dev), p.k_data.to(dev), p.v_data.to(dev)
        ind, ptr, lpl = p.indices.to(dev), p.indptr.to(dev), p.last_page_len.to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((p.batch, p.num_qo_heads), dtype=torch.float32, device=dev)
        ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                                 p.page_size, p.total_used_pages, dev)
        stores = [(k, v)] + [(k.clone(), v.clone()) for _ in range(args.rotate - 1)]
        turn = [0]

        def step():
            ks, vs = stores[turn[0] % len(stores)]
            turn[0] += 1
            fad.decode_paged(q, ks, vs, ind, ptr, lpl, p.scale, o=o, lse=lse, workspace=ws,
                             layout=p.layout, window=args.window, softcap=args.softcap,
                             mask=dev_mask)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} calls)", file=sys.stderr, flush=True)

    # timed region: K whole calls, nothing else on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    # the same K calls again with the library's HIP events around its attention
    # kernel (the event markers themselves add a little to each call, so this
    # region is kept out of `value`)
    fad.fa_debug_timing_enable(1)
    fad.fa_debug_timing_read()  # reset
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    main_ms, call_ms, calls = fad.fa_debug_timing_read()
    fad.fa_debug_timing_enable(0)
    per_call = per_call_times(step, args.steps, dev, flush=False)
    per_call_cold = per_call_times(step, args.steps, dev, flush=True) if args.flush else None
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    kernel_ms = main_ms / max(calls, 1)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    chunk, bound, gt, kind = fad.fa_debug_plan(fad.DTYPE_CODES[p.dtype],
                                               getattr(p, "batch", 1), p.num_qo_heads,
                                               p.num_kv_heads, p.head_dim,
                                               getattr(p, "page_size", getattr(p, "max_kv_len", 1)),
                                               getattr(p, "total_used_pages", 1))
    print(f"[bench] {args.steps} calls: {ms_per_step * 1e3:.1f} us/call, attention kernel "
          f"{kernel_ms * 1e3:.1f} us (call with event markers {call_ms / max(calls, 1) * 1e3:.1f} "
          f"us), {value:.0f} GB/s call, {achieved:.0f} GB/s kernel", file=sys.stderr, flush=True)

    # the committed counter figures were taken on plain calls (no window, cap or mask)
    plain = not (args.window or args.softcap or mask is not None)
    traffic = committed_traffic(p.name) if plain else None
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) values, seeded page tables; no dataset)",
        "config": {**describe(p), "window": args.window, "softcap": args.softcap,
                   "mask_keep": args.mask_keep,
                   "kv_copies_rotated": args.rotate,
                   "algorithmic_bytes_per_call": int(nbytes),
                   "chunk_rows": chunk, "heads_per_workgroup": gt,
                   "attention_kernel": "mfma" if kind == 1 else f"kind {kind}"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "traffic_over_algorithmic":
                         traffic["traffic_over_algorithmic"] if traffic else None,
                     "kernel_us": round(kernel_ms * 1e3, 2),
                     "kernel": "decode attention with fused split merge (fa::decode_*_kernel)"},
    }
    if args.append and not isinstance(p, W.ContigProblem):
        line["append"] = time_append(p, {"k": k, "v": v, "ind": ind, "ptr": ptr, "lpl": lpl},
                                     dev, args.steps, args.warmup)
    if args.merge_parts > 0:
        line["merge"] = time_merge(p, dev, args.merge_parts, args.steps, args.warmup)
    if args.graph_calls > 0:
        us = graph_call_time(step, args.graph_calls, max(1, args.steps // args.graph_calls) + 4)
        line["graph_per_call"] = {"calls_per_graph": args.graph_calls, "us_per_call": round(us, 2),
                                  "GBps": round(nbytes / (us * 1e-6) / 1e9, 2)}
    line["per_call"] = per_call
    if per_call_cold:
        line["per_call_flushed"] = per_call_cold
    if args.probe:
        line["hbm_probe"] = hbm_probe(dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(p, nbytes, args.window, args.softcap, mask)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
