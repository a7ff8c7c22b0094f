"""Benchmark: batched paged bf16 GQA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3|c4|c5|c2|c1]

One step is one call of the library's decode entry point over the whole batch
(one launch of the attention kernel, which also finds its split units and
merges them), with inputs resident in HBM.  Prints one JSON line.

value = algorithmic bytes per call / time per call (GB/s, 1e9 B/s) over K
back-to-back calls bracketed by HIP events on the stream the kernel is
launched on; the algorithmic bytes are the valid K and V rows, q, o, lse and
the page table, counted once each.  Since a call is one kernel launch, that
bracket also gives the kernel's average launch period (roofline.kernel_us,
which includes the gap between back-to-back launches, so it never exceeds the
call); roofline.trace_kernel_us is the kernel's own mean duration from the
committed rocprofv3 trace of the same command while the kernel sources still
hash as they did then.

Also in the line, by default: per_call (p10 / median / p90 of single calls,
each in its own event pair) unflushed and with the caches flushed before each
call (a 512 MiB write); `rotated`, the calls cycled over 4 device copies of
the K/V store so no call finds the previous call's rows in the last-level
cache; hbm_probe (the library's read probe and a device copy); for the
default workload, a sub-record for the second primary workload (C4); and
cpu_baseline, the float64 oracle on this host's cores.
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


def cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(p, nbytes, window=0, softcap=0.0, mask=None, min_seconds=10.0, max_runs=200):
    """The float64 oracle, as it stands, over the whole workload on this host's
    cores: whole calls repeated until min_seconds of wall time have passed (a
    bounded sample of about 10 s), median per call."""
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
            "kind": "oracle", "cpu_model": cpu_model(), "seconds_per_call": round(dt, 3),
            "sample": f"whole {p.name} calls (every request and head) repeated for "
                      f"{sum(times):.1f} s: median of {len(times)} calls"}


def trace_record(workload_name):
    """The attention kernel's mean duration from a committed rocprofv3 kernel
    trace of this workload (profiles/*_kernel_trace.md, line `trace-record:`),
    or None if there is none or the kernel sources changed since."""
    import glob
    sha = kernel_source_sha()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_kernel_trace.md"))):
        for line in open(path):
            if line.startswith("trace-record:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("workload") == workload_name and rec.get("kernel_source_sha") == sha:
                    return dict(rec, file=os.path.relpath(path, ROOT))
    return None


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


def timed_us(step, steps):
    """Mean µs per call of `steps` back-to-back calls, bracketed by HIP events on
    the current stream (the stream the library launches on)."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def graph_flushed_time(step, dev, n_calls, reps):
    """Mean µs per call inside a HIP graph with the caches flushed before every
    call: a graph of n_calls (512 MiB flush, call) pairs minus a graph of the
    n_calls flushes alone, per call."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    both = graph_call_time(lambda: (scratch.fill_(1), step()), n_calls, reps)
    flush = graph_call_time(lambda: scratch.fill_(1), n_calls, reps)
    del scratch
    return both - flush


class Bench:
    """One workload on the device: its inputs, a step (one library call), and
    the measurements of the line."""

    def __init__(self, p, dev, args, mask=None):
        self.p, self.dev, self.args = p, dev, args
        self.mask = mask
        if isinstance(p, W.ContigProblem):
            self.q, self.k, self.v = p.q.to(dev), p.k_cache.to(dev), p.v_cache.to(dev)
            self.lse = torch.empty(p.num_qo_heads, dtype=torch.float32, device=dev)
            self.ws = fad.workspace_paged(1, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                                          p.max_kv_len, 1, dev)
        else:
            self.q, self.k, self.v = p.q.to(dev), p.k_data.to(dev), p.v_data.to(dev)
            self.ind, self.ptr = p.indices.to(dev), p.indptr.to(dev)
            self.lpl = p.last_page_len.to(dev)
            self.lse = torch.empty((p.batch, p.num_qo_heads), dtype=torch.float32, device=dev)
            self.ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                                          p.page_size, p.total_used_pages, dev)
        self.o = torch.empty_like(self.q)
        self.stores = [(self.k, self.v)]
        self.turn = 0

    def call(self, k, v):
        p, a = self.p, self.args
        if isinstance(p, W.ContigProblem):
            fad.decode_contig(self.q, k, v, p.valid_kv_len, p.scale, o=self.o, lse=self.lse,
                              workspace=self.ws, layout=p.layout, window=a.window,
                              softcap=a.softcap, mask=self.mask)
        else:
            fad.decode_paged(self.q, k, v, self.ind, self.ptr, self.lpl, p.scale, o=self.o,
                             lse=self.lse, workspace=self.ws, layout=p.layout, window=a.window,
                             softcap=a.softcap, mask=self.mask)

    def step(self):
        """One call on the resident store."""
        self.call(self.k, self.v)

    def rotated_step(self):
        """One call on the next of the store's copies."""
        k, v = self.stores[self.turn % len(self.stores)]
        self.turn += 1
        self.call(k, v)

    def rotated(self, copies, steps, nbytes):
        """Back-to-back calls cycling over `copies` device copies of the K/V
        store, so no call finds the previous call's rows in the last-level
        cache (as successive layers of a model would)."""
        self.stores = [(self.k, self.v)] + [(self.k.clone(), self.v.clone())
                                            for _ in range(copies - 1)]
        for _ in range(copies):
            self.rotated_step()
        us = timed_us(self.rotated_step, steps)
        self.stores = [(self.k, self.v)]
        torch.cuda.empty_cache()
        return {"kv_copies": copies, "us_per_call": round(us, 2),
                "GBps": round(nbytes / (us * 1e-6) / 1e9, 2),
                "pct_of_hbm_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}


def measure(b, nbytes, steps, warmup, flush, rotate):
    """The headline measurement of a workload (warm-up, then `steps` timed calls)
    and its per-call, flushed and rotated figures."""
    for _ in range(warmup):
        b.step()
    torch.cuda.synchronize()
    us = timed_us(b.step, steps)
    out = {"us_per_call": us, "GBps": nbytes / (us * 1e-6) / 1e9,
           "per_call": per_call_times(b.step, steps, b.dev, flush=False)}
    if flush:
        out["per_call_flushed"] = per_call_times(b.step, steps, b.dev, flush=True)
    if rotate > 1 and not isinstance(b.p, W.ContigProblem):
        out["rotated"] = b.rotated(rotate, steps, nbytes)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the first ~50 calls of a process run 1-3% slower than later ones (the
    # clocks settle under load), so the default warm-up covers them
    ap.add_argument("--warmup", type=int, default=100)
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
                         "overhead between calls), plain and with the caches flushed")
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
    ap.add_argument("--mask-run", type=int, default=0,
                    help="custom mask in runs of this many rows kept or dropped together "
                         "(a block-sparse mask; 0: rows drawn one by one)")
    ap.add_argument("--rotate", type=int, default=4,
                    help="paged workloads: also time calls cycling over this many device "
                         "copies of the K/V store (1: off)")
    ap.add_argument("--no-flush", action="store_true",
                    help="leave out the per-call figures with the caches flushed")
    ap.add_argument("--no-probe", action="store_true",
                    help="leave out the read probe and device copy")
    ap.add_argument("--no-second", action="store_true",
                    help="leave out the second primary workload's sub-record")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requests and KV heads would shard across GPUs with no exchange)",
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
        keep = W.random_mask(4242, lens, keep=args.mask_keep,
                             blocks=args.mask_run if args.mask_run > 0 else False)
        mask = W.pack_mask(keep)
        dev_mask = torch.from_numpy(mask).to(dev)
    nbytes = algorithmic_bytes(p, args.window, keep)
    b = Bench(p, dev, args, dev_mask)

    # timed region: K whole calls (one attention-kernel launch each), nothing
    # else on the stream, between HIP events on that stream
    m = measure(b, nbytes, args.steps, args.warmup, not args.no_flush, args.rotate)
    us = m["us_per_call"]
    ms_per_step = us * 1e-3
    value = m["GBps"]
    chunk, bound, gt, kind = fad.fa_debug_plan(fad.DTYPE_CODES[p.dtype],
                                               getattr(p, "batch", 1), p.num_qo_heads,
                                               p.num_kv_heads, p.head_dim,
                                               getattr(p, "page_size", getattr(p, "max_kv_len", 1)),
                                               getattr(p, "total_used_pages", 1))
    print(f"[bench] {args.steps} calls: {us:.1f} us/call, {value:.0f} GB/s "
          f"({100.0 * value / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})", file=sys.stderr,
          flush=True)

    # the committed counter and trace figures were taken on plain calls
    plain = not (args.window or args.softcap or mask is not None)
    traffic = committed_traffic(p.name) if plain else None
    trace = trace_record(p.name) if plain else None
    roofline = {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4),
                "traffic": traffic["traffic_bytes"] if traffic else None,
                "traffic_over_algorithmic":
                    traffic["traffic_over_algorithmic"] if traffic else None,
                "kernel_us": round(us, 2),
                "kernel_us_source": "HIP events on the launch stream around the timed "
                                    "calls, one kernel launch per call (launch period)",
                "trace_kernel_us": trace["mean_us"] if trace else None,
                "trace_frac": round(nbytes / (trace["mean_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                if trace else None,
                "kernel": "decode attention with fused split merge (fa::decode_mfma_kernel)"}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(us, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) values, seeded page tables; no dataset)",
        "config": {**describe(p), "window": args.window, "softcap": args.softcap,
                   "mask_keep": args.mask_keep, "mask_run": args.mask_run,
                   "algorithmic_bytes_per_call": int(nbytes),
                   "chunk_rows": chunk, "heads_per_workgroup": gt,
                   "attention_kernel": "mfma" if kind == 1 else f"kind {kind}"},
        "roofline": roofline,
        "per_call": m["per_call"],
    }
    for key in ("per_call_flushed", "rotated"):
        if key in m:
            line[key] = m[key]
    if args.append and not isinstance(p, W.ContigProblem):
        line["append"] = time_append(p, {"k": b.k, "v": b.v, "ind": b.ind, "ptr": b.ptr,
                                         "lpl": b.lpl}, dev, args.steps, args.warmup)
    if args.merge_parts > 0:
        line["merge"] = time_merge(p, dev, args.merge_parts, args.steps, args.warmup)
    if args.graph_calls > 0:
        reps = max(1, args.steps // args.graph_calls) + 4
        g_us = graph_call_time(b.step, args.graph_calls, reps)
        line["graph_per_call"] = {"calls_per_graph": args.graph_calls, "us_per_call": round(g_us, 2),
                                  "GBps": round(nbytes / (g_us * 1e-6) / 1e9, 2)}
        if not args.no_flush:
            f_us = graph_flushed_time(b.step, dev, args.graph_calls, reps)
            line["graph_per_call_flushed"] = {
                "calls_per_graph": args.graph_calls, "us_per_call": round(f_us, 2),
                "GBps": round(nbytes / (f_us * 1e-6) / 1e9, 2),
                "method": "graph of (512 MiB flush, call) pairs minus a graph of the flushes"}
    second = None
    if args.workload == "c3" and not args.no_second and args.qo_heads is None and \
            args.dtype is None and args.layout == "hnd" and plain:
        del b
        torch.cuda.empty_cache()
        print("[bench] second primary workload: c4", file=sys.stderr, flush=True)
        p2 = W.FULL["c4"]()
        n2 = algorithmic_bytes(p2)
        b2 = Bench(p2, dev, args)
        m2 = measure(b2, n2, args.steps, args.warmup, not args.no_flush, args.rotate)
        t2 = trace_record(p2.name)
        second = {"config": describe(p2), "algorithmic_bytes_per_call": int(n2),
                  "us_per_call": round(m2["us_per_call"], 2), "GBps": round(m2["GBps"], 2),
                  "pct_of_hbm_peak": round(100.0 * m2["GBps"] / HBM_PEAK_GBS, 2),
                  "trace_kernel_us": t2["mean_us"] if t2 else None,
                  **{k: m2[k] for k in ("per_call", "per_call_flushed", "rotated") if k in m2}}
        line["second_primary"] = second
        print(f"[bench] c4: {m2['us_per_call']:.1f} us/call, {m2['GBps']:.0f} GB/s",
              file=sys.stderr, flush=True)
        del b2, p2
        torch.cuda.empty_cache()
    if not args.no_probe:
        line["hbm_probe"] = hbm_probe(dev)
    if not args.no_cpu_baseline:
        print("[bench] timing the float64 oracle on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(p, nbytes, args.window, args.softcap, mask)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
