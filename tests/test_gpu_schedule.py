"""The split-unit schedule the decode kernels compute on the device, and the
merge counters that ride on it.

The schedule is checked exactly (integers) against a plain restatement here:
every split unit of every request appears once, full-length units first in
request order, then each request's last (shorter) unit by length class,
longest class first, request order inside a class, then the unused work
indices.  Request lengths follow the page-table definition (the
baracuda-kernels batch_paged_decode page, module doc "Layout").
"""
import zlib

import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import workloads as W
from gpu_util import announce, compare, device, oracle_of, run, to_dev

pytestmark = pytest.mark.gpu

N_CLASSES = 16


@pytest.fixture(scope="module")
def dev():
    return device()


def expected_schedule(lens, page_size, chunk, units_bound):
    lens = [int(x) for x in lens]
    B = len(lens)
    full = [L // chunk for L in lens]
    part = [1 if (L % chunk or L == 0) else 0 for L in lens]
    units = [f + q for f, q in zip(full, part)]
    u0 = np.concatenate([[0], np.cumsum(units)])[:-1]
    row0 = np.concatenate([[0], np.cumsum(lens)])[:-1]
    n_pages, _ = W.pages_for_lens(lens, page_size)
    base = np.concatenate([[0], np.cumsum(n_pages)])[:-1]
    order = [(b, c) for b in range(B) for c in range(full[b])]
    width = chunk // N_CLASSES
    last = [b for b in range(B) if part[b]]
    last.sort(key=lambda b: (-min((lens[b] - full[b] * chunk) // width, N_CLASSES - 1), b))
    order += [(b, full[b]) for b in last]
    assert len(order) <= units_bound
    rows = [[b, c, units[b], lens[b], int(u0[b]), int(base[b]), int(row0[b]) & 0xffffffff,
             int(row0[b]) >> 32] for b, c in order]
    rows += [[-1, 0, 0, 0, 0, 0, 0, 0]] * (units_bound - len(order))
    out = np.array(rows, dtype=np.int64)
    out[:, 6] = out[:, 6].astype(np.uint32).astype(np.int32)  # low word as int32 bits
    return out.astype(np.int32)


def _lens_case(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    if name == "c3-like":      # B=64, L ~ U[512, 8192]
        return 16, rng.integers(512, 8193, 64), (32, 8, 128)
    if name == "c4-like":      # B=32, all 32768
        return 32, np.full(32, 32768), (64, 8, 128)
    if name == "skew":         # B=128, mostly short, a few empty, one very long
        lens = rng.integers(1, 600, 128)
        lens[rng.integers(0, 128, 6)] = 0
        lens[7] = 42110
        return 16, lens, (16, 4, 256)
    if name == "many":         # several scheduling rounds of 1024 requests
        lens = rng.integers(0, 3000, 3000)
        lens[rng.integers(0, 3000, 300)] = 0
        return 16, lens, (32, 8, 128)
    if name == "round-edge":   # 1025 requests: one past a round
        return 7, rng.integers(0, 5000, 1025), (8, 2, 64)
    if name == "one-empty":
        return 16, np.array([0]), (8, 1, 128)
    if name == "exact-chunks":  # lengths that are whole multiples of the split
        return 16, np.array([256 * 16, 0, 256 * 32, 1, 4096]), (32, 8, 128)
    raise KeyError(name)


@pytest.mark.parametrize("name", ["c3-like", "c4-like", "skew", "many", "round-edge",
                                  "one-empty", "exact-chunks"])
def test_schedule_matches_definition(dev, name):
    page_size, lens, (hq, hkv, d) = _lens_case(name)
    n_pages, lpl = W.pages_for_lens(lens, page_size)
    indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    used = int(indptr[-1])
    chunk, bound, _, _ = fad.fa_debug_plan(fad.FA_DTYPE_BF16, len(lens), hq, hkv, d, page_size,
                                           used)
    announce(f"schedule {name}: B={len(lens)} chunk={chunk} bound={bound}")
    out = torch.full((bound * 8,), 12345, dtype=torch.int32, device=dev)
    fad.fa_debug_schedule(fad.FA_DTYPE_BF16, len(lens), hq, hkv, d, page_size, used,
                          torch.from_numpy(indptr).to(dev),
                          torch.from_numpy(lpl.astype(np.int32)).to(dev), out)
    got = out.cpu().numpy().reshape(bound, 8)
    want = expected_schedule(lens, page_size, chunk, bound)
    bad = np.nonzero(np.any(got != want, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} work indices differ; first {bad[0]}: "
                           f"got {got[bad[0]].tolist()} want {want[bad[0]].tolist()}")


def test_schedule_rejects_short_output(dev):
    lens = np.array([100, 200])
    n_pages, lpl = W.pages_for_lens(lens, 16)
    indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    _, bound, _, _ = fad.fa_debug_plan(fad.FA_DTYPE_BF16, 2, 8, 2, 128, 16, int(indptr[-1]))
    out = torch.zeros(bound * 8 - 1, dtype=torch.int32, device=dev)
    with pytest.raises(fad.FaError) as e:
        fad.fa_debug_schedule(fad.FA_DTYPE_BF16, 2, 8, 2, 128, 16, int(indptr[-1]),
                              torch.from_numpy(indptr).to(dev),
                              torch.from_numpy(lpl.astype(np.int32)).to(dev), out)
    assert e.value.status == fad.FA_ERR_WORKSPACE_TOO_SMALL


# ------------------------------------------------------- merge counters

def _split_problem(dtype="bf16", seed=77):
    """Requests long enough to split into several units, plus short and empty ones."""
    lens = np.array([9000, 0, 17, 4096, 25000, 300, 12345, 1])
    return W.make_paged("split-mix", dtype, len(lens), 16, 4, 128, 16, seed, lens=lens,
                        pool_slack=0.1)


def _launch_size(p):
    _, bound, gt, _ = fad.fa_debug_plan(fad.DTYPE_CODES[p.dtype], p.batch, p.num_qo_heads,
                                        p.num_kv_heads, p.head_dim, p.page_size,
                                        p.total_used_pages)
    return bound * p.num_kv_heads * -(-(p.num_qo_heads // p.num_kv_heads) // gt)


def test_garbage_workspace(dev):
    """The workspace needs no clearing: random bytes in it change nothing,
    neither in the arrival counters nor in the counter that hands out work
    items past the first resident round (two workgroups per compute unit)."""
    p = _split_problem()
    assert _launch_size(p) > 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    d = to_dev(p, dev)
    ref_o, ref_l = run(p, d)
    ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                             p.page_size, p.total_used_pages, dev)
    for trial in range(3):
        g = torch.Generator(device="cpu").manual_seed(trial)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=g))
        if trial == 2:
            ws.fill_(255)
        o, l = run(p, d, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"trial {trial}"
    ro, rl = oracle_of(p)
    compare(p.dtype, ref_o, ref_l, ro, rl, p.name)


def test_workspace_shared_across_shapes(dev):
    """One workspace buffer serving calls of different shapes in turn: each
    call finds counters that the other shape left as partial results or at
    rest at other offsets, and still matches a call on a fresh workspace."""
    pa = _split_problem(seed=81)
    pb = W.make_paged("split-mix-b", "f16", 5, 8, 2, 64, 16, 82,
                      lens=np.array([20000, 3, 0, 7777, 16384]), pool_slack=0.1)
    da, db = to_dev(pa, dev), to_dev(pb, dev)
    refs = [run(pa, da), run(pb, db)]
    torch.cuda.synchronize()
    sizes = [fad.workspace_paged(q.batch, q.num_qo_heads, q.num_kv_heads, q.head_dim,
                                 q.page_size, q.total_used_pages, dev).numel() for q in (pa, pb)]
    ws = torch.empty(max(sizes), dtype=torch.uint8, device=dev)
    for step, (q, d, ref) in enumerate([(pa, da, refs[0]), (pb, db, refs[1]), (pa, da, refs[0]),
                                        (pb, db, refs[1]), (pb, db, refs[1])]):
        o, l = run(q, d, workspace=ws[:sizes[0 if q is pa else 1]])
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(l, ref[1]), f"step {step} ({q.name})"
    for q, ref in ((pa, refs[0]), (pb, refs[1])):
        ro, rl = oracle_of(q)
        compare(q.dtype, ref[0], ref[1], ro, rl, q.name)


@pytest.mark.parametrize("qo_heads", [16, 64], ids=["G4", "G32-two-blocks"])
def test_graph_replay(dev, qo_heads):
    """A captured call replays correctly again and again (each merge leaves its
    arrival counter at rest), with eager work in between; G = 32 takes the
    two-block workgroups."""
    p = _split_problem(seed=78)
    if qo_heads != p.num_qo_heads:
        lens = _lens_of(p)
        p = W.make_paged("split-mix-g32", p.dtype, p.batch, qo_heads, 2, 128, 16, 78,
                         lens=lens, pool_slack=0.1)
    d = to_dev(p, dev)
    ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                             p.page_size, p.total_used_pages, dev)
    o = torch.empty_like(d["q"])
    lse = torch.empty((p.batch, p.num_qo_heads), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(p, d, o=o, lse=lse, workspace=ws)  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(p, d, o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    q0 = d["q"].clone()
    for r in range(4):
        # new query values in the captured buffer; eager reference on its own workspace
        d["q"].copy_(q0 * (1.0 + 0.25 * r))
        eo, el = run(p, d)
        torch.cuda.synchronize()
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(lse, el), f"replay {r}"
    announce("graph replays match eager")


def _lens_of(p):
    return np.asarray(p.kv_lens, dtype=np.int64)


def test_graph_replay_merge(dev):
    """The separate merge captured in a graph: every replay, with new partials
    copied in and eager work in between, equals the eager call bit for bit."""
    rng = np.random.default_rng(12)
    s_, rows, d = 6, 300, 128
    o_p = torch.from_numpy(rng.standard_normal((s_, rows, d)).astype(np.float32)).to(dev)
    l_p = torch.from_numpy((rng.standard_normal((s_, rows)) * 3).astype(np.float32)).to(dev)
    l_p[2, ::7] = -float("inf")
    o = torch.empty((rows, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        fad.merge_states(o_p, l_p, o=o, lse=lse)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fad.merge_states(o_p, l_p, o=o, lse=lse)
    torch.cuda.synchronize()
    o0, l0 = o_p.clone(), l_p.clone()
    for r in range(4):
        o_p.copy_(o0 * (1.0 - 0.2 * r))
        l_p.copy_(l0 + 0.5 * r)
        eo, el = fad.merge_states(o_p, l_p, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        o.zero_()
        lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), eo.view(torch.int16)), f"replay {r}"
        assert torch.equal(lse.view(torch.int32), el.view(torch.int32)), f"replay {r}"
    announce("merge graph replays match eager")


def test_read_probe_runs(dev):
    """The bandwidth probe reads the whole buffer and leaves the sink alone."""
    buf = torch.full((1 << 20,), 3, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    fad.fa_debug_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    with pytest.raises(fad.FaError):
        fad.fa_debug_read_probe(buf[:100], sink)


@pytest.mark.parametrize("dtype,d,hq,length", [("f32", 64, 8, 100_000),
                                               ("bf16", 64, 16, 200_000),
                                               ("f16", 128, 4, 20_000)])
def test_many_unit_merge(dev, dtype, d, hq, length):
    """Requests split into hundreds of units: the merge reads the lse in several
    lane rounds and stages its weights in LDS in several chunks."""
    p = W.make_contig("long", dtype, hq, 1, d, length + 7, length, seed=length)
    chunk, bound, _, _ = fad.fa_debug_plan(fad.DTYPE_CODES[dtype], 1, hq, 1, d, length + 7, 1)
    announce(f"many-unit merge {dtype} D{d} Hq{hq} L{length}: chunk {chunk}, "
             f"{-(-length // chunk)} units")
    assert -(-length // chunk) > 64
    o, lse = run(p, to_dev(p, dev))
    torch.cuda.synchronize()
    ro, rl = oracle_of(p)
    compare(dtype, o, lse, ro, rl, p.name)


# ------------------------------------------------ tables that break the contract

def _broken_tables(T, batch_hint=None):
    """(name, indptr, last_page_len offsets) of page tables that break the
    contract: overlapping ranges, a non-monotone indptr, values outside
    [0, T]."""
    return [
        ("overlap", np.array([0, T, 0, T, 0, T], dtype=np.int64)),
        ("non-monotone", np.array([0, T // 2, T // 5, T, T // 3, T - 1, 2], dtype=np.int64)),
        ("out-of-range", np.array([-40, 10, T + 50, 1 << 30, -(1 << 30), T], dtype=np.int64)),
    ]


def _envelope(indptr, T):
    """Page range of each request as the schedule defines it for any table:
    request b owns [s_b, s_{b+1}) with s_b = max over k <= b of
    clamp(indptr[k], 0, T)."""
    c = np.clip(indptr, 0, T)
    s = np.maximum.accumulate(c)
    return s[:-1], s[1:] - s[:-1]


@pytest.mark.parametrize("which", [0, 1, 2], ids=["overlap", "non-monotone", "out-of-range"])
def test_schedule_broken_table(dev, which):
    """Whatever the table holds, every split unit of every request appears once
    below units_bound and no request's partial slots reach past it; page
    ranges follow the running maximum of the clamped indptr."""
    page_size, hq, hkv, d, T = 16, 32, 8, 128, 3000
    name, indptr = _broken_tables(T)[which]
    batch = indptr.size - 1
    rng = np.random.default_rng(which)
    lpl = rng.integers(-3, page_size + 5, batch)
    chunk, bound, _, _ = fad.fa_debug_plan(fad.FA_DTYPE_BF16, batch, hq, hkv, d, page_size, T)
    out = torch.full((bound * 8,), 12345, dtype=torch.int32, device=dev)
    fad.fa_debug_schedule(fad.FA_DTYPE_BF16, batch, hq, hkv, d, page_size, T,
                          torch.from_numpy(indptr.astype(np.int32)).to(dev),
                          torch.from_numpy(lpl.astype(np.int32)).to(dev), out)
    got = out.cpu().numpy().reshape(bound, 8)
    starts, n = _envelope(indptr, T)
    lens = np.where(n > 0, (n - 1) * page_size + np.clip(lpl, 0, page_size), 0)
    announce(f"broken table {name}: lens {lens.tolist()}, chunk {chunk}, bound {bound}")
    assert int(n.sum()) <= T
    seen = {}
    for row in got:
        b = int(row[0])
        if b < 0:
            continue
        assert row[3] == lens[b] and row[5] == starts[b], (name, row.tolist())
        assert row[4] + row[2] <= bound, (name, row.tolist())
        seen.setdefault(b, []).append(int(row[1]))
    for b in range(batch):
        units = max(1, -(-int(lens[b]) // chunk))
        assert sorted(seen.get(b, [])) == list(range(units)), (name, b)


def test_valid_call_after_broken_table(dev):
    """A call with a broken table (overlapping page ranges of long requests)
    stays inside its buffers and leaves no counter part counted, so the next,
    valid call on the same workspace equals a call on a fresh one bit for bit
    and matches the oracle."""
    p = _split_problem(seed=83)
    d = to_dev(p, dev)
    ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                             p.page_size, p.total_used_pages, dev)
    T = p.total_used_pages
    for name, ptr in _broken_tables(T):
        bad = ptr[:p.batch + 1] if ptr.size >= p.batch + 1 else \
            np.concatenate([ptr, np.full(p.batch + 1 - ptr.size, T)])
        announce(f"broken table {name}: indptr {bad.tolist()}")
        bad_d = dict(d, indptr=torch.from_numpy(bad.astype(np.int32)).to(dev),
                     lpl=torch.from_numpy(np.full(p.batch, p.page_size + 7,
                                                  dtype=np.int32)).to(dev))
        run(p, bad_d, workspace=ws)
        torch.cuda.synchronize()
        assert fad.fa_debug_counters_in_use(p.batch, p.num_qo_heads, p.num_kv_heads,
                                            p.head_dim, p.page_size, T, ws) == 0, name
        o, lse = run(p, d, workspace=ws)
        ref_o, ref_l = run(p, d)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o.view(torch.int16)), name
        assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), name
    ro, rl = oracle_of(p)
    compare(p.dtype, o, lse, ro, rl, p.name)


def test_counters_at_rest_after_calls(dev):
    """After split calls (eager, on garbage and on reused workspaces) no counter
    is left part counted."""
    p = _split_problem(seed=84)
    d = to_dev(p, dev)
    ws = fad.workspace_paged(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                             p.page_size, p.total_used_pages, dev)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8))
    args = (p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim, p.page_size,
            p.total_used_pages)
    for _ in range(3):
        run(p, d, workspace=ws)
        torch.cuda.synchronize()
        assert fad.fa_debug_counters_in_use(*args, ws) == 0
