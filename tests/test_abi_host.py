"""Host-side tests of the C ABI (no GPU needed).

The library must load and export every function the public headers declare.
Argument checks happen on the host before any HIP call, so each rejection path
can be exercised here with placeholder pointers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import decode_attention_query_amd as fad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below is rejected first
MIS2 = ctypes.c_void_p(0x1002)  # misaligned for every array the library reads or writes
MIS8 = ctypes.c_void_p(0x1008)  # 8-byte aligned: enough for int32 / f32, not for 16-byte moves


def _declared_functions():
    names = set()
    for fn in os.listdir(INCLUDE):
        if fn.endswith(".h"):
            text = open(os.path.join(INCLUDE, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = fad.load_library()
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert declared == set(fad.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for code, name in fad.STATUS_NAMES.items():
        assert fad.fa_status_string(code) == name


def test_workspace_size():
    ws = fad.fa_decode_workspace_size
    assert ws(64, 32, 8, 128, 16, 17408) > 0
    assert ws(1, 8, 2, 64, 256, 1) > 0
    # invalid problems report 0
    assert ws(0, 32, 8, 128, 16, 10) == 0
    assert ws(4, 30, 8, 128, 16, 10) == 0       # group not integral
    assert ws(4, 32, 8, 96, 16, 10) == 0        # head_dim unsupported
    assert ws(4, 32, 8, 128, 0, 10) == 0
    assert ws(4, 32, 8, 128, 16, -1) == 0
    assert ws(4, 32, 8, 128, 1 << 20, 1 << 12) == 0  # 2^32 rows
    # grows with the problem
    assert ws(64, 32, 8, 128, 16, 40000) >= ws(64, 32, 8, 128, 16, 1000)
    assert ws(64, 32, 8, 256, 16, 1000) >= ws(64, 32, 8, 128, 16, 1000)


def test_plan_covers_units():
    """The unit bound covers any request lengths the page table allows."""
    for dtype, b, hq, hkv, d, p, used in [(2, 64, 32, 8, 128, 16, 17408),
                                          (2, 32, 64, 8, 128, 32, 32768),
                                          (1, 128, 16, 4, 256, 16, 33000),
                                          (0, 1, 8, 2, 64, 256, 1),
                                          (2, 3, 12, 4, 64, 3, 7),
                                          (2, 4, 28, 4, 128, 16, 90),   # G = 7
                                          (1, 2, 71, 1, 128, 16, 40),   # G = 71
                                          (1, 2, 96, 2, 64, 16, 40)]:   # G = 48
        chunk, bound, gt, kind = fad.fa_debug_plan(dtype, b, hq, hkv, d, p, used)
        assert chunk > 0 and chunk % 128 == 0
        # heads per workgroup: the whole group up to 16, else two blocks of 16
        assert gt == min(hq // hkv, 32)
        # worst case: every row in one request, or spread so each request wastes a unit
        rows = used * p
        assert bound >= -(-rows // chunk) + (b - 1)


def _paged(*, dtype=2, batch=2, hq=8, hkv=2, d=128, page=16, pages=10, used=4,
           ptrs=None, ws=FAKE, ws_bytes=1 << 30, fn="fa_decode_paged"):
    lib = fad.load_library()
    q = k = v = ind = ptr = lpl = o = lse = FAKE
    if ptrs:
        q, k, v, ind, ptr, lpl, o, lse = [ptrs.get(n, FAKE) for n in
                                          ("q", "k", "v", "ind", "ptr", "lpl", "o", "lse")]
    return getattr(lib, fn)(dtype, batch, hq, hkv, d, page, pages, used, 0.125, q, k, v, ind,
                            ptr, lpl, o, lse, ws, ws_bytes, None)


def _contig(*, dtype=1, hq=8, hkv=2, d=64, max_len=256, valid=128, ptrs=None, ws=FAKE,
            ws_bytes=1 << 30, fn="fa_decode_contig"):
    lib = fad.load_library()
    q = k = v = o = lse = FAKE
    if ptrs:
        q, k, v, o, lse = [ptrs.get(n, FAKE) for n in ("q", "k", "v", "o", "lse")]
    return getattr(lib, fn)(dtype, hq, hkv, d, max_len, valid, 0.125, q, k, v, o, lse, ws,
                            ws_bytes, None)


INV, UNS, WS = fad.FA_ERR_INVALID_PROBLEM, fad.FA_ERR_UNSUPPORTED, fad.FA_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), UNS),
    (dict(dtype=-1), UNS),
    (dict(batch=0), INV),
    (dict(hq=0), INV),
    (dict(hkv=0), INV),
    (dict(page=0), INV),
    (dict(pages=0), INV),
    (dict(hq=12, hkv=8), INV),
    (dict(d=96), UNS),
    (dict(d=512), UNS),
    (dict(used=-1), INV),
    (dict(ptrs={"q": None}), INV),
    (dict(ptrs={"k": None}), INV),
    (dict(ptrs={"v": None}), INV),
    (dict(ptrs={"ind": None}), INV),
    (dict(ptrs={"ptr": None}), INV),
    (dict(ptrs={"lpl": None}), INV),
    (dict(ptrs={"o": None}), INV),
    (dict(ptrs={"lse": None}), INV),
    (dict(ptrs={"q": MIS2}), INV),                     # 16-byte arrays off by 2 or 8
    (dict(ptrs={"k": MIS8}), INV),
    (dict(ptrs={"v": MIS2}), INV),
    (dict(ptrs={"o": MIS8}), INV),
    (dict(ws=MIS8), INV),
    (dict(ptrs={"ind": MIS2}), INV),                   # 4-byte arrays off by 2
    (dict(ptrs={"ptr": MIS2}), INV),
    (dict(ptrs={"lpl": MIS2}), INV),
    (dict(ptrs={"lse": MIS2}), INV),
    (dict(ptrs={"q": MIS2}, page=1 << 20, used=1 << 11, pages=1 << 11), INV),  # before range
    (dict(page=1 << 20, used=1 << 11, pages=1 << 11), UNS),
    (dict(hq=70000, hkv=70000), UNS),                  # more query heads than a launch takes
    (dict(pages=1 << 30, hkv=64, hq=64, page=1 << 9), UNS),  # pool beyond 10^15 elements
    # 2^31 workgroups or more (32,768 heads of one KV head: 1,024 two-block workgroups per unit)
    (dict(batch=1 << 21, hq=32768, hkv=1), UNS),
    (dict(batch=1 << 21, hq=32768, hkv=1, ws=None), UNS),  # ... checked before the workspace
    (dict(ws=None), WS),
    (dict(ws_bytes=16), WS),
    # order: the dtype is checked before the extents, the extents before head_dim
    (dict(dtype=7, batch=0), UNS),
    (dict(batch=0, d=96), INV),
    (dict(d=96, ptrs={"q": None}), UNS),
    (dict(ptrs={"q": None}, ws=None), INV),
])
@pytest.mark.parametrize("fn", ["fa_decode_paged", "fa_decode_paged_nhd"])
def test_paged_rejects(kw, status, fn):
    assert _paged(**kw, fn=fn) == status


def _noalloc(*, dtype=2, batch=2, hq=8, hkv=2, d=128, page=16, pages=10, used=4, ptrs=None):
    lib = fad.load_library()
    q = k = v = ind = ptr = lpl = o = lse = FAKE
    if ptrs:
        q, k, v, ind, ptr, lpl, o, lse = [ptrs.get(n, FAKE) for n in
                                          ("q", "k", "v", "ind", "ptr", "lpl", "o", "lse")]
    return lib.fa_decode_paged_noalloc(dtype, batch, hq, hkv, d, page, pages, used, 0.125, q, k,
                                       v, ind, ptr, lpl, o, lse, None)


def test_noalloc_rejects_like_paged():
    """The allocation-free entry point makes fa_decode_paged's checks in the
    same order (no workspace argument), and refuses a problem whose workspace
    would not fit its static array -- all before any device call."""
    cases = [
        (dict(dtype=3), UNS), (dict(batch=0), INV), (dict(hq=12, hkv=8), INV),
        (dict(d=96), UNS), (dict(used=-1), INV), (dict(ptrs={"q": None}), INV),
        (dict(ptrs={"ind": None}), INV), (dict(ptrs={"lse": None}), INV),
        (dict(ptrs={"k": MIS8}), INV), (dict(ptrs={"ptr": MIS2}), INV),
        (dict(page=1 << 20, used=1 << 11, pages=1 << 11), UNS),
        (dict(hq=70000, hkv=70000), UNS), (dict(batch=1 << 21, hq=32768, hkv=1), UNS),
        (dict(dtype=7, batch=0), UNS), (dict(d=96, ptrs={"q": None}), UNS),
    ]
    for kw, status in cases:
        assert _noalloc(**kw) == status, kw
        assert _paged(**kw) == status, kw
    big = dict(batch=2048, hq=64, hkv=8, d=256, used=0)
    assert fad.fa_decode_workspace_size(2048, 64, 8, 256, 16, 0) > fad.FA_NOALLOC_SCRATCH_BYTES
    assert _noalloc(**big) == WS


def test_paged_workspace_exact_boundary():
    need = fad.fa_decode_workspace_size(2, 8, 2, 128, 16, 4)
    assert _paged(ws_bytes=need - 1) == WS


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=5), UNS),
    (dict(hq=0), INV),
    (dict(hkv=0), INV),
    (dict(max_len=0, valid=0), INV),
    (dict(hq=6, hkv=4), INV),
    (dict(d=32), UNS),
    (dict(ptrs={"q": None}), INV),
    (dict(ptrs={"k": None}), INV),
    (dict(ptrs={"v": None}), INV),
    (dict(ptrs={"o": None}), INV),
    (dict(ptrs={"q": MIS8}), INV),
    (dict(ptrs={"k": MIS2}), INV),
    (dict(ptrs={"v": MIS8}), INV),
    (dict(ptrs={"o": MIS2}), INV),
    (dict(ptrs={"lse": MIS2}), INV),
    (dict(ws=MIS8), INV),
    (dict(valid=-1), INV),
    (dict(valid=257), INV),
    (dict(ws=None), WS),
    (dict(ws_bytes=0), WS),
])
@pytest.mark.parametrize("fn", ["fa_decode_contig", "fa_decode_contig_nhd"])
def test_contig_rejects(kw, status, fn):
    assert _contig(**kw, fn=fn) == status


@pytest.mark.parametrize("fn", ["fa_debug_gather_paged", "fa_debug_gather_paged_nhd"])
def test_gather_rejects(fn):
    gather = getattr(fad.load_library(), fn)
    args = [2, 2, 2, 128, 16, 10, 4, FAKE, FAKE, FAKE, FAKE, FAKE]
    assert gather(*args, -1, FAKE, 1 << 30, None) == INV
    assert gather(*args, 10, None, 0, None) == WS
    bad = list(args)
    bad[3] = 100
    assert gather(*bad, 10, FAKE, 1 << 30, None) == UNS
    for i, mis in ((7, MIS8), (8, MIS2), (9, MIS2), (10, MIS2), (11, MIS8)):
        bad = list(args)
        bad[i] = mis
        assert gather(*bad, 10, FAKE, 1 << 30, None) == INV, i
    assert gather(*args, 10, MIS8, 1 << 30, None) == INV


@pytest.mark.parametrize("fn", ["fa_append_paged", "fa_append_paged_nhd"])
def test_append_rejects(fn):
    append = getattr(fad.load_library(), fn)
    ok = [2, 2, 2, 128, 16, 10, 4]
    ptrs = [FAKE] * 7
    assert append(7, *ok[1:], *ptrs, None) == UNS
    assert append(2, 0, *ok[2:], *ptrs, None) == INV
    assert append(2, 2, 2, 96, *ok[4:], *ptrs, None) == UNS
    assert append(2, 2, 2, 128, 16, 0, 4, *ptrs, None) == INV
    assert append(2, 2, 2, 128, 16, 10, -1, *ptrs, None) == INV
    for i in range(7):
        bad = list(ptrs)
        bad[i] = None
        assert append(*ok, *bad, None) == INV, i
    assert append(2, 2, 2, 128, 1 << 20, 1 << 11, 1 << 11, *ptrs, None) == UNS
    # k_new, v_new 16-byte; indices, indptr, last_page_len 4-byte; k_data, v_data 16-byte
    for i, mis in enumerate((MIS8, MIS8, MIS2, MIS2, MIS2, MIS8, MIS8)):
        bad = list(ptrs)
        bad[i] = mis
        assert append(*ok, *bad, None) == INV, i


def test_options_reject():
    lib = fad.load_library()
    base = [2, 2, 8, 2, 128, 16, 10, 4, 0.125] + [FAKE] * 8 + [FAKE, 1 << 30, None]
    for opts, status in ((fad.DecodeOptions(2, 0, 0.0, None), UNS),
                         (fad.DecodeOptions(-1, 0, 0.0, None), UNS),
                         (fad.DecodeOptions(0, -1, 0.0, None), INV),
                         (fad.DecodeOptions(0, 0, -1.0, None), INV),
                         (fad.DecodeOptions(0, 0, float("inf"), None), INV),
                         (fad.DecodeOptions(0, 0, float("nan"), None), INV),
                         (fad.DecodeOptions(0, 0, 0.0, MIS2.value), INV),
                         (fad.DecodeOptions(0, 0, 0.0, None, FAKE.value, 0), INV)):
        assert lib.fa_decode_paged_opts(ctypes.byref(opts), *base) == status
        assert lib.fa_decode_contig_opts(ctypes.byref(opts), 1, 8, 2, 64, 256, 128, 0.125,
                                         FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                                         None) == status
    # valid options, then the plain entry point's own checks
    ok = fad.DecodeOptions(1, 64, 30.0, None)
    assert lib.fa_decode_paged_opts(ctypes.byref(ok), 7, *base[1:]) == UNS
    assert lib.fa_decode_paged_opts(None, 2, 0, *base[2:]) == INV


def test_schedule_and_probe_reject():
    lib = fad.load_library()
    base = [2, 2, 8, 2, 128, 16, 4]
    assert lib.fa_debug_schedule(7, *base[1:], FAKE, FAKE, FAKE, 1 << 20, None) == UNS
    assert lib.fa_debug_schedule(*base, None, FAKE, FAKE, 1 << 20, None) == INV
    assert lib.fa_debug_schedule(*base, FAKE, FAKE, None, 1 << 20, None) == INV
    assert lib.fa_debug_schedule(*base, FAKE, FAKE, FAKE, 7, None) == WS
    assert lib.fa_debug_read_probe(None, 8192, FAKE, None) == INV
    assert lib.fa_debug_read_probe(FAKE, 8192, None, None) == INV
    assert lib.fa_debug_read_probe(FAKE, 0, FAKE, None) == INV
    assert lib.fa_debug_read_probe(FAKE, 8192 + 16, FAKE, None) == INV
    assert lib.fa_debug_read_probe(MIS8, 8192, FAKE, None) == INV
    assert lib.fa_debug_read_probe(FAKE, 8192, MIS2, None) == INV
    assert lib.fa_debug_schedule(*base, MIS2, FAKE, FAKE, 1 << 20, None) == INV
    assert lib.fa_debug_schedule(*base, FAKE, FAKE, MIS2, 1 << 20, None) == INV


def test_binding_rejects_host_tensors():
    """The binding refuses buffers that are not device memory before calling in."""
    import torch
    q = torch.zeros(8, 64)
    with pytest.raises(ValueError):
        fad.fa_decode_contig(0, 8, 2, 64, 16, 8, 0.125, q, q, q, q, None, q)


def test_timing_hooks_without_calls():
    fad.fa_debug_timing_enable(1)
    main_ms, call_ms, n = fad.fa_debug_timing_read()
    fad.fa_debug_timing_enable(0)
    assert (main_ms, call_ms, n) == (0.0, 0.0, 0)


def test_merge_rejects():
    merge = fad.load_library().fa_merge_states
    ptrs = [FAKE] * 4
    assert merge(3, 16, 2, 128, *ptrs, None) == UNS
    assert merge(0, -1, 2, 128, *ptrs, None) == INV
    assert merge(0, 16, 0, 128, *ptrs, None) == INV
    assert merge(0, 16, 2, 96, *ptrs, None) == UNS
    # no rows: accepted before the buffers are looked at, nothing enqueued
    assert merge(0, 0, 2, 128, None, None, None, None, None) == fad.FA_OK
    for i in range(3):
        bad = list(ptrs)
        bad[i] = None
        assert merge(0, 16, 2, 128, *bad, None) == INV, i
    # o_parts and o 16-byte, lse_parts and lse 4-byte
    for i, mis in enumerate((MIS8, MIS2, MIS8, MIS2)):
        bad = list(ptrs)
        bad[i] = mis
        assert merge(0, 16, 2, 128, *bad, None) == INV, i
    assert merge(0, 1 << 30, 1 << 14, 256, *ptrs, None) == UNS
    # order: dtype, then extents, then head_dim, then pointers
    assert merge(9, -1, 0, 96, None, None, None, None, None) == UNS
    assert merge(1, -1, 2, 96, None, None, None, None, None) == INV
    assert merge(1, 16, 2, 96, None, None, None, None, None) == UNS


def test_merge_binding_reports_no_parts():
    """Zero parts reach the library, which reports an invalid problem (no
    buffer is looked at, so host tensors of the right shape suffice)."""
    import torch
    with pytest.raises(fad.FaError) as e:
        fad.merge_states(torch.zeros((0, 4, 64)), torch.zeros((0, 4)), stream=0)
    assert e.value.status == fad.FA_ERR_INVALID_PROBLEM
