"""Guard canaries: the library writes nothing outside its output buffers and
the workspace.

Every output (o, lse), the workspace and, for the append, the paged store
are carved out of a larger allocation with a 4 KiB guard region before and
after, filled with a fixed byte pattern; after the calls each guard must be
unchanged.  Covers the full C3 and C5 decode (split units and their merges),
the window / soft-cap / ALiBi / mask variants, the allocation-free entry
point's outputs, the decode-time append and the standalone merge.
"""
import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import workloads as W
from gpu_util import announce, device, to_dev

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side
PATTERN = 0xA5


@pytest.fixture(scope="module")
def dev():
    return device()


class Guarded:
    """A device tensor of the given shape and dtype sitting between two guard
    regions of GUARD bytes (the data starts 4 KiB in, so alignment is kept)."""

    def __init__(self, shape, dtype, dev, fill=None):
        numel = int(np.prod(shape))
        es = torch.empty((), dtype=dtype).element_size()
        self.nbytes = numel * es
        self.raw = torch.full((2 * GUARD + self.nbytes,), PATTERN, dtype=torch.uint8,
                              device=dev)
        self.t = self.raw[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        lo = self.raw[:GUARD]
        hi = self.raw[GUARD + self.nbytes:]
        assert bool((lo == PATTERN).all()), f"{what}: guard before the buffer overwritten"
        assert bool((hi == PATTERN).all()), f"{what}: guard after the buffer overwritten"


def _guarded_decode(p, d, dev, **kw):
    o = Guarded(tuple(d["q"].shape), d["q"].dtype, dev)
    lse = Guarded((p.batch, p.num_qo_heads), torch.float32, dev)
    need = fad.fa_decode_workspace_size(p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
                                        p.page_size, p.total_used_pages)
    ws = Guarded((need,), torch.uint8, dev)
    fad.decode_paged(d["q"], d["k"], d["v"], d["indices"], d["indptr"], d["lpl"], p.scale,
                     o=o.t, lse=lse.t, workspace=ws.t, layout=p.layout, **kw)
    return o, lse, ws


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_guards_full_decode(dev, name):
    p = W.FULL[name]()
    announce(f"guards full {p.name}")
    d = to_dev(p, dev)
    for variant, kw in (("plain", {}), ("window", dict(window=700)),
                        ("cap+alibi", dict(softcap=30.0,
                                           alibi=torch.linspace(0.01, 0.3, p.num_qo_heads,
                                                                device=dev))),
                        ("mask", dict(mask=torch.from_numpy(W.pack_mask(W.random_mask(
                            5, p.kv_lens, keep=0.5))).to(dev)))):
        for rep in range(2):  # the second call finds the counters at rest
            o, lse, ws = _guarded_decode(p, d, dev, **kw)
            for g, what in ((o, "o"), (lse, "lse"), (ws, "workspace")):
                g.check(f"{p.name} {variant} call {rep}: {what}")
    # token-major store
    pn = W.token_major(p)
    o, lse, ws = _guarded_decode(pn, to_dev(pn, dev), dev)
    for g, what in ((o, "o"), (lse, "lse"), (ws, "workspace")):
        g.check(f"{pn.name}: {what}")
    torch.cuda.empty_cache()


def test_guards_noalloc_outputs(dev):
    p = W.SMALL["c3"]()
    d = to_dev(p, dev)
    o = Guarded(tuple(d["q"].shape), d["q"].dtype, dev)
    lse = Guarded((p.batch, p.num_qo_heads), torch.float32, dev)
    fad.fa_decode_paged_noalloc(fad.DTYPE_CODES[p.dtype], p.batch, p.num_qo_heads,
                                p.num_kv_heads, p.head_dim, p.page_size, p.num_total_pages,
                                p.total_used_pages, p.scale, d["q"], d["k"], d["v"],
                                d["indices"], d["indptr"], d["lpl"], o.t, lse.t)
    o.check("noalloc o")
    lse.check("noalloc lse")


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
def test_guards_append(dev, layout):
    p = W.SMALL["c5"]()
    if layout == "nhd":
        p = W.token_major(p)
    k = Guarded(tuple(p.k_data.shape), p.k_data.dtype, dev, fill=p.k_data.to(dev))
    v = Guarded(tuple(p.v_data.shape), p.v_data.dtype, dev, fill=p.v_data.to(dev))
    shape = (p.batch, p.num_kv_heads, p.head_dim)
    g = torch.Generator(device="cpu").manual_seed(3)
    k_new = torch.randn(shape, generator=g).to(p.k_data.dtype).to(dev)
    v_new = torch.randn(shape, generator=g).to(p.k_data.dtype).to(dev)
    fad.append_paged(k_new, v_new, k.t, v.t, p.indices.to(dev), p.indptr.to(dev),
                     p.last_page_len.to(dev), layout=layout)
    k.check(f"append {layout}: k store")
    v.check(f"append {layout}: v store")


def test_guards_merge(dev):
    rng = np.random.default_rng(4)
    s_, rows, d = 5, 777, 256
    o_p = torch.from_numpy(rng.standard_normal((s_, rows, d)).astype(np.float32)).to(dev)
    l_p = torch.from_numpy((rng.standard_normal((s_, rows)) * 3).astype(np.float32)).to(dev)
    for dt in (torch.float32, torch.float16, torch.bfloat16):
        o = Guarded((rows, d), dt, dev)
        lse = Guarded((rows,), torch.float32, dev)
        fad.merge_states(o_p, l_p, o=o.t, lse=lse.t)
        o.check(f"merge {dt}: o")
        lse.check(f"merge {dt}: lse")
