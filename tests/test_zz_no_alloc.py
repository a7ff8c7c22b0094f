"""fa_decode_paged_noalloc: the paged decode with its scratch in the library's
static device array instead of a caller's workspace.

Two calls in a row through the C ABI, the second on a smaller problem (so it
finds the first call's partials and counters in the array), each compared bit
for bit with fa_decode_paged on a workspace of its own, and with the float64
oracle at the stated tolerances.
"""
import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import workloads as W
from gpu_util import announce, compare, device, oracle_of, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _problems():
    big = W.make_paged("noalloc-big", "bf16", 8, 32, 8, 128, 16, 301,
                       lens=np.array([9000, 0, 17, 4096, 25000, 300, 12345, 1]),
                       pool_slack=0.1)
    small = W.make_paged("noalloc-small", "f16", 3, 8, 2, 64, 16, 302,
                         lens=np.array([5000, 2, 700]), pool_slack=0.2)
    return big, small


def _call(fn, p, d, o, lse, *ws):
    fn(fad.DTYPE_CODES[p.dtype], p.batch, p.num_qo_heads, p.num_kv_heads, p.head_dim,
       p.page_size, p.num_total_pages, p.total_used_pages, p.scale, d["q"], d["k"], d["v"],
       d["indices"], d["indptr"], d["lpl"], o, lse, *ws)


def test_noalloc_matches_workspace_entry_point(dev):
    for step, p in enumerate(_problems()):
        need = fad.fa_decode_workspace_size(p.batch, p.num_qo_heads, p.num_kv_heads,
                                            p.head_dim, p.page_size, p.total_used_pages)
        announce(f"noalloc call {step}: {p.name}, workspace {need} bytes")
        assert 0 < need <= fad.FA_NOALLOC_SCRATCH_BYTES
        d = to_dev(p, dev)
        o = torch.full_like(d["q"], float("nan"))
        lse = torch.full((p.batch, p.num_qo_heads), float("nan"), dtype=torch.float32,
                         device=dev)
        _call(fad.fa_decode_paged_noalloc, p, d, o, lse)
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        o_ref = torch.empty_like(d["q"])
        lse_ref = torch.empty_like(lse)
        _call(fad.fa_decode_paged, p, d, o_ref, lse_ref, ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), p.name
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), p.name
        ro, rl = oracle_of(p)
        eo, el = compare(p.dtype, o, lse, ro, rl, p.name)
        announce(f"  bit-identical to fa_decode_paged; max|do|={eo:.2e} max|dlse|={el:.2e}")


def test_noalloc_rejects_oversized_problem(dev):
    """A problem whose workspace exceeds the static array is refused on the host."""
    batch, hq, hkv, d = 2048, 64, 8, 256
    assert fad.fa_decode_workspace_size(batch, hq, hkv, d, 16, 0) > \
        fad.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((batch, hq, d), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, hkv, 16, d), dtype=torch.bfloat16, device=dev)
    ptr = torch.zeros(batch + 1, dtype=torch.int32, device=dev)
    lpl = torch.zeros(batch, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((batch, hq), dtype=torch.float32, device=dev)
    with pytest.raises(fad.FaError) as e:
        fad.fa_decode_paged_noalloc(fad.FA_DTYPE_BF16, batch, hq, hkv, d, 16, 1, 0, 0.0625, q,
                                    kv, kv, None, ptr, lpl, o, lse)
    assert e.value.status == fad.FA_ERR_WORKSPACE_TOO_SMALL
