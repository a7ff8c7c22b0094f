"""A captured decode loop: per token, for every layer, append the token's K/V
into that layer's paged store and decode over it, all in one HIP graph that is
replayed token after token while the page tables grow (the resident-cache
decode step of the ferrox-cuda page, with the KV buffers kept on the device
and the step captured once).

Every replay is compared, bit for bit, with the same calls issued eagerly on
copies of the stores, and the final token with the float64 oracle.
"""
import numpy as np
import pytest
import torch

import decode_attention_query_amd as fad
import oracle
import workloads as W
from gpu_util import announce, compare, device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _tables(lens, page_size, capacity_pages, perm):
    """Page table for the given lengths; request b takes pages of its own
    fixed slice of perm, so a growing request keeps its earlier pages."""
    batch = len(lens)
    per = capacity_pages // batch
    n_pages = [(L + page_size - 1) // page_size for L in lens]
    indices = np.zeros(capacity_pages, dtype=np.int32)
    indptr = np.zeros(batch + 1, dtype=np.int32)
    k = 0
    for b in range(batch):
        indptr[b] = k
        indices[k:k + n_pages[b]] = perm[b * per: b * per + n_pages[b]]
        k += n_pages[b]
    indptr[batch] = k
    lpl = np.array([(L - 1) % page_size + 1 if L else 0 for L in lens], dtype=np.int32)
    return indices, indptr, lpl


def test_captured_decode_loop(dev):
    layers, batch, hq, hkv, d, page_size, dtype = 3, 4, 16, 4, 128, 16, "bf16"
    tdt = W.TORCH_DTYPES[dtype]
    tokens = 6
    start = [1, 15, 40, 100]                     # lengths before the first step
    capacity = 4 * 16                            # page slots per table (16 per request)
    pool = capacity + 8
    rng = np.random.default_rng(31)
    perm = rng.permutation(pool).astype(np.int32)
    g = torch.Generator().manual_seed(31)
    stores = [[(torch.randn((pool, hkv, page_size, d), generator=g) * 0.5).to(tdt).to(dev)
               for _ in range(2)] for _ in range(layers)]
    eager = [[t.clone() for t in kv] for kv in stores]
    # captured buffers: page table (capacity-sized), per-layer q and new K/V, outputs
    ind = torch.zeros(capacity, dtype=torch.int32, device=dev)
    ptr = torch.zeros(batch + 1, dtype=torch.int32, device=dev)
    lpl = torch.zeros(batch, dtype=torch.int32, device=dev)
    q = [torch.zeros((batch, hq, d), dtype=tdt, device=dev) for _ in range(layers)]
    kn = [torch.zeros((batch, hkv, d), dtype=tdt, device=dev) for _ in range(layers)]
    vn = [torch.zeros((batch, hkv, d), dtype=tdt, device=dev) for _ in range(layers)]
    o = [torch.zeros((batch, hq, d), dtype=tdt, device=dev) for _ in range(layers)]
    lse = [torch.zeros((batch, hq), dtype=torch.float32, device=dev) for _ in range(layers)]
    ws = fad.workspace_paged(batch, hq, hkv, d, page_size, capacity, dev)
    scale = float(np.float32(1 / np.sqrt(d)))

    def step(st, outs):
        for layer in range(layers):
            k, v = st[layer]
            fad.fa_append_paged(fad.DTYPE_CODES[dtype], batch, hkv, d, page_size, pool, capacity,
                                kn[layer], vn[layer], ind, ptr, lpl, k, v)
            fad.fa_decode_paged(fad.DTYPE_CODES[dtype], batch, hq, hkv, d, page_size, pool,
                                capacity, scale, q[layer], k, v, ind, ptr, lpl, outs[0][layer],
                                outs[1][layer], ws)

    def set_token(t):
        lens = [L + t + 1 for L in start]        # the table already counts the new token
        i, p, l = _tables(lens, page_size, capacity, perm)
        ind.copy_(torch.from_numpy(i))
        ptr.copy_(torch.from_numpy(p))
        lpl.copy_(torch.from_numpy(l))
        for layer in range(layers):
            q[layer].copy_(torch.randn((batch, hq, d), generator=g).to(tdt))
            kn[layer].copy_(torch.randn((batch, hkv, d), generator=g).to(tdt))
            vn[layer].copy_(torch.randn((batch, hkv, d), generator=g).to(tdt))
        return lens

    # warm up on a side stream, then capture one whole step
    set_token(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    warm = [[t.clone() for t in kv] for kv in stores]
    with torch.cuda.stream(side):
        step(warm, (o, lse))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del warm
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(stores, (o, lse))
    torch.cuda.synchronize()

    eo = [torch.empty_like(t) for t in o]
    el = [torch.empty_like(t) for t in lse]
    for t in range(tokens):
        lens = set_token(t)
        announce(f"captured loop token {t}: lengths {lens}")
        step(eager, (eo, el))                    # eager reference on its own stores
        graph.replay()
        torch.cuda.synchronize()
        for layer in range(layers):
            assert torch.equal(o[layer], eo[layer]) and torch.equal(lse[layer], el[layer]), \
                (t, layer)
            for kv in range(2):
                assert torch.equal(stores[layer][kv], eager[layer][kv]), (t, layer, kv)
    # last token against the oracle
    i, p, l = _tables(lens, page_size, capacity, perm)
    n_used = int(p[-1])
    for layer in range(layers):
        ro, rl = oracle.decode_paged(dtype, W.bits(q[layer].cpu()), W.bits(stores[layer][0].cpu()),
                                     W.bits(stores[layer][1].cpu()), i[:n_used], p, l, scale)
        compare(dtype, o[layer], lse[layer], ro, rl, f"layer {layer}")
