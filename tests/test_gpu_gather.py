"""The page-table gather the decode kernel performs, bit for bit.

fa_debug_gather_paged runs the decode kernel's own address path -- its split
units, the unit's page ids staged in LDS, and the tile loads of issue_tile
(16-row blocks at a page's base plus a row stride when the page size is a
multiple of 16, per-row resolution otherwise) -- and writes out what it
loaded.  Each case compares that with the oracle's gather, byte for byte, for
K and V: the full-size paged workloads in both K/V layouts, and page sizes
16, 32, 48 and 64 as well as ones that are not multiples of 16, over element
types and head dims.  Page table: the baracuda-kernels batch_paged_decode
page, module doc "Layout".
"""
import zlib

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce, check_gather, device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_gather_full_workload(dev, name, layout):
    p = W.FULL[name]()
    if layout == "nhd":
        p = W.token_major(p)
    announce(f"gather full {p.name}")
    check_gather(p, dev)
    torch.cuda.empty_cache()


# dtype, head_dim, num_kv_heads, page_size: element widths change the tile
# height (32 rows for 16-bit, 16 for f32) and the rows per load instruction
PAGE_CASES = [
    ("bf16", 128, 8, 16), ("f16", 256, 4, 16), ("f32", 64, 2, 16),
    ("bf16", 128, 2, 32), ("f32", 256, 1, 32), ("f16", 64, 3, 32),
    ("f16", 128, 2, 48), ("bf16", 256, 1, 48), ("f32", 128, 4, 48),
    ("bf16", 64, 2, 64), ("f16", 128, 1, 64), ("f32", 256, 2, 64),
    ("bf16", 128, 2, 5), ("f16", 256, 1, 24), ("f32", 64, 2, 7), ("bf16", 64, 1, 1),
]


@pytest.mark.parametrize("layout", ["hnd", "nhd"])
@pytest.mark.parametrize("case", PAGE_CASES, ids=lambda c: f"{c[0]}-D{c[1]}-P{c[3]}")
def test_gather_page_sizes(dev, case, layout):
    """Lengths around page and tile edges, a request split over many units
    (the split is at least 128 rows), an empty request and an empty last page,
    pages permuted in a pool with unreferenced slack."""
    dtype, d, hkv, page_size = case
    seed = zlib.crc32(str(case).encode())
    lens = np.array([0, 1, page_size - 1 if page_size > 1 else 2, page_size, page_size + 1, 31,
                     32, 33, 127, 129, 1000, 4099, 9001])
    n_pages, lpl = W.pages_for_lens(lens, page_size)
    n_pages, lpl = n_pages.copy(), lpl.copy()
    # request 3 (a whole number of pages) gets one more, empty page
    n_pages[3] += 1
    lpl[3] = 0
    p = W.make_paged(f"gather-P{page_size}", dtype, len(lens), hkv, hkv, d, page_size, seed,
                     n_pages=n_pages, last_page_len=lpl, pool_slack=0.3)
    if layout == "nhd":
        p = W.token_major(p)
    announce(f"gather {case} {layout}: {p.total_used_pages} pages")
    check_gather(p, dev)
