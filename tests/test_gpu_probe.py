"""The measurement kernels (include/attn_probe.h) through the C ABI: each leaves the checksum
its work must produce, so a ceiling `bench.py --workload ceilings` reports comes from work
that was done.  Small grids; the sums are exact (integers in fp32 below 2^24, wrapping
32-bit word sums)."""

import numpy as np
import pytest
import torch

from online_softmax_attn_amd import binding as b

pytestmark = pytest.mark.gpu

FIXED = 0.641185744504986  # the solution of x = 2^(-x)


def word_sum(x):
    return int(x.view(torch.int32).cpu().numpy().astype(np.int64).sum()) % 2**32


def total(out):
    return int(out.cpu().numpy().astype(np.int64).sum()) % 2**32


@pytest.mark.parametrize("fp8,k", [(0, 16), (1, 64)])
@pytest.mark.parametrize("blocks,iters", [(1, 1), (7, 64), (512, 300)])
def test_mfma_probe_checksum(fp8, k, blocks, iters):
    out = b.attn_probe_mfma(fp8, blocks, iters)
    torch.cuda.synchronize()
    assert out.shape == (blocks * 4,)
    assert torch.all(out == float(64 * k * iters)), out[:8]


@pytest.mark.parametrize("blocks,iters", [(1, 100), (33, 1000)])
def test_exp_probe_converges_to_the_fixed_point(blocks, iters):
    out = b.attn_probe_exp(blocks, iters)
    torch.cuda.synchronize()
    assert out.shape == (blocks * 256,)
    assert torch.all((out - 8 * FIXED).abs() < 1e-4), out[:4]


@pytest.mark.parametrize("pages,blocks", [(1, 1), (10, 3), (257, 16), (4096, 64)])
def test_read_probe_sums_every_word_once(pages, blocks):
    g = torch.Generator().manual_seed(pages)
    src = torch.randint(-2**31, 2**31 - 1, (pages * 1024,), dtype=torch.int32, generator=g)
    out = b.attn_probe_read(src.cuda(), blocks)
    torch.cuda.synchronize()
    assert total(out) == word_sum(src)


@pytest.mark.parametrize("pool_pages,n,blocks", [(1, 1, 1), (64, 100, 2), (300, 300, 8),
                                                  (1000, 5000, 40)])
def test_read_pages_probe_sums_the_pages_in_order(pool_pages, n, blocks):
    g = torch.Generator().manual_seed(n)
    pool = torch.randint(-2**31, 2**31 - 1, (pool_pages, 1024), dtype=torch.int32, generator=g)
    order = torch.randint(0, pool_pages, (n,), dtype=torch.int32, generator=g)
    out = b.attn_probe_read_pages(pool.cuda(), order.cuda(), blocks)
    torch.cuda.synchronize()
    want = word_sum(pool[order.long()])
    assert total(out) == want
