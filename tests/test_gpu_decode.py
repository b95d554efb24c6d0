"""Parity of attn_decode_paged with the oracle's decode on the contiguous per-sequence
caches (the oracle never sees the paged pool, so the block-table translation is checked
independently), plus poison in unused slots and split-count invariance (merge law)."""

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import errs, to64

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 1e-2, 1e-3


def gpu_decode(w, kv_split=0):
    q = w.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    attn.attn_decode_paged(q, w.k_cache.cuda(), w.v_cache.cuda(), w.block_table.cuda(),
                           w.seq_lens.tolist(), max_seq_len=w.max_seq_len, kv_split=kv_split,
                           out=out, lse=lse)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


@pytest.mark.parametrize("lens,split", [([1], 0), ([1, 15, 16, 17], 16), ([33, 250, 256, 257], 32),
                                        ([1000, 3, 700], 0), ([4096, 1, 2049], 1024),
                                        ([300, 301], 48)])
def test_decode_shapes(lens, split):
    w = workloads.paged(lens, 3, 128, seed=sum(lens), poison=True, spare_blocks=3)
    print(f"case: decode lens={lens} split={split}", flush=True)
    o, lse = gpu_decode(w, split)
    ro, rl = oracle.decode(w.q, w.k_seqs, w.v_seqs)
    mx, mean = errs(o, ro)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse, rl, rtol=2e-6, atol=2e-5)
    if lens[0] == 1:  # a single cached token returns its value exactly
        np.testing.assert_array_equal(o[0], to64(w.v_seqs[0][:, 0]))


@pytest.mark.parametrize("poison", [False, True])
def test_decode_workload(poison):
    w = workloads.paged_decode(poison=poison)
    print(f"case: paged decode B=32 H=32 poison={poison}", flush=True)
    o, lse = gpu_decode(w)
    ro, rl = oracle.decode(w.q, w.k_seqs, w.v_seqs)
    mx, mean = errs(o, ro)
    print(f"max-abs {mx:.5f} mean-abs {mean:.2e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse, rl, rtol=2e-6, atol=2e-5)


def test_decode_split_invariance():
    """Merging partial (m, l, u) summaries is exact in real arithmetic: any split length
    gives the same output up to rounding."""
    w = workloads.paged([5000, 77, 1024, 3333], 4, 128, seed=51)
    ro, _ = oracle.decode(w.q, w.k_seqs, w.v_seqs)
    outs = [gpu_decode(w, s)[0] for s in (16, 64, 256, 1024)]
    for o in outs:
        mx, mean = errs(o, ro)
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 2 * 2.0 ** -8  # a couple of bf16 ulps at |o| < 1


@pytest.mark.parametrize("kv_heads,window", [(None, 0), (2, 300)])
def test_decode_workspace_contents_unused(kv_heads, window):
    """The split workspace is scratch: what it holds before the call (zero bytes, then NaN
    bytes) never reaches the output, also where most splits of the grid lie past a short
    sequence's end (lengths 1 and 20 beside 3000)."""
    lens = [3000, 1, 20, 1500]
    w = workloads.paged(lens, 8, 128, seed=61, kv_heads=kv_heads, poison=True)
    print(f"case: decode workspace poison lens={lens} kv_heads={kv_heads} window={window}", flush=True)
    q, kc, vc, bt = w.q.cuda(), w.k_cache.cuda(), w.v_cache.cuda(), w.block_table.cuda()
    need = attn.attn_decode_workspace_bytes(len(lens), 8, 128, w.max_seq_len, 64,
                                            kv_heads=kv_heads, window=window)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        o, lse = attn.attn_decode_paged(q, kc, vc, bt, lens, max_seq_len=w.max_seq_len,
                                        window=window, kv_split=64, workspace=ws, return_lse=True)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert bool(torch.isfinite(a).all())
        assert torch.equal(a, b)


def test_decode_and_backward_on_a_side_stream():
    """Entry points called with stream=<a side stream>: the binding allocates the outputs, the
    workspaces and the uploaded lengths on that stream, so the default stream's allocations
    made meanwhile (here filled with NaN) never take memory the side stream's kernels still
    use.  Results match the oracle."""
    print("case: decode and backward on a side stream", flush=True)
    side = torch.cuda.Stream()
    w = workloads.paged([700, 33, 1500, 4000], 4, 128, seed=78, kv_heads=2)
    q, kc, vc, tbl = w.q.cuda(), w.k_cache.cuda(), w.v_cache.cuda(), w.block_table.cuda()
    qp, kp, vp = workloads.prefill(1, 4, 300, 128, seed=79, kv_heads=2)
    do = torch.randn(1, 4, 300, 128, generator=torch.Generator().manual_seed(80)).to(torch.bfloat16)
    qpd, kpd, vpd, dod = qp.cuda(), kp.cuda(), vp.cuda(), do.cuda()
    o_f, lse_f = attn.attn_fwd(qpd, kpd, vpd, causal=True, return_lse=True)
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        o = attn.attn_decode_paged(q, kc, vc, tbl, w.seq_lens.tolist(), max_seq_len=w.max_seq_len,
                                   stream=side)
        grads = attn.attn_bwd(qpd, kpd, vpd, o_f, dod, lse_f, causal=True, stream=side)
        # default-stream traffic while the side stream runs
        junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(8)]
        del junk
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ro, _ = oracle.decode(w.q, w.k_seqs, w.v_seqs)
    mx, mean = errs(to64(o), ro)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    refs = oracle.attention_grad(qp, kp, vp, do, causal=True)
    mags = oracle.attention_grad_magnitudes(qp, kp, vp, do, causal=True)
    for g, r, a in zip(grads, refs, mags):
        assert np.all(np.abs(to64(g) - r) <= 2.0 ** -6 * a + 1e-6)
