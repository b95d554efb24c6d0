"""Parity of attn_fwd_chunk (C ABI through the binding): a chunk of queries at positions
q_start .. q_start + n_q - 1 against a key sequence of n_kv rows, checked against
oracle.attention_chunk (fp64), and against attn_fwd over the whole sequence.

Tolerances as for the bf16 prefill: max-abs 1e-2 and mean-abs 1e-3 on the output, LSE within
2^-8 (the normaliser sums bf16-rounded weights, each within 2^-8 relative of exact).  Where
the chunk's query tiles coincide with the whole-sequence run's (q_start a multiple of the
128-query tile), every query sees the same work in the same order and the result is
compared bit for bit."""

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import errs, to64

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 1e-2, 1e-3
BF16_LSE_ATOL = 2.0 ** -8

# (B, H, H_kv, n_q, n_kv, q_start, causal, window)
CASES = [
    (1, 2, 2, 64, 64, 0, True, 0),         # the whole sequence as one chunk
    (2, 4, 2, 100, 300, 200, True, 0),     # the last rows of a sequence
    (1, 4, 4, 129, 1000, 500, True, 0),    # a chunk in the middle, ragged tile
    (2, 2, 1, 257, 700, 300, False, 0),    # no mask: every key admitted
    (1, 4, 2, 200, 900, 650, True, 128),   # window
    (1, 2, 2, 1, 513, 512, True, 0),       # a single query at the last position
    (1, 3, 3, 300, 300, 0, True, 64),
    (2, 32, 8, 130, 400, 100, True, 0),    # B*H a multiple of 64: eight heads per XCD at a time
    (2, 9, 3, 4096, 4608, 512, True, 0),   # 576 query tiles: more than the GPU holds at once
    (1, 20, 20, 3333, 4000, 600, False, 0),  # 540 tiles, unmasked, ragged last tile
]


# head_dim 64 (the same kernel at half the dims)
D64_CASES = [
    (2, 4, 2, 100, 300, 200, True, 0),
    (1, 4, 2, 200, 900, 650, True, 128),
    (2, 2, 1, 257, 700, 300, False, 0),
]


@pytest.mark.parametrize("d,B,H,Hkv,nq,nkv,q0,causal,window",
                         [(128, *c) for c in CASES] + [(64, *c) for c in D64_CASES])
def test_chunk_matches_oracle(d, B, H, Hkv, nq, nkv, q0, causal, window):
    print(f"case: chunk d={d} B={B} H={H} Hkv={Hkv} n_q={nq} n_kv={nkv} q_start={q0} causal={causal} window={window}",
          flush=True)
    q, _, _ = workloads.prefill(B, H, nq, d, seed=nq + nkv + q0, kv_heads=Hkv)
    _, k, v = workloads.prefill(B, H, nkv, d, seed=7 * nkv + q0, kv_heads=Hkv)
    o, lse = attn.attn_fwd_chunk(q.cuda(), k.cuda(), v.cuda(), q0, causal=causal, window=window,
                                 return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_chunk(q, k, v, q0, causal=causal, window=window)
    o, lse = to64(o), to64(lse)
    mx, mean = errs(o, ro)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=BF16_LSE_ATOL)


@pytest.mark.parametrize("d,window", [(128, 0), (128, 300), (64, 0), (64, 300)])
def test_aligned_chunks_reproduce_the_whole_sequence_bit_for_bit(d, window):
    q, k, v = (x.cuda() for x in workloads.prefill(2, 4, 1000, d, seed=91, kv_heads=2))
    whole, whole_l = attn.attn_fwd(q, k, v, causal=True, window=window, return_lse=True)
    cuts = [0, 128, 512, 640, 1000]
    for a, c in zip(cuts[:-1], cuts[1:]):
        o, l = attn.attn_fwd_chunk(q[:, :, a:c].contiguous(), k, v, a, causal=True, window=window,
                                   return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o, whole[:, :, a:c]) and torch.equal(l, whole_l[:, :, a:c]), (a, c)


@pytest.mark.slow
def test_sequence_parallel_share_gathered_at_full_size():
    """Device 0's query chunks (0 and 15 of 16, 2048 rows each) of the long-context workload
    [1,32,32768,128] against the whole gathered K/V, as the sequence-parallel bench times
    them, on sampled rows (each chunk's first and last among them) against the oracle."""
    w = workloads.long_prefill()
    k, v = w["k"].cuda(), w["v"].cuda()
    c = 2048
    g = torch.Generator().manual_seed(82)
    for i in (0, 15):
        print(f"case: gathered sequence-parallel share, query chunk {i} of 16", flush=True)
        qi = w["q"][:, :, i * c:(i + 1) * c].contiguous().cuda()
        o, lse = attn.attn_fwd_chunk(qi, k, v, i * c, causal=True, return_lse=True)
        torch.cuda.synchronize()
        o, lse = to64(o), to64(lse)
        rows = np.stack([np.sort(np.concatenate([[0, c - 1], torch.randperm(c - 2, generator=g)[:14].numpy() + 1]))
                         for _ in range(32)]) + i * c
        ro, rl = oracle.attention_rows(w["q"], w["k"], w["v"], rows, causal=True)
        got = np.stack([o[0, h, rows[h] - i * c] for h in range(32)])[None]
        mx, mean = errs(got, ro)
        print(f"sampled rows max-abs {mx:.5f} mean-abs {mean:.2e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (i, mx, mean)
        got_l = np.stack([lse[0, h, rows[h] - i * c] for h in range(32)])[None]
        np.testing.assert_allclose(got_l, rl, rtol=0, atol=BF16_LSE_ATOL)
