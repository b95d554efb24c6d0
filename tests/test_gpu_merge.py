"""Parity of attn_merge (C ABI through the binding) with oracle.merge_outputs, and of the
per-device step of sequence-parallel attention: a query chunk's attention against key
chunks (attn_fwd, causal on the diagonal chunk), merged with attn_merge, against the
oracle's causal attention over the whole sequence.

Tolerances: fp32 parts: |o - ref| <= 1e-6 relative to max|ref| (one fp32 weight and one
fp32 division per element); lse within 1e-6.  bf16 parts: the merged value is rounded to
bf16 once more, so half a bf16 ulp of |ref| (at most 2^-8 |ref|: 8 significant bits) plus
2^-12 of max|ref| for the fp32 arithmetic.
The chunked prefill keeps the prefill's bf16 bar (max-abs 1e-2, mean-abs 1e-3, LSE 2^-8):
each chunk's output is rounded to bf16 before the merge, and merging averages those
roundings with weights summing to 1.
"""

import math

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


def random_parts(S, rows, d, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    outs = torch.randn(S, rows, d, generator=g).to(dtype)
    lses = torch.randn(S, rows, generator=g) * 30.0
    empty = torch.rand(S, rows, generator=g) < 0.2
    lses[empty] = -math.inf
    lses[:, 0] = -math.inf            # a row no part admits
    lses[0, 1] = 1e4                  # one part dominates row 1
    outs[empty.unsqueeze(-1).expand_as(outs)] = float("nan")  # never used
    outs[0, 1] = torch.randn(d, generator=g).to(dtype)         # the dominant part is live
    return outs, lses


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("S,rows,d", [(1, 37, 64), (3, 100, 128), (8, 1000, 64), (17, 257, 128)])
def test_merge_matches_oracle(dtype, S, rows, d):
    print(f"case: merge dtype={dtype} S={S} rows={rows} d={d}", flush=True)
    outs, lses = random_parts(S, rows, d, seed=S * 1000 + rows + d, dtype=dtype)
    o, lse = attn.attn_merge(outs.cuda(), lses.cuda(), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_outputs(to64(outs), lses.double().numpy())
    o, lse = to64(o), to64(lse)
    assert np.all(o[0] == 0) and lse[0] == -np.inf
    live = np.isfinite(rl)
    np.testing.assert_array_equal(np.isfinite(lse), live)
    np.testing.assert_allclose(lse[live], rl[live], rtol=1e-6, atol=1e-6)
    scale = np.abs(ro).max()
    if dtype == torch.float32:
        assert np.abs(o - ro).max() <= 1e-6 * scale
    else:
        bound = np.abs(ro) * 2.0 ** -8 + 2.0 ** -12 * scale  # half an ulp of 8 significant bits
        assert np.all(np.abs(o - ro) <= bound)


def test_single_part_is_returned_unchanged():
    outs, lses = random_parts(1, 300, 128, seed=5, dtype=torch.bfloat16)
    o, lse = attn.attn_merge(outs.cuda(), lses.cuda(), return_lse=True)
    torch.cuda.synchronize()
    live = torch.isfinite(lses[0])
    assert torch.equal(o.cpu()[live], outs[0][live])
    assert torch.equal(lse.cpu()[live], lses[0][live])


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
@pytest.mark.parametrize("chunks", [2, 4])
def test_chunked_causal_prefill_matches_oracle(dtype, d, chunks):
    # sequence-parallel form: query chunk i attends to key chunks j < i without a mask and
    # to its own chunk causally; the chunk results merge into the causal attention
    B, H, n = 1, 3, 384
    print(f"case: chunked causal prefill dtype={dtype} d={d} chunks={chunks}", flush=True)
    q, k, v = workloads.prefill(B, H, n, d, seed=71 + chunks)
    if dtype == torch.float32:
        q, k, v = q.float(), k.float(), v.float()
    ro, rl = oracle.attention(q, k, v, causal=True)
    qd, kd, vd = q.to(dtype).cuda(), k.to(dtype).cuda(), v.to(dtype).cuda()
    c = n // chunks
    scale = 1.0 / math.sqrt(d)
    for i in range(chunks):
        qi = qd[:, :, i * c:(i + 1) * c].contiguous()
        outs, lses = [], []
        for j in range(i + 1):
            kj = kd[:, :, j * c:(j + 1) * c].contiguous()
            vj = vd[:, :, j * c:(j + 1) * c].contiguous()
            o, l = attn.attn_fwd(qi, kj, vj, causal=(j == i), scale=scale, return_lse=True)
            outs.append(o)
            lses.append(l)
        o, lse = attn.attn_merge(torch.stack(outs), torch.stack(lses), return_lse=True)
        torch.cuda.synchronize()
        o, lse = to64(o), to64(lse)
        ref_o, ref_l = ro[:, :, i * c:(i + 1) * c], rl[:, :, i * c:(i + 1) * c]
        if dtype == torch.float32:
            assert np.abs(o - ref_o).max() <= 1e-5
            np.testing.assert_allclose(lse, ref_l, rtol=0, atol=1e-5)
        else:
            rows = np.ones(o.shape[:3], dtype=bool)
            mx, mean = errs(o, ref_o, rows)
            assert mx <= BF16_MAX and mean <= BF16_MEAN, (i, mx, mean)
            np.testing.assert_allclose(lse, ref_l, rtol=0, atol=BF16_LSE_ATOL)


@pytest.mark.slow
def test_sequence_parallel_share_at_full_size():
    """Device 0's share of the long-context workload [1,32,32768,128] cut into 16 chunks of
    2048 for 8 devices (query chunks 0 and 15, as the sequence-parallel bench times it): each
    chunk's attention against the key chunks up to it, merged, checked on sampled rows of
    both chunks (the chunk's first and last rows among them) against the oracle's causal
    attention over the whole sequence."""
    w = workloads.long_prefill()
    q, k, v = w["q"].cuda(), w["k"].cuda(), w["v"].cuda()
    c = 2048
    g = torch.Generator().manual_seed(81)
    for i in (0, 15):
        print(f"case: sequence-parallel share, query chunk {i} of 16", flush=True)
        qi = q[:, :, i * c:(i + 1) * c].contiguous()
        outs, lses = [], []
        for j in range(i + 1):
            kj = k[:, :, j * c:(j + 1) * c].contiguous()
            vj = v[:, :, j * c:(j + 1) * c].contiguous()
            o, l = attn.attn_fwd(qi, kj, vj, causal=(j == i), return_lse=True)
            outs.append(o)
            lses.append(l)
        o, lse = attn.attn_merge(torch.stack(outs), torch.stack(lses), return_lse=True)
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
