"""Parity of the FP8 E4M3 path (attn_quantize_fp8, attn_fwd_fp8) with the oracle's FP8 loop.

The quantisation is integer work: codes and scales must match the oracle bit for bit (both
divide in fp32 and round to nearest even).  The attention then runs on identical E4M3
operands; the GPU and the oracle's tiled FP8 loop differ by the precision of the score
sums and exponentials.  Element-wise the GPU output must lie within half a bf16 ulp of the
oracle's value (its own output rounding: a dequantised s_V * v8 is in general not a bf16
number) plus 2^-10; mean-abs against the oracle rounded to bf16 within 1e-3; LSE within
2^-8.

The element-wise bound is widened by the oracle's near-tie slack, and the share of elements
that rely on it is bounded (tests/fp8_check.py, whose CPU test shows the check rejects
planted mistakes of an FP8 kernel)."""

import math

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from fp8_check import ACC_REL, TIE_REL, check
from metrics import errs, to64
from oracle import fp8

pytestmark = pytest.mark.gpu


def oracle_quantized(q, k, v, lens):
    return [fp8.quantize_blocks(t, seq_lens=lens) for t in (q, k, v)]


@pytest.mark.parametrize("B,H,n,lens", [(1, 1, 1, None), (2, 3, 100, [100, 37]), (1, 2, 256, None),
                                        (2, 2, 300, [1, 250])])
def test_quantize_codes_and_scales_are_bit_exact(B, H, n, lens):
    x = workloads.prefill(B, H, n, 128, seed=n + B, lens=lens, poison=lens is not None)[0]
    x[0, 0, 0, :5] = 0.0                       # exact zeros (and an all-zero stretch)
    print(f"case: quantize B={B} H={H} n={n} lens={lens}", flush=True)
    xd = x.cuda()
    c_row, s_row = attn.attn_quantize_fp8(xd, seq_lens=lens)
    c_tr, s_tr = attn.attn_quantize_fp8(xd, seq_lens=lens, transpose=True)
    torch.cuda.synchronize()
    vals, sc = fp8.quantize_blocks(x, seq_lens=lens)
    want = fp8.e4m3_encode(vals)
    np.testing.assert_array_equal(s_row.cpu().numpy(), sc)
    np.testing.assert_array_equal(s_tr.cpu().numpy(), sc)
    np.testing.assert_array_equal(c_row.cpu().numpy(), want)
    tr = c_tr.cpu().numpy()
    np.testing.assert_array_equal(tr[..., :n], np.swapaxes(want, 2, 3))
    assert np.all(tr[..., n:] == 0)


def gpu_fp8(q, k, v, *, causal, lens):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    q8, sq = attn.attn_quantize_fp8(qd, seq_lens=lens)
    k8, sk = attn.attn_quantize_fp8(kd, seq_lens=lens)
    v8, sv = attn.attn_quantize_fp8(vd, seq_lens=lens, transpose=True)
    out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    attn.attn_fwd_fp8(q8, k8, v8, sq, sk, sv, causal=causal, seq_lens=lens, out=out, lse=lse)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


def oracle_fp8(q, k, v, *, causal, lens, heads=None):
    (q8, sq), (k8, sk), (v8, sv) = oracle_quantized(q, k, v, lens)
    if heads is not None:  # a slice of query heads (with their K/V heads)
        G = q.shape[1] // k.shape[1]
        kv = sorted({h // G for h in heads})
        q8, sq = q8[:, heads], sq[:, heads]
        k8, sk, v8, sv = k8[:, kv], sk[:, kv], v8[:, kv], sv[:, kv]
    return fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=float(np.float32(1 / math.sqrt(128))),
                             causal=causal, seq_lens=lens, tie_rel=TIE_REL, acc_rel=ACC_REL)


def valid_rows(B, H, n, lens):
    rows = np.ones((B, H, n), dtype=bool)
    if lens is not None:
        for b, L in enumerate(lens):
            rows[b, :, L:] = False
    return rows


# (B, H, H_kv, n, causal, lens)
FP8_CASES = [
    (1, 1, 1, 1, False, None), (1, 2, 2, 64, True, None), (2, 2, 2, 130, True, None),
    (1, 3, 3, 127, False, None), (2, 4, 2, 300, True, [300, 129]), (3, 2, 1, 200, False, [1, 64, 200]),
    (1, 4, 4, 1000, True, None), (2, 8, 2, 257, True, None),
    (2, 32, 8, 200, True, [200, 77]),  # B*H a multiple of 64: eight heads per XCD at a time
]


@pytest.mark.parametrize("B,H,Hkv,n,causal,lens", FP8_CASES)
def test_fp8_forward_matches_oracle_fp8_loop(B, H, Hkv, n, causal, lens):
    q, k, v = workloads.prefill(B, H, n, 128, seed=5 * n + H, lens=lens, poison=lens is not None,
                                kv_heads=Hkv)
    print(f"case: fp8 fwd B={B} H={H} Hkv={Hkv} n={n} causal={causal} lens={lens}", flush=True)
    o, lse = gpu_fp8(q, k, v, causal=causal, lens=lens)
    check(o, lse, oracle_fp8(q, k, v, causal=causal, lens=lens), valid_rows(B, H, n, lens))
    if lens is not None:
        for b, L in enumerate(lens):
            assert np.all(o[b, :, L:] == 0) and np.all(lse[b, :, L:] == -np.inf)


def test_fp8_causal_prefill_workload_sampled_heads():
    """The causal prefill workload [4, 32, 2048, 128]: GPU on all heads, the oracle's FP8 loop
    on 4 heads of batch row 0; the exact attention on the same heads bounds the FP8 error."""
    w = workloads.causal_prefill()
    print("case: fp8 causal prefill [4,32,2048,128]", flush=True)
    o, lse = gpu_fp8(w["q"], w["k"], w["v"], causal=True, lens=None)
    heads = [0, 9, 18, 31]
    ref = oracle_fp8(w["q"][0:1], w["k"][0:1], w["v"][0:1], causal=True, lens=None, heads=heads)
    got = o[0:1][:, heads]
    check(got, lse[0:1][:, heads], ref)
    ex, _ = oracle.attention(w["q"][0:1, heads], w["k"][0:1, heads], w["v"][0:1, heads], causal=True)
    emx, emean = errs(got, ex)
    print(f"vs exact attention: max-abs {emx:.4f} mean-abs {emean:.2e}")
    assert emean <= 2.0 ** -4 * np.abs(to64(w["v"][0:1, heads])).mean()
