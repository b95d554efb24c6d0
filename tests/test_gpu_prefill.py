"""Parity of attn_fwd (C ABI through the ctypes binding) with the fp64 oracle on seeded
inputs: every workload shape, ragged tails, masks, padding poison, and closed forms.

Tolerances: fp32 inputs max-abs <= 1e-5; bf16 inputs max-abs <= 1e-2 and mean-abs <= 1e-3,
against the oracle run on the same bf16-rounded values."""

import math

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import bf16_floor, errs, to64

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 1e-2, 1e-3
# The bf16 path's normaliser l sums the bf16-rounded weights that also enter P.V; each is
# within a relative 2^-8 of its exact value, so |ln l_gpu - ln l| <= 2^-8 to first order.
BF16_LSE_ATOL = 2.0 ** -8


def gpu_fwd(q, k, v, *, causal, seq_lens=None, scale=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full_like(qd, float("nan"))                  # proves every element is written
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    attn.attn_fwd(qd, kd, vd, causal=causal, seq_lens=seq_lens, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


def valid_rows(B, H, n, lens):
    rows = np.ones((B, H, n), dtype=bool)
    if lens is not None:
        for b, L in enumerate(lens):
            rows[b, :, L:] = False
    return rows


def check_padding(o, lse, lens):
    if lens is None:
        return
    for b, L in enumerate(lens):
        assert np.all(o[b, :, L:] == 0)
        assert np.all(lse[b, :, L:] == -np.inf)


# ------------------------------------------------------------------ fp32 path
def test_fp32_toy_workload():
    w = workloads.toy()
    print("case: toy fp32 [1,1,256,64]", flush=True)
    o, lse = gpu_fwd(w["q"], w["k"], w["v"], causal=False)
    ro, rl = oracle.attention(w["q"], w["k"], w["v"], scale=float(np.float32(1 / 8)))
    mx, _ = errs(o, ro)
    assert mx <= F32_TOL, mx
    np.testing.assert_allclose(lse, rl, rtol=1e-6, atol=1e-5)


@pytest.mark.parametrize("poison", [False, True])
def test_fp32_stress_workload(poison):
    w = workloads.stress(poison=poison)
    lens = w["seq_lens"]
    print(f"case: stress fp32 lens={lens} poison={poison}", flush=True)
    o, lse = gpu_fwd(w["q"], w["k"], w["v"], causal=False, seq_lens=lens)
    ro, rl = oracle.attention(w["q"], w["k"], w["v"], scale=0.125, seq_lens=lens)
    rows = valid_rows(4, 4, 1000, lens)
    mx, _ = errs(o, ro, rows)
    assert mx <= F32_TOL, mx
    check_padding(o, lse, lens)
    # the length-1 row returns its only value exactly
    b1 = lens.index(1)
    assert np.array_equal(o[b1, :, 0], to64(w["v"][b1, :, 0]))
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=1e-6)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n,causal,lens", [(1, False, None), (33, True, None), (100, True, [100, 37]),
                                           (257, False, [5, 257]), (130, True, [1, 64])])
def test_fp32_shapes(d, n, causal, lens):
    q, k, v = workloads.prefill(2, 3, n, d, dtype=torch.float32, seed=n + d, qk_scale=4.0,
                                lens=lens, poison=lens is not None)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"case: fp32 d={d} n={n} causal={causal} lens={lens}", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=causal, seq_lens=lens)
    ro, _ = oracle.attention(q, k, v, scale=scale, causal=causal, seq_lens=lens)
    mx, _ = errs(o, ro, valid_rows(2, 3, n, lens))
    assert mx <= F32_TOL, mx
    check_padding(o, lse, lens)


# ------------------------------------------------------------------ bf16 path
BF16_CASES = [
    (1, 1, 1, False, None), (1, 2, 17, True, None), (2, 2, 64, True, None), (1, 3, 127, False, None),
    (2, 1, 128, True, None), (1, 2, 129, True, None), (2, 2, 300, False, None), (1, 2, 300, True, None),
    (3, 2, 200, True, [1, 150, 200]), (2, 2, 257, False, [64, 129]), (1, 1, 1000, True, None),
    # B*H a multiple of 64: the grid runs eight heads per XCD at a time
    (2, 32, 300, True, [300, 77]), (1, 64, 130, False, None),
]


@pytest.mark.parametrize("B,H,n,causal,lens", BF16_CASES)
def test_bf16_shapes(B, H, n, causal, lens):
    q, k, v = workloads.prefill(B, H, n, 128, seed=7 * n + B, lens=lens, poison=lens is not None)
    print(f"case: bf16 B={B} H={H} n={n} causal={causal} lens={lens}", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=causal, seq_lens=lens)
    ro, rl = oracle.attention(q, k, v, causal=causal, seq_lens=lens)
    rows = valid_rows(B, H, n, lens)
    mx, mean = errs(o, ro, rows)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    check_padding(o, lse, lens)
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=0, atol=BF16_LSE_ATOL)


@pytest.mark.parametrize("B,H,n,causal,lens", [
    (4, 16, 2048, True, [2048, 1000, 300, 17]),   # 1024 query tiles, many of them padding
    (2, 40, 1600, False, [1600, 999]),            # 1040 tiles, no mask, ragged lengths
    (3, 24, 1100, True, None),                    # 648 tiles: a partial last round
])
def test_bf16_more_tiles_than_resident_workgroups(B, H, n, causal, lens):
    """Shapes with more query tiles than the GPU holds workgroups at once (two per CU), with
    padding tiles (wholly past a length) among the later ones, ragged lengths, no mask, and
    a partial last wave of workgroups."""
    q, k, v = workloads.prefill(B, H, n, 128, seed=3 * n + H, lens=lens, poison=lens is not None)
    print(f"case: bf16 many tiles B={B} H={H} n={n} causal={causal} lens={lens}", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=causal, seq_lens=lens)
    ro, rl = oracle.attention(q, k, v, causal=causal, seq_lens=lens)
    rows = valid_rows(B, H, n, lens)
    mx, mean = errs(o, ro, rows)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    check_padding(o, lse, lens)
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=0, atol=BF16_LSE_ATOL)


# head_dim 64: the same kernel instantiated for half the dims (half the operand registers,
# accumulators, tile bytes and products per step); the same bf16 bar
BF16_D64_CASES = [
    (1, 1, 1, False, None), (1, 2, 17, True, None), (2, 2, 129, True, None),
    (2, 2, 300, False, [300, 77]), (3, 2, 200, True, [1, 150, 200]), (1, 4, 1000, True, None),
    (2, 32, 300, True, [300, 77]), (4, 16, 2048, True, [2048, 1000, 300, 17]),
]


@pytest.mark.parametrize("B,H,n,causal,lens", BF16_D64_CASES)
def test_bf16_head_dim_64(B, H, n, causal, lens):
    q, k, v = workloads.prefill(B, H, n, 64, seed=5 * n + B + H, lens=lens, poison=lens is not None)
    print(f"case: bf16 d=64 B={B} H={H} n={n} causal={causal} lens={lens}", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=causal, seq_lens=lens)
    ro, rl = oracle.attention(q, k, v, causal=causal, seq_lens=lens)
    rows = valid_rows(B, H, n, lens)
    mx, mean = errs(o, ro, rows)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    check_padding(o, lse, lens)
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=0, atol=BF16_LSE_ATOL)


def test_bf16_head_dim_64_deterministic():
    q, k, v = workloads.prefill(2, 4, 777, 64, seed=43)
    a, _ = gpu_fwd(q, k, v, causal=True)
    b, _ = gpu_fwd(q, k, v, causal=True)
    assert np.array_equal(a, b)


def test_bf16_causal_prefill_workload():
    w = workloads.causal_prefill()
    print("case: causal prefill bf16 [4,32,2048,128]", flush=True)
    o, lse = gpu_fwd(w["q"], w["k"], w["v"], causal=True)
    ro, rl = oracle.attention(w["q"], w["k"], w["v"], causal=True)
    mx, mean = errs(o, ro)
    print(f"max-abs {mx:.5f} mean-abs {mean:.2e} bf16 output floor {bf16_floor(ro):.5f}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=BF16_LSE_ATOL)


def test_bf16_causal_prefill_key_shift_invariance():
    """K + 1 w^T shifts each row's scores by a constant: the output must not move beyond
    the bf16 tolerance (the shifted keys are re-rounded to bf16, so compare to the oracle)."""
    q, k, v = workloads.prefill(2, 4, 2048, 128, seed=31)
    w = torch.randn(128, generator=torch.Generator().manual_seed(32)).to(torch.bfloat16)
    k2 = (k.float() + w.float()).to(torch.bfloat16)
    o1, _ = gpu_fwd(q, k, v, causal=True)
    o2, _ = gpu_fwd(q, k2, v, causal=True)
    ro, _ = oracle.attention(q, k, v, causal=True)
    for o in (o1, o2):
        mx, mean = errs(o, ro)
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)


def test_bf16_deterministic():
    q, k, v = workloads.prefill(2, 4, 777, 128, seed=41)
    a, _ = gpu_fwd(q, k, v, causal=True)
    b, _ = gpu_fwd(q, k, v, causal=True)
    assert np.array_equal(a, b)


@pytest.mark.slow
def test_bf16_long_context_sampled_rows():
    w = workloads.long_prefill()
    print("case: long-context bf16 [1,32,32768,128], 64 sampled rows per head", flush=True)
    o, lse = gpu_fwd(w["q"], w["k"], w["v"], causal=True)
    rows = w["rows"].numpy()
    ro, rl = oracle.attention_rows(w["q"], w["k"], w["v"], rows, causal=True)
    got = np.stack([o[0, h, rows[h]] for h in range(32)])[None]
    mx, mean = errs(got, ro)
    print(f"sampled rows max-abs {mx:.5f} mean-abs {mean:.2e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    got_l = np.stack([lse[0, h, rows[h]] for h in range(32)])[None]
    np.testing.assert_allclose(got_l, rl, rtol=0, atol=BF16_LSE_ATOL)


@pytest.mark.slow
def test_bf16_long_context_zero_queries_give_prefix_means():
    """Q = 0 makes every admitted score equal, so row i's output is the mean of v_0..v_i:
    checked on all 32768 rows of every head against an fp64 cumulative sum."""
    w = workloads.long_prefill()
    q = torch.zeros_like(w["q"])
    o, lse = gpu_fwd(q, w["k"], w["v"], causal=True)
    v = to64(w["v"])
    want = np.cumsum(v, axis=2) / np.arange(1, 32769)[None, None, :, None]
    mx, mean = errs(o, want)
    print(f"prefix-mean max-abs {mx:.5f} mean-abs {mean:.2e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse[0], np.broadcast_to(np.log(np.arange(1, 32769)), (32, 32768)),
                               rtol=1e-6, atol=1e-5)
