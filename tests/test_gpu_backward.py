"""Parity of attn_bwd with the oracle's fp64 gradients, on seeded inputs: the GPU forward
supplies o and lse (as in training), the GPU backward recomputes the weights from them.

Tolerance (derived from the arithmetic): every gradient element is a sum of terms in each
of which one factor carries bf16 rounding — the weight P or dS packed for the MFMA (relative
2^-9), the bf16 output O inside D = <dO, O> (2^-9), and the forward's log-sum-exp, whose
normaliser summed bf16-rounded weights (2^-9).  Per term that is under 2^-7 relative, so
each element is held to 2^-6 of the sum of the absolute values of its own terms (the
oracle's attention_grad_magnitudes), plus an absolute 1e-6 for the fp32 accumulation order
where the exact gradient vanishes (a single key sends no gradient to q or k, but D and dP
are summed in different orders).  The tensor mean is held to 2^-7 of the reference mean."""

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import to64

pytestmark = pytest.mark.gpu

MEAN_REL, MAX_REL, ATOL = 2.0 ** -7, 2.0 ** -6, 1e-6


def run(B, H, n, causal, lens, seed):
    q, k, v = workloads.prefill(B, H, n, 128, seed=seed, lens=lens, poison=lens is not None)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(B, H, n, 128, generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd(qd, kd, vd, causal=causal, seq_lens=lens, return_lse=True)
    grads = [torch.full(q.shape, float("nan"), device="cuda") for _ in range(3)]
    attn.attn_bwd(qd, kd, vd, o, dod, lse, causal=causal, seq_lens=lens, dq=grads[0],
                  dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return (q, k, v, do), [to64(x) for x in grads]


def check(got, ref, mag, name):
    """Element-wise |err| <= 2^-6 * (sum of |terms| of that element) + 1e-6, and the mean."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = np.abs(got - ref)
    bound = MAX_REL * mag + ATOL
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    print(f"{name}: max err/bound {float((err / bound).max()):.3f}; max err {err.max():.2e}")
    assert np.all(err <= bound), (name, worst, err[worst], mag[worst])
    assert err.mean() <= MEAN_REL * np.abs(ref).mean() + ATOL, (name, err.mean(), np.abs(ref).mean())


CASES = [(1, 1, 1, False, None), (1, 1, 64, False, None), (1, 2, 64, True, None),
         (2, 2, 130, True, None), (2, 2, 200, False, [77, 200]), (3, 2, 257, True, [1, 100, 257]),
         (1, 4, 1000, True, None),
         (2, 32, 200, True, [200, 77])]  # B*H a multiple of 64: eight heads per XCD at a time


@pytest.mark.parametrize("B,H,n,causal,lens", CASES)
def test_backward_shapes(B, H, n, causal, lens):
    print(f"case: bwd B={B} H={H} n={n} causal={causal} lens={lens}", flush=True)
    (q, k, v, do), got = run(B, H, n, causal, lens, seed=11 * n + B)
    ref = oracle.attention_grad(q, k, v, do, causal=causal, seq_lens=lens)
    mag = oracle.attention_grad_magnitudes(q, k, v, do, causal=causal, seq_lens=lens)
    for name, x, r, a in zip(("dq", "dk", "dv"), got, ref, mag):
        check(x, r, a, name)
        if lens is not None:
            for b, L in enumerate(lens):
                assert np.all(x[b, :, L:] == 0), name


@pytest.mark.slow
def test_backward_causal_prefill_shape():
    """[4, 32, 2048, 128] causal; oracle on the first 16 heads of batch row 0."""
    print("case: bwd [4,32,2048,128] causal", flush=True)
    (q, k, v, do), got = run(4, 32, 2048, True, None, seed=3)
    sl = (slice(0, 1), slice(0, 16))
    ref = oracle.attention_grad(q[sl], k[sl], v[sl], do[sl], causal=True)
    mag = oracle.attention_grad_magnitudes(q[sl], k[sl], v[sl], do[sl], causal=True)
    for name, x, r, a in zip(("dq", "dk", "dv"), got, ref, mag):
        check(x[sl], r, a, name)


def test_backward_closed_forms():
    """sum_j dK_j = 0 (a shift of every key changes nothing) and sum_j dV_j = sum_i dO_i
    (a shift of every value shifts every output), up to the weights' bf16 rounding."""
    (q, k, v, do), (dq, dk, dv) = run(2, 3, 333, True, None, seed=21)
    tot = np.abs(dk).sum(axis=2)
    assert np.all(np.abs(dk.sum(axis=2)) <= MEAN_REL * tot + 1e-6)
    want = to64(do).sum(axis=2)
    assert np.all(np.abs(dv.sum(axis=2) - want) <= MEAN_REL * np.abs(to64(do)).sum(axis=2))


def test_backward_deterministic():
    _, a = run(1, 2, 300, True, None, seed=31)
    _, b = run(1, 2, 300, True, None, seed=31)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_workspace_contents_unused():
    """The workspace is scratch: what it holds before the call (zero bytes, then NaN bytes)
    never reaches the gradients, also with padding rows and query tiles wholly past a
    sequence's end (length 40 of 300 leaves two of its three 128-row tiles empty)."""
    B, H, n, lens = 2, 2, 300, [300, 40]
    print(f"case: bwd workspace poison B={B} H={H} n={n} lens={lens}", flush=True)
    q, k, v = workloads.prefill(B, H, n, 128, seed=41, lens=lens, poison=True)
    g = torch.Generator().manual_seed(42)
    do = torch.randn(B, H, n, 128, generator=g).to(torch.bfloat16).cuda()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o, lse = attn.attn_fwd(qd, kd, vd, causal=True, seq_lens=lens, return_lse=True)
    need = attn.attn_bwd_workspace_bytes(B, H, n)
    outs = []
    for fill in (0, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")
        outs.append(attn.attn_bwd(qd, kd, vd, o, do, lse, causal=True, seq_lens=lens, workspace=ws))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert bool(torch.isfinite(a).all())
        assert torch.equal(a, b)
