"""Parity of grouped K/V heads and the causal sliding window with the fp64 oracle, through
the C ABI: prefill (fp32 and bf16), paged decode and the backward pass.

Query head h reads K/V head h // (H / H_kv); a window w admits keys i - w < j <= i (decode:
the last w cached tokens).  Same tolerances as the plain paths: fp32 max-abs 1e-5; bf16
max-abs 1e-2 and mean-abs 1e-3; gradients within the relative bounds derived in
test_gpu_backward.py.  The gradients' absolute floor is 1e-5 here: a window of one leaves
each row a single key, where the exact dQ and dK vanish and what remains is the fp32
difference dP - D of two 128-term dot products that agree in exact arithmetic (rounding of
order sqrt(128) 2^-24 |dO| |v| ~ 1e-6 per row, times scale |k|; over hundreds of rows the
maximum reaches 1e-6)."""

import math

import numpy as np
import pytest
import torch

import online_softmax_attn_amd as attn
import oracle
import workloads
from metrics import errs, to64

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 1e-2, 1e-3
BF16_LSE_ATOL = 2.0 ** -8
MEAN_REL, MAX_REL, ATOL = 2.0 ** -7, 2.0 ** -6, 1e-5


def gpu_fwd(q, k, v, *, causal, window=0, seq_lens=None, scale=None):
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    attn.attn_fwd(qd, kd, vd, causal=causal, window=window, seq_lens=seq_lens, scale=scale,
                  out=out, lse=lse)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


def valid_rows(B, H, n, lens):
    rows = np.ones((B, H, n), dtype=bool)
    if lens is not None:
        for b, L in enumerate(lens):
            rows[b, :, L:] = False
    return rows


# ------------------------------------------------------------------ prefill, bf16
# (B, H, H_kv, n, causal, window, lens)
BF16_CASES = [
    (1, 4, 1, 300, True, 0, None),           # one K/V head for all query heads
    (1, 4, 2, 300, False, 0, None),
    (2, 6, 3, 513, True, 0, None),
    (2, 8, 2, 257, True, 64, [257, 100]),     # window with lengths and padding poison
    (1, 4, 2, 700, True, 200, None),          # window not a multiple of the tile
    (1, 2, 2, 640, True, 128, None),          # window a multiple of the tile
    (1, 4, 4, 1000, True, 1, None),           # window of one: every row returns its own value
    (1, 8, 1, 333, True, 1000, None),         # window longer than the sequence: plain causal
    (3, 4, 1, 200, True, 37, [1, 150, 200]),
    (2, 32, 8, 300, True, 100, [300, 150]),  # B*H a multiple of 64: eight heads per XCD at a time
]


# the same at head_dim 64
BF16_D64_CASES = [
    (1, 4, 1, 300, True, 0, None),
    (2, 8, 2, 257, True, 64, [257, 100]),
    (1, 4, 2, 700, True, 200, None),
    (1, 4, 4, 1000, True, 1, None),
    (2, 32, 8, 300, True, 100, [300, 150]),
]


@pytest.mark.parametrize("d,B,H,Hkv,n,causal,window,lens",
                         [(128, *c) for c in BF16_CASES] + [(64, *c) for c in BF16_D64_CASES])
def test_bf16_grouped_window(d, B, H, Hkv, n, causal, window, lens):
    q, k, v = workloads.prefill(B, H, n, d, seed=13 * n + H + window, lens=lens,
                                poison=lens is not None, kv_heads=Hkv)
    print(f"case: bf16 d={d} B={B} H={H} Hkv={Hkv} n={n} causal={causal} window={window} lens={lens}",
          flush=True)
    o, lse = gpu_fwd(q, k, v, causal=causal, window=window, seq_lens=lens)
    ro, rl = oracle.attention(q, k, v, causal=causal, window=window, seq_lens=lens)
    rows = valid_rows(B, H, n, lens)
    mx, mean = errs(o, ro, rows)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=0, atol=BF16_LSE_ATOL)
    if lens is not None:
        for b, L in enumerate(lens):
            assert np.all(o[b, :, L:] == 0) and np.all(lse[b, :, L:] == -np.inf)
    if window == 1:
        G = H // Hkv
        want = np.repeat(to64(v), G, axis=1)
        assert np.abs(o - want).max() <= 2.0 ** -8 * np.abs(want).max()


def _sampled_rows(H, n, fixed, per_head, seed):
    """[H, len(fixed) + per_head]: per head the fixed positions plus `per_head` distinct
    seeded random others, sorted."""
    g = torch.Generator().manual_seed(seed)
    fixed = np.asarray(fixed)
    rows = []
    for _ in range(H):
        r = torch.randperm(n, generator=g).numpy()
        r = r[~np.isin(r, fixed)][:per_head]
        rows.append(np.sort(np.concatenate([fixed, r])))
    return np.stack(rows)


@pytest.mark.slow
def test_bf16_window_workload_sampled_rows():
    """The causal window-1024 prefill [1,32,16384,128] as it is timed (seed 6): the GPU on all
    rows; the oracle on sampled rows of every head, among them rows before the window fills
    (i < 1024), on both sides of the window edge and of tile edges, and the last row."""
    q, k, v = workloads.prefill(1, 32, 16384, 128, seed=6)
    print("case: window-1024 prefill [1,32,16384,128], sampled rows", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=True, window=1024)
    fixed = [0, 1, 63, 64, 127, 128, 1022, 1023, 1024, 1025, 1087, 1088, 8191, 8192, 16383]
    rows = _sampled_rows(32, 16384, fixed, 33, seed=66)
    ro, rl = oracle.attention_rows(q, k, v, rows, causal=True, window=1024)
    got = np.stack([o[0, h, rows[h]] for h in range(32)])[None]
    mx, mean = errs(got, ro)
    print(f"sampled rows max-abs {mx:.5f} mean-abs {mean:.2e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    got_l = np.stack([lse[0, h, rows[h]] for h in range(32)])[None]
    np.testing.assert_allclose(got_l, rl, rtol=0, atol=BF16_LSE_ATOL)


@pytest.mark.slow
def test_bf16_grouped_workload_sampled_rows():
    """The grouped-heads causal prefill [4,32,2048,128] with 8 K/V heads as it is timed
    (seed 3): the GPU on all rows; the oracle on 32 rows of every (batch, head), tile edges
    and the last row among them."""
    q, k, v = workloads.prefill(4, 32, 2048, 128, seed=3, kv_heads=8)
    print("case: grouped prefill [4,32,2048,128] H_kv=8, sampled rows", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=True)
    fixed = [0, 63, 64, 127, 128, 1023, 1024, 2047]
    rows = np.stack([_sampled_rows(32, 2048, fixed, 24, seed=67 + b) for b in range(4)])
    ro, rl = oracle.attention_rows(q, k, v, rows, causal=True)
    got = np.stack([np.stack([o[b, h, rows[b, h]] for h in range(32)]) for b in range(4)])
    mx, mean = errs(got, ro)
    print(f"sampled rows max-abs {mx:.5f} mean-abs {mean:.2e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    got_l = np.stack([np.stack([lse[b, h, rows[b, h]] for h in range(32)]) for b in range(4)])
    np.testing.assert_allclose(got_l, rl, rtol=0, atol=BF16_LSE_ATOL)


def test_bf16_window_equals_causal_when_longer_than_sequence():
    q, k, v = workloads.prefill(2, 4, 777, 128, seed=61, kv_heads=2)
    a, la = gpu_fwd(q, k, v, causal=True, window=777)
    b, lb = gpu_fwd(q, k, v, causal=True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_bf16_grouped_equals_repeated_heads():
    """Grouped heads read the shared K/V; repeating each K/V head G times and running plain
    multi-head attention must give the same bits."""
    q, k, v = workloads.prefill(2, 8, 500, 128, seed=62, kv_heads=2)
    a, la = gpu_fwd(q, k, v, causal=True, window=100)
    kr, vr = (x.repeat_interleave(4, dim=1).contiguous() for x in (k, v))
    b, lb = gpu_fwd(q, kr, vr, causal=True, window=100)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


# ------------------------------------------------------------------ prefill, fp32
@pytest.mark.parametrize("d,H,Hkv,n,window,lens", [(64, 4, 2, 100, 16, [100, 37]),
                                                   (128, 2, 1, 130, 0, None),
                                                   (64, 6, 2, 257, 33, None),
                                                   (128, 4, 4, 90, 1, [90, 3])])
def test_fp32_grouped_window(d, H, Hkv, n, window, lens):
    q, k, v = workloads.prefill(2, H, n, d, dtype=torch.float32, seed=n + d + window,
                                qk_scale=4.0, lens=lens, poison=lens is not None, kv_heads=Hkv)
    scale = float(np.float32(1 / math.sqrt(d)))
    print(f"case: fp32 d={d} H={H} Hkv={Hkv} n={n} window={window} lens={lens}", flush=True)
    o, lse = gpu_fwd(q, k, v, causal=True, window=window, seq_lens=lens)
    ro, rl = oracle.attention(q, k, v, scale=scale, causal=True, window=window, seq_lens=lens)
    rows = valid_rows(2, H, n, lens)
    mx, _ = errs(o, ro, rows)
    assert mx <= F32_TOL, mx
    np.testing.assert_allclose(lse[rows], rl[rows], rtol=1e-6, atol=1e-5)


# ------------------------------------------------------------------ paged decode
def gpu_decode(w, *, window=0, kv_split=0):
    q = w.q.cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:2], float("nan"), device="cuda")
    attn.attn_decode_paged(q, w.k_cache.cuda(), w.v_cache.cuda(), w.block_table.cuda(),
                           w.seq_lens.tolist(), max_seq_len=w.max_seq_len, window=window,
                           kv_split=kv_split, out=out, lse=lse)
    torch.cuda.synchronize()
    return to64(out), to64(lse)


def check_decode_lse(lse, rl, group):
    """Groups of 2 or more query heads decode on the matrix cores, whose normaliser sums the
    bf16-rounded weights that enter P.V (as the bf16 prefill does): LSE within 2^-8.  Single
    heads sum fp32 weights on the vector units: LSE within 2e-6 relative."""
    if group >= 2:
        np.testing.assert_allclose(lse, rl, rtol=0, atol=BF16_LSE_ATOL)
    else:
        np.testing.assert_allclose(lse, rl, rtol=2e-6, atol=2e-5)


# (lens, H, H_kv, window, split): group sizes 1 (vector kernel), 2, 3, 4, 8 and 16
# (matrix-core kernel)
DECODE_CASES = [
    ([1, 15, 16, 17], 8, 2, 0, 16), ([33, 250, 256, 257], 8, 8, 20, 32),
    ([1000, 3, 700], 16, 2, 0, 0), ([1000, 3, 700], 16, 2, 100, 0),
    ([4096, 1, 2049], 6, 2, 1500, 256), ([300, 301], 32, 2, 17, 48),
    ([5000, 77], 12, 3, 1024, 64), ([2000], 4, 1, 1, 16), ([517, 9], 16, 4, 9, 0),
]


@pytest.mark.parametrize("lens,H,Hkv,window,split", DECODE_CASES)
def test_decode_grouped_window(lens, H, Hkv, window, split):
    w = workloads.paged(lens, H, 128, seed=sum(lens) + H, poison=True, spare_blocks=2,
                        kv_heads=Hkv)
    print(f"case: decode lens={lens} H={H} Hkv={Hkv} window={window} split={split}", flush=True)
    o, lse = gpu_decode(w, window=window, kv_split=split)
    ro, rl = oracle.decode(w.q, w.k_seqs, w.v_seqs, window=window)
    mx, mean = errs(o, ro)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
    check_decode_lse(lse, rl, H // Hkv)


def test_decode_grouped_workload():
    """The decode workload's lengths with 8 K/V heads for 32 query heads and a 4096 window."""
    g = torch.Generator().manual_seed(4)
    lens = [int(x) for x in torch.randint(1024, 8193, (32,), generator=g)]
    w = workloads.paged(lens, 32, 128, seed=44, max_seq_len=8192, kv_heads=8)
    for window in (0, 4096):
        print(f"case: decode workload H=32 Hkv=8 window={window}", flush=True)
        o, lse = gpu_decode(w, window=window)
        ro, rl = oracle.decode(w.q, w.k_seqs, w.v_seqs, window=window)
        mx, mean = errs(o, ro)
        print(f"max-abs {mx:.5f} mean-abs {mean:.2e}")
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
        check_decode_lse(lse, rl, 4)


@pytest.mark.parametrize("G", [8, 16, 32, 48])
def test_decode_large_groups_on_matrix_cores(G):
    """Grouped heads take the matrix-core kernel (up to 32 heads per wave; 48 = one full and
    one partial set of columns)."""
    lens = [3000, 17, 1024, 555]
    w = workloads.paged(lens, 2 * G, 128, seed=G, poison=True, spare_blocks=1, kv_heads=2,
                        max_seq_len=4096)
    for window, split in ((0, 0), (0, 48), (700, 64), (16, 16)):
        print(f"case: decode G={G} window={window} split={split}", flush=True)
        o, lse = gpu_decode(w, window=window, kv_split=split)
        ro, rl = oracle.decode(w.q, w.k_seqs, w.v_seqs, window=window)
        mx, mean = errs(o, ro)
        assert mx <= BF16_MAX and mean <= BF16_MEAN, (mx, mean)
        check_decode_lse(lse, rl, G)


# ------------------------------------------------------------------ backward
def check_grad(got, ref, mag, name):
    """Element-wise |err| <= 2^-6 * (sum of |terms| of that element) + ATOL, and the mean
    (the bounds of tests/test_gpu_backward.py)."""
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    err = np.abs(got - ref)
    bound = MAX_REL * mag + ATOL
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (name, worst, err[worst], mag[worst])
    assert err.mean() <= MEAN_REL * np.abs(ref).mean() + ATOL, (name, err.mean(), np.abs(ref).mean())


@pytest.mark.parametrize("B,H,Hkv,n,window,lens", [
    (1, 4, 1, 200, 0, None), (2, 4, 2, 257, 64, [257, 100]), (1, 6, 3, 600, 130, None),
    (1, 2, 2, 300, 1, None), (2, 8, 2, 129, 500, [1, 129]),
])
def test_backward_grouped_window(B, H, Hkv, n, window, lens):
    q, k, v = workloads.prefill(B, H, n, 128, seed=17 * n + H, lens=lens, poison=lens is not None,
                                kv_heads=Hkv)
    do = torch.randn(B, H, n, 128, generator=torch.Generator().manual_seed(n)).to(torch.bfloat16)
    print(f"case: bwd B={B} H={H} Hkv={Hkv} n={n} window={window} lens={lens}", flush=True)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.attn_fwd(qd, kd, vd, causal=True, window=window, seq_lens=lens, return_lse=True)
    dq = torch.full(q.shape, float("nan"), device="cuda")
    dk = torch.full(k.shape, float("nan"), device="cuda")
    dv = torch.full(k.shape, float("nan"), device="cuda")
    attn.attn_bwd(qd, kd, vd, o, dod, lse, causal=True, window=window, seq_lens=lens, dq=dq,
                  dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.attention_grad(q, k, v, do, causal=True, window=window, seq_lens=lens)
    mag = oracle.attention_grad_magnitudes(q, k, v, do, causal=True, window=window, seq_lens=lens)
    for name, x, r, a in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, mag):
        x = to64(x)
        check_grad(x, r, a, name)
        if lens is not None:
            for b, L in enumerate(lens):
                assert np.all(x[b, :, L:] == 0), name
