"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out (casts, padding, paging); it holds
none of the attention arithmetic, so both the GPU path's tests and the CPU oracle can use
it.  Every draw comes from ``torch.Generator('cpu').manual_seed(seed)`` in a fixed order, in
fp32, then cast (bf16 casts round to nearest even), so a seed names one input set exactly.

Workloads (the shapes the method's pages reason about; no public dataset is involved):
  toy        B=1, H=1, n=256, d=64, fp32, Q/K/V ~ N(0,1), no mask
  stress     B=4, H=4, n=1000, d=64, fp32, lengths a seeded permutation of (1,17,128,1000),
             Q and K ~ 40 N(0,1) (scaled scores reach the thousands), V ~ U(-3,3)
  prefill    B=4, H=32, n=2048, d=128, bf16 N(0,1), causal
  decode     B=32 sequences, H=32, d=128, lengths U{1024..8192}, bf16 N(0,1), paged in
             16-token blocks placed by a seeded permutation of the pool
  long       B=1, H=32, n=32768, d=128, bf16 N(0,1), causal; 64 sampled query rows per head
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

STRESS_LENGTHS = (1, 17, 128, 1000)

# name -> (seed, description)
WORKLOADS = {
    "toy": (1, "B=1 H=1 n=256 d=64 fp32 N(0,1), no mask"),
    "stress": (2, "B=4 H=4 n=1000 d=64 fp32, lengths perm(1,17,128,1000), Q,K x40, V U(-3,3), non-causal"),
    "prefill": (3, "B=4 H=32 n=2048 d=128 bf16 N(0,1), causal"),
    "decode": (4, "B=32 H=32 d=128 bf16, KV lengths U{1024..8192}, 16-token pages, permuted pool"),
    "long": (5, "B=1 H=32 n=32768 d=128 bf16 N(0,1), causal, 64 sampled rows per head"),
}


def _gen(seed: int) -> torch.Generator:
    return torch.Generator("cpu").manual_seed(int(seed))


def _cast(x: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    return x if dtype == torch.float32 else x.to(dtype)


# --------------------------------------------------------------------------- prefill
def prefill(B, H, n, d, *, dtype=torch.bfloat16, seed=0, qk_scale=1.0, v_uniform=None,
            lens=None, poison=False, kv_heads=None):
    """Q [B, H, n, d], then K and V [B, kv_heads, n, d] (kv_heads defaults to H), drawn in
    the order Q, K, V.

    qk_scale multiplies the N(0,1) draws of Q and K; v_uniform=a draws V ~ U(-a, a)
    instead of N(0,1).  lens (optional, host ints) marks positions >= n_b as padding;
    with poison=True those positions of Q, K and V are set to NaN after the draws.
    """
    g = _gen(seed)
    Hkv = H if kv_heads is None else int(kv_heads)
    q = torch.randn(B, H, n, d, generator=g) * qk_scale
    k = torch.randn(B, Hkv, n, d, generator=g) * qk_scale
    if v_uniform is None:
        v = torch.randn(B, Hkv, n, d, generator=g)
    else:
        v = torch.rand(B, Hkv, n, d, generator=g) * (2 * v_uniform) - v_uniform
    q, k, v = _cast(q, dtype), _cast(k, dtype), _cast(v, dtype)
    if poison and lens is not None:
        for b, L in enumerate(lens):
            for t in (q, k, v):
                t[b, :, int(L):] = float("nan")
    return q, k, v


def toy(seed=1):
    q, k, v = prefill(1, 1, 256, 64, dtype=torch.float32, seed=seed)
    return dict(q=q, k=k, v=v, seq_lens=None, causal=False)


def stress(seed=2, poison=False):
    g = _gen(seed)
    perm = torch.randperm(4, generator=g)
    lens = [STRESS_LENGTHS[int(i)] for i in perm]
    q = torch.randn(4, 4, 1000, 64, generator=g) * 40
    k = torch.randn(4, 4, 1000, 64, generator=g) * 40
    v = torch.rand(4, 4, 1000, 64, generator=g) * 6 - 3
    if poison:
        for b, L in enumerate(lens):
            for t in (q, k, v):
                t[b, :, L:] = float("nan")
    return dict(q=q, k=k, v=v, seq_lens=lens, causal=False)


def causal_prefill(seed=3):
    q, k, v = prefill(4, 32, 2048, 128, dtype=torch.bfloat16, seed=seed)
    return dict(q=q, k=k, v=v, seq_lens=None, causal=True)


def long_prefill(seed=5, rows_per_head=64):
    g = _gen(seed)
    B, H, n, d = 1, 32, 32768, 128
    q = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    rows = torch.stack([torch.randperm(n, generator=g)[:rows_per_head] for _ in range(H)])
    return dict(q=q, k=k, v=v, seq_lens=None, causal=True, rows=rows)


# --------------------------------------------------------------------------- paged decode
@dataclass
class PagedDecode:
    q: torch.Tensor            # [B, H, d]
    k_seqs: list               # B tensors [H_kv, len_b, d] (contiguous, for the oracle)
    v_seqs: list
    k_cache: torch.Tensor      # [num_blocks, H_kv, block_size, d]
    v_cache: torch.Tensor
    block_table: torch.Tensor  # int32 [B, max_blocks_per_seq], -1 past a sequence's end
    seq_lens: torch.Tensor     # int32 [B]
    block_size: int
    max_seq_len: int

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def paged(lens, H, d, *, seed=0, block_size=16, dtype=torch.bfloat16, max_seq_len=None,
          poison=False, spare_blocks=0, kv_heads=None):
    """One query per sequence and a paged K/V pool holding each sequence's cache.

    Draw order: Q [B,H,d]; then for each sequence b: K_b [H_kv,len_b,d], V_b [H_kv,len_b,d]
    (H_kv = kv_heads, default H);
    then a permutation of the pool's blocks.  Logical block i of sequence b (in the order
    sequence 0's blocks, sequence 1's blocks, ...) is stored at the physical block the
    permutation gives.  Slots past a sequence's length in its last block hold 0 (NaN with
    poison=True); spare_blocks extra pool blocks nobody references hold 0 (NaN with poison).
    """
    lens = [int(x) for x in lens]
    if max_seq_len is None:
        max_seq_len = max(lens)
    return _paged_from(_gen(seed), lens, H, d, block_size, max_seq_len=max_seq_len,
                       poison=poison, dtype=dtype, spare_blocks=spare_blocks, kv_heads=kv_heads)


def paged_decode(seed=4, poison=False):
    """The decode workload: lengths U{1024..8192} for 32 sequences, H=32, d=128, bf16.

    The lengths are the generator's first draw; the rest follows `paged`'s order.
    """
    B, H, d, bs = 32, 32, 128, 16
    g = _gen(seed)
    lens = [int(x) for x in torch.randint(1024, 8193, (B,), generator=g)]
    return _paged_from(g, lens, H, d, bs, max_seq_len=8192, poison=poison)


def _paged_from(g, lens, H, d, block_size, *, max_seq_len, poison=False, dtype=torch.bfloat16,
                spare_blocks=0, kv_heads=None):
    B = len(lens)
    q = _cast(torch.randn(B, H, d, generator=g), dtype)
    H = H if kv_heads is None else int(kv_heads)  # the cache holds the K/V heads
    k_seqs, v_seqs = [], []
    for L in lens:
        k_seqs.append(_cast(torch.randn(H, L, d, generator=g), dtype))
        v_seqs.append(_cast(torch.randn(H, L, d, generator=g), dtype))
    nblk = [math.ceil(L / block_size) for L in lens]
    total = sum(nblk) + spare_blocks
    perm = torch.randperm(total, generator=g)
    max_blocks = math.ceil(max_seq_len / block_size)
    fill = float("nan") if poison else 0.0
    k_cache = torch.full((total, H, block_size, d), fill, dtype=dtype)
    v_cache = torch.full((total, H, block_size, d), fill, dtype=dtype)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    base = 0
    for b, L in enumerate(lens):
        phys = perm[base:base + nblk[b]]
        table[b, :nblk[b]] = phys.to(torch.int32)
        padded = nblk[b] * block_size
        for src, dst in ((k_seqs[b], k_cache), (v_seqs[b], v_cache)):
            buf = torch.full((H, padded, d), fill, dtype=dtype)
            buf[:, :L] = src
            dst[phys] = buf.view(H, nblk[b], block_size, d).permute(1, 0, 2, 3)
        base += nblk[b]
    return PagedDecode(q=q, k_seqs=k_seqs, v_seqs=v_seqs, k_cache=k_cache, v_cache=v_cache,
                       block_table=table, seq_lens=torch.tensor(lens, dtype=torch.int32),
                       block_size=block_size, max_seq_len=max_seq_len)
