"""Materialised fp64 attention: the plain definition, one (batch, head) at a time.

TEST INFRASTRUCTURE (see the package docstring): never imported by the product path.

Definition followed (pierluigilucio.it "Sviluppo AI ed Algebra Lineare", section
"Formulazione Algebrica della Self-Attention", steps 1-4; maeste.it attention-matrix page,
the formula and its "softmax" and "V" paragraphs):

    S_ij = scale * <q_i, k_j>                     scale = 1/sqrt(d_head) by default
    A_ij = exp(S_ij) / sum_{j' valid} exp(S_ij')  over the keys admitted by the mask
    o_i  = sum_j A_ij v_j

Masks: a causal mask gives query i the keys j <= i (maeste.it: future tokens are set to
-inf before the softmax); a length mask of n_b admits queries and keys < n_b only.  Two
variants the pages name as complements of exact attention without defining them
(aimpact.prandi.net FlashAttention page, "Impatto pratico": grouped-query attention and
sliding-window attention; maeste.it: a sliding window limits each token's reach) are read
in their plainest form: with H query heads and H_kv key/value heads, query head h uses K/V
head h // (H / H_kv); a causal window of w admits keys i - w < j <= i.  The
maximum is subtracted before exponentiating (el-ai.com section 1: it multiplies numerator
and denominator by the same factor).  A row with no admitted key has no distribution
(el-ai.com section 5 asks for an explicit convention): its output is 0 and its
log-sum-exp is -inf.

Everything is materialised — S, the weights, the normaliser — exactly the three-pass
computation the tiled method avoids; that is what makes it a reference.
"""

from __future__ import annotations

import math

import numpy as np


def to_f64(x) -> np.ndarray:
    """Exact upcast of a NumPy array or a CPU/GPU torch tensor (fp32 or bf16) to float64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    try:  # torch tensor: bf16 -> fp32 is exact, fp32 -> fp64 is exact
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def attend(S: np.ndarray, V: np.ndarray, valid: np.ndarray | None = None):
    """Row softmax of scaled scores followed by the weighted sum of values.

    S: [nq, nk] fp64 scores (already scaled).  V: [nk, dv].  valid: bool [nq, nk] or None.
    Returns (O [nq, dv], lse [nq]) with lse_i = log sum_{j valid} exp(S_ij) (natural log).
    Rows with no valid key: O = 0, lse = -inf.
    """
    S = np.asarray(S, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if valid is None:
        valid = np.ones(S.shape, dtype=bool)
    has_key = valid.any(axis=1)
    Sm = np.where(valid, S, -np.inf)
    m = np.where(has_key, Sm.max(axis=1, initial=-np.inf), 0.0)
    W = np.where(valid, np.exp(Sm - m[:, None]), 0.0)
    l = W.sum(axis=1)
    safe_l = np.where(has_key, l, 1.0)
    O = (W @ V) / safe_l[:, None]
    O[~has_key] = 0.0
    lse = np.where(has_key, m + np.log(safe_l), -np.inf)
    return O, lse


def _valid(nq: int, nk: int, causal: bool, window: int = 0) -> np.ndarray:
    """Admitted (query, key) pairs of one square block (query i, key j)."""
    qi = np.arange(nq)[:, None]
    kj = np.arange(nk)[None, :]
    ok = np.ones((nq, nk), dtype=bool)
    if causal:
        ok &= kj <= qi
    if window:
        ok &= kj > qi - window
    return ok


def _group(H: int, Hkv: int) -> int:
    if Hkv <= 0 or H % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    return H // Hkv


def attention(q, k, v, *, scale: float | None = None, causal: bool = False, seq_lens=None,
              window: int = 0):
    """Prefill attention: q [B, H, n, d]; k, v [B, H_kv, n, d] with H a multiple of H_kv.

    seq_lens: optional length per batch row (host ints); queries and keys at positions
    >= n_b are padding: their outputs are 0 / lse -inf and they are never read.
    window: 0 for none, else keys i - window < j (with causal: the last `window` tokens).
    Returns (O [B, H, n, d] fp64, LSE [B, H, n] fp64).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, n, d = q.shape
    G = _group(H, k.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [n] * B if seq_lens is None else [int(x) for x in seq_lens]
    O = np.zeros((B, H, n, v.shape[-1]))
    LSE = np.full((B, H, n), -np.inf)
    for b in range(B):
        L = lens[b]
        if L <= 0:
            continue
        valid = _valid(L, L, causal, window)
        for h in range(H):
            S = scale * (q[b, h, :L] @ k[b, h // G, :L].T)
            O[b, h, :L], LSE[b, h, :L] = attend(S, v[b, h // G, :L], valid)
    return O, LSE


def attention_chunk(q, k, v, q_start: int, *, scale: float | None = None, causal: bool = False,
                    window: int = 0):
    """Attention of a chunk of queries at positions q_start .. q_start + n_q - 1 of a key
    sequence: q [B, H, n_q, d]; k, v [B, H_kv, n_kv, d].  The causal mask (maeste.it: future
    keys set to -inf) and the window compare key positions with those query positions.
    Returns (O [B, H, n_q, d] fp64, LSE [B, H, n_q] fp64).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, nq, d = q.shape
    nk = k.shape[2]
    if not 0 <= q_start <= nk - nq:
        raise ValueError("the chunk must lie inside the key sequence")
    G = _group(H, k.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = q_start + np.arange(nq)[:, None]
    kj = np.arange(nk)[None, :]
    valid = np.ones((nq, nk), dtype=bool)
    if causal:
        valid &= kj <= pos
    if window:
        valid &= kj > pos - window
    O = np.zeros((B, H, nq, v.shape[-1]))
    LSE = np.full((B, H, nq), -np.inf)
    for b in range(B):
        for h in range(H):
            S = scale * (q[b, h] @ k[b, h // G].T)
            O[b, h], LSE[b, h] = attend(S, v[b, h // G], valid)
    return O, LSE


def attention_rows(q, k, v, rows, *, scale: float | None = None, causal: bool = False, seq_lens=None,
                   window: int = 0):
    """Attention for selected query rows only (the sampled check of long sequences).

    rows: int array [B, H, R] (or [H, R] when B == 1) of query positions.
    Returns (O [B, H, R, d], LSE [B, H, R]).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, H, n, d = q.shape
    G = _group(H, k.shape[1])
    rows = np.asarray(rows)
    if rows.ndim == 2:
        rows = rows[None]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [n] * B if seq_lens is None else [int(x) for x in seq_lens]
    R = rows.shape[-1]
    O = np.zeros((B, H, R, v.shape[-1]))
    LSE = np.full((B, H, R), -np.inf)
    for b in range(B):
        L = lens[b]
        for h in range(H):
            r = rows[b, h]
            S = scale * (q[b, h, r] @ k[b, h // G, :L].T)
            valid = np.ones((R, L), dtype=bool)
            if causal:
                valid &= np.arange(L)[None, :] <= r[:, None]
            if window:
                valid &= np.arange(L)[None, :] > r[:, None] - window
            valid &= (r < L)[:, None]
            O[b, h], LSE[b, h] = attend(S, v[b, h // G, :L], valid)
    return O, LSE


def decode(q, k_seqs, v_seqs, *, scale: float | None = None, window: int = 0):
    """One query per sequence against that sequence's cache.

    q: [B, H, d]; k_seqs / v_seqs: length-B lists of [H_kv, len_b, d] contiguous caches.
    The query sits at position len_b - 1: it admits every cached key, or with a window the
    keys j > len_b - 1 - window.  Returns (O [B, H, d], LSE [B, H]).
    """
    q = to_f64(q)
    B, H, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, H, d))
    LSE = np.full((B, H), -np.inf)
    for b in range(B):
        kb, vb = to_f64(k_seqs[b]), to_f64(v_seqs[b])
        G = _group(H, kb.shape[0])
        L = kb.shape[1]
        valid = np.ones((1, L), dtype=bool)
        if window:
            valid &= np.arange(L)[None, :] > L - 1 - window
        for h in range(H):
            S = scale * (q[b, h][None, :] @ kb[h // G].T)
            o, lse = attend(S, vb[h // G], valid)
            O[b, h], LSE[b, h] = o[0], lse[0]
    return O, LSE
