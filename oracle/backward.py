"""Gradients of exact attention, materialised in fp64 — TEST INFRASTRUCTURE.

pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (section "Ricalcolo nel Backward Pass")
describes the backward pass of the tiled method: it keeps only the per-row normalisation
statistics of the forward pass and recomputes the score and probability blocks from Q, K
and V.  What that backward pass computes is the plain derivative of the attention output;
the same page names the tool ("Matrici Jacobiane", the multivariate chain rule).  Written
out for L = sum(O * dO) with O = P V and P = softmax(S) row-wise, S = scale * Q K^T:

    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)      (Jacobian of a softmax row applied to dP)
    dQ = scale * dS K        dK = scale * dS^T Q

Masked pairs have P = 0 and so carry no gradient; a query row with no admitted key (length
padding) has O = 0 and contributes nothing.  Everything is materialised per (batch, head),
in float64.  Pinned in tests/test_oracle_backward.py by 50-digit finite differences of the
forward definition and by closed forms.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _group, _valid, to_f64


def _probabilities(S: np.ndarray, valid: np.ndarray) -> np.ndarray:
    has_key = valid.any(axis=1)
    Sm = np.where(valid, S, -np.inf)
    m = np.where(has_key, Sm.max(axis=1, initial=-np.inf), 0.0)
    W = np.where(valid, np.exp(Sm - m[:, None]), 0.0)
    l = W.sum(axis=1)
    return W / np.where(has_key, l, 1.0)[:, None]


def attention_grad(q, k, v, dout, *, scale: float | None = None, causal: bool = False,
                   seq_lens=None, window: int = 0):
    """(dQ, dK, dV) of sum(attention(q, k, v) * dout); q, dout [B, H, n, d], k, v
    [B, H_kv, n, d].  With grouped heads a K/V head's gradient sums over its query heads."""
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    B, H, n, d = q.shape
    G = _group(H, k.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [n] * B if seq_lens is None else [int(x) for x in seq_lens]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = lens[b]
        if L <= 0:
            continue
        valid = _valid(L, L, causal, window)
        for h in range(H):
            hk = h // G
            Q, K, V, dO = q[b, h, :L], k[b, hk, :L], v[b, hk, :L], dout[b, h, :L]
            P = _probabilities(scale * (Q @ K.T), valid)
            dP = dO @ V.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dv[b, hk, :L] += P.T @ dO
            dq[b, h, :L] = scale * (dS @ K)
            dk[b, hk, :L] += scale * (dS.T @ Q)
    return dq, dk, dv


def attention_grad_magnitudes(q, k, v, dout, *, scale: float | None = None, causal: bool = False,
                              seq_lens=None, window: int = 0):
    """Per-element sums of the absolute values of the terms each gradient element adds up,
    in the decomposition written above (a tolerance scale for evaluations that round some
    factor of every term):

        |dV|_jc = sum_i P_ij |dO_ic|
        |dQ|_ic = scale * sum_j P_ij (|dP_ij| + D+_i) |K_jc|
        |dK|_jc = scale * sum_i P_ij (|dP_ij| + D+_i) |Q_ic|

    with D+_i = sum_c |dO_ic O_ic| bounding the row term D_i = sum_k P_ik dP_ik = <dO_i, O_i>.
    By the triangle inequality each is at least the magnitude of the gradient element it
    belongs to.  Returns (Aq, Ak, Av) shaped like (dQ, dK, dV)."""
    q, k, v, dout = to_f64(q), to_f64(k), to_f64(v), to_f64(dout)
    B, H, n, d = q.shape
    G = _group(H, k.shape[1])
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = [n] * B if seq_lens is None else [int(x) for x in seq_lens]
    aq, ak, av = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        L = lens[b]
        if L <= 0:
            continue
        valid = _valid(L, L, causal, window)
        for h in range(H):
            hk = h // G
            Q, K, V, dO = q[b, h, :L], k[b, hk, :L], v[b, hk, :L], dout[b, h, :L]
            P = _probabilities(scale * (Q @ K.T), valid)
            O = P @ V
            d_plus = np.abs(dO * O).sum(axis=1, keepdims=True)
            T = P * (np.abs(dO @ V.T) + d_plus)
            av[b, hk, :L] += P.T @ np.abs(dO)
            aq[b, h, :L] = scale * (T @ np.abs(K))
            ak[b, hk, :L] += scale * (T.T @ np.abs(Q))
    return aq, ak, av
