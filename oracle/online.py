"""The running (m, l, u) summary of one attention row, in fp64 — TEST INFRASTRUCTURE.

Follows el-ai.com "Attenzione: softmax online, riscalamento e memoria":
  * section 2: after a prefix of keys keep m (prefix maximum), l (sum of exp(s - m)) and
    u (the same sum weighted by the values).  For a new pair (s, v) the new maximum is
    m' = max(m, s); both l AND u are multiplied by exp(m - m') and only then is the new
    key's exp(s - m') and exp(s - m') * v added.  The recurrence here starts from the state
    of no key at all, (m, l, u) = (-inf, 0, 0), whose carry factor is taken as 0, so the
    first key yields the page's initial state (s_1, 1, v_1) without forming -inf - (-inf).
  * section 4: two summaries of disjoint key sets merge the same way: take the larger
    maximum, bring both normalisers and numerators to it, add.
The output is o = u / l.  These routines are the algorithm written out step by step in
plain Python/NumPy; the materialised definition lives in attention.py.
"""

from __future__ import annotations

import math

import numpy as np


def online_softmax_scalar(scores, values, *, rescale_numerator: bool = True):
    """Sequential (m, l, u) recurrence over one row.

    scores: sequence of N >= 1 finite floats; values: N vectors.
    rescale_numerator=False reproduces the flawed variant that rescales only l
    (el-ai.com section 3 shows it gives a wrong first component).
    Returns (o, steps) where steps[t] = (m, l, o_t) after t + 1 keys.
    """
    scores = [float(s) for s in scores]
    values = [np.asarray(x, dtype=np.float64) for x in values]
    if not scores:
        raise ValueError("a row needs at least one admitted key")
    if any(not math.isfinite(s) for s in scores):
        raise ValueError("scores must be finite")
    m, l, u = -math.inf, 0.0, np.zeros_like(values[0])   # no key seen yet
    steps = []
    for s, x in zip(scores, values):
        m_next = max(m, s)
        carry = 0.0 if m == -math.inf else math.exp(m - m_next)  # earlier terms, rebased
        w = math.exp(s - m_next)                                  # the new key's weight
        l = carry * l + w
        u = (carry * u if rescale_numerator else u) + w * x
        m = m_next
        steps.append((m, l, u / l))
    return u / l, steps


def summarize(scores, values):
    """(m, l, u) of one block, computed directly: m = max s, l = sum e^(s-m), u = sum e^(s-m) v."""
    s = np.asarray(scores, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64)
    m = float(s.max())
    w = np.exp(s - m)
    return m, float(w.sum()), w @ V


def merge(a, b):
    """Summary of the union of two disjoint key sets (el-ai.com section 4)."""
    m_a, l_a, u_a = a
    m_b, l_b, u_b = b
    m = max(m_a, m_b)
    f_a = math.exp(m_a - m)
    f_b = math.exp(m_b - m)
    return m, l_a * f_a + l_b * f_b, u_a * f_a + u_b * f_b


def blocked_softmax(scores, values, block: int):
    """o for one row computed block by block: summarize each block, fold with merge."""
    s = np.asarray(scores, dtype=np.float64)
    V = np.asarray(values, dtype=np.float64)
    state = None
    for start in range(0, len(s), block):
        part = summarize(s[start:start + block], V[start:start + block])
        state = part if state is None else merge(state, part)
    m, l, u = state
    return u / l


def merge_outputs(outs, lses):
    """Attention over the union of disjoint key sets from each set's output and LSE.

    outs: [S, rows, d] outputs, each normalised over its own keys; lses: [S, rows] natural
    log-sum-exp of each set's scaled scores (-inf where a set admits no key of the row).
    A part (o_s, L_s) is the summary (m, l, u) = (L_s, 1, o_s) of el-ai.com section 2 (the
    reference may be any constant), and the parts fold with the section-4 merge above.
    Returns (o [rows, d], lse [rows]); rows no part admits give o = 0, lse = -inf.
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    S, rows, d = outs.shape
    o = np.zeros((rows, d))
    lse = np.full(rows, -np.inf)
    for r in range(rows):
        state = None
        for s in range(S):
            if not np.isfinite(lses[s, r]):
                continue  # a set with no admitted key contributes nothing
            part = (float(lses[s, r]), 1.0, outs[s, r])
            state = part if state is None else merge(state, part)
        if state is not None:
            m, l, u = state
            o[r] = u / l
            lse[r] = m + math.log(l)
    return o, lse
