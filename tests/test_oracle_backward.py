"""Pins of the oracle's attention gradients (CPU only): the derivative's definition at 50
digits, and closed forms that follow from the invariances of the forward pass."""

import math

import mpmath
import numpy as np
import pytest

import oracle

mpmath.mp.dps = 50


def _mp_loss(q, k, v, dout, scale, causal, L):
    """sum(O * dout) by the forward definition at 50 digits (rows >= L are padding)."""
    n, d, dv = len(q), len(q[0]), len(v[0])
    total = mpmath.mpf(0)
    for i in range(min(n, L)):
        keys = [j for j in range(L) if (not causal or j <= i)]
        w = [mpmath.exp(scale * mpmath.fsum(q[i][c] * k[j][c] for c in range(d))) for j in keys]
        den = mpmath.fsum(w)
        for c in range(dv):
            o = mpmath.fsum(wj * v[j][c] for wj, j in zip(w, keys)) / den
            total += o * dout[i][c]
    return total


def _mp_grad(x, f, h=mpmath.mpf("1e-15")):
    g = np.zeros((len(x), len(x[0])))
    for i in range(len(x)):
        for c in range(len(x[0])):
            old = x[i][c]
            x[i][c] = old + h
            up = f()
            x[i][c] = old - h
            dn = f()
            x[i][c] = old
            g[i, c] = float((up - dn) / (2 * h))
    return g


@pytest.mark.parametrize("case", range(8))
def test_gradients_against_50_digit_finite_differences(case):
    rng = np.random.default_rng(300 + case)
    n = [1, 2, 3, 4, 5, 3, 4, 5][case]
    d = [1, 2, 3, 2, 3, 1, 3, 2][case]
    causal = bool(case % 2)
    L = n if case < 6 else n - 2
    spread = [1.0, 3.0, 8.0][case % 3]
    q, k, v, do = (rng.normal(size=(n, d)) * s for s in (spread, spread, 1.0, 1.0))
    scale = 1 / math.sqrt(d)
    dq, dk, dv = oracle.attention_grad(q[None, None], k[None, None], v[None, None], do[None, None],
                                       causal=causal, seq_lens=[L])
    mq = [[mpmath.mpf(float(x)) for x in row] for row in q]
    mk = [[mpmath.mpf(float(x)) for x in row] for row in k]
    mv = [[mpmath.mpf(float(x)) for x in row] for row in v]
    mdo = [[mpmath.mpf(float(x)) for x in row] for row in do]
    msc = mpmath.mpf(scale)

    def f():
        return _mp_loss(mq, mk, mv, mdo, msc, causal, L)

    for got, x in ((dq, mq), (dk, mk), (dv, mv)):
        want = _mp_grad(x, f)
        np.testing.assert_allclose(got[0, 0], want, rtol=1e-12, atol=1e-13)


def _mp_loss_heads(qs, k, v, dos, scale, window):
    """sum over query heads of the causal windowed loss, all heads sharing one K/V head."""
    total = mpmath.mpf(0)
    n, d = len(k), len(k[0])
    for q, do in zip(qs, dos):
        for i in range(n):
            keys = [j for j in range(n) if j <= i and (not window or j > i - window)]
            w = [mpmath.exp(scale * mpmath.fsum(q[i][c] * k[j][c] for c in range(d))) for j in keys]
            den = mpmath.fsum(w)
            for c in range(len(v[0])):
                total += mpmath.fsum(wj * v[j][c] for wj, j in zip(w, keys)) / den * do[i][c]
    return total


@pytest.mark.parametrize("case", range(3))
def test_grouped_window_gradients_against_50_digit_finite_differences(case):
    """Two query heads on one K/V head: dK and dV sum both heads' contributions."""
    rng = np.random.default_rng(400 + case)
    n, d, window = [(4, 2, 2), (5, 2, 3), (3, 3, 0)][case]
    q = rng.normal(size=(2, n, d)) * 2
    k = rng.normal(size=(n, d)) * 2
    v, do = rng.normal(size=(n, d)), rng.normal(size=(2, n, d))
    dq, dk, dv = oracle.attention_grad(q[None], k[None, None], v[None, None], do[None],
                                       causal=True, window=window)
    mp = lambda a: [[mpmath.mpf(float(x)) for x in row] for row in a]
    mq, mk, mv, mdo = [mp(q[0]), mp(q[1])], mp(k), mp(v), [mp(do[0]), mp(do[1])]
    msc = mpmath.mpf(1 / math.sqrt(d))

    def f():
        return _mp_loss_heads(mq, mk, mv, mdo, msc, window)

    for got, x in ((dq[0, 0], mq[0]), (dq[0, 1], mq[1]), (dk[0, 0], mk), (dv[0, 0], mv)):
        np.testing.assert_allclose(got, _mp_grad(x, f), rtol=1e-12, atol=1e-13)


def test_key_sum_and_value_sum_closed_forms():
    """K + 1 w^T leaves every output unchanged, so sum_j dK_j = 0; V + 1 c^T shifts every
    valid output by c, so sum_j dV_j = sum over valid rows of dO_i."""
    rng = np.random.default_rng(310)
    B, H, n, d = 2, 2, 24, 6
    q, k, v, do = (rng.normal(size=(B, H, n, d)) for _ in range(4))
    for causal in (False, True):
        lens = [n, 13]
        dq, dk, dv = oracle.attention_grad(q, k, v, do, causal=causal, seq_lens=lens)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        for b, L in enumerate(lens):
            np.testing.assert_allclose(dv[b].sum(axis=1), do[b, :, :L].sum(axis=1), atol=1e-12)
            assert np.all(dq[b, :, L:] == 0) and np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


def test_zero_queries_give_zero_key_gradient_and_single_key_rows():
    rng = np.random.default_rng(311)
    q = np.zeros((1, 1, 9, 4))
    k, v, do = (rng.normal(size=(1, 1, 9, 4)) for _ in range(3))
    dq, dk, dv = oracle.attention_grad(q, k, v, do, causal=True)
    assert np.all(dk == 0)
    # row 0 sees only key 0: its weight is identically 1, so it sends no gradient to q_0
    np.testing.assert_allclose(dq[0, 0, 0], 0.0, atol=1e-15)
    # a length-1 sequence: dV_0 = dO_0, no gradient to q or k
    dq1, dk1, dv1 = oracle.attention_grad(q + 1.0, k, v, do, seq_lens=[1])
    np.testing.assert_array_equal(dv1[0, 0, 0], do[0, 0, 0])
    assert np.all(dq1 == 0) and np.all(dk1 == 0)


# ------------------------------------------------------------------ term magnitudes
def _terms_loop(q, k, v, do, scale, causal):
    """|terms| of each gradient element by explicit loops over (i, j, c) on one head."""
    n, d = q.shape
    S = np.array([[scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in range(n)] for i in range(n)])
    ok = np.array([[(not causal) or j <= i for j in range(n)] for i in range(n)])
    P = np.zeros((n, n))
    for i in range(n):
        w = [math.exp(S[i, j]) if ok[i, j] else 0.0 for j in range(n)]
        P[i] = np.array(w) / sum(w)
    O = P @ v
    aq, ak, av = np.zeros((n, d)), np.zeros((n, d)), np.zeros((n, d))
    for i in range(n):
        dplus = sum(abs(do[i, c] * O[i, c]) for c in range(d))
        for j in range(n):
            dp = sum(do[i, c] * v[j, c] for c in range(d))
            t = P[i, j] * (abs(dp) + dplus)
            for c in range(d):
                av[j, c] += P[i, j] * abs(do[i, c])
                aq[i, c] += scale * t * abs(k[j, c])
                ak[j, c] += scale * t * abs(q[i, c])
    return aq, ak, av


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_magnitudes_against_explicit_term_loops(causal):
    rng = np.random.default_rng(17 + causal)
    q, k, v, do = (rng.normal(size=(5, 3)) for _ in range(4))
    got = oracle.attention_grad_magnitudes(q[None, None], k[None, None], v[None, None],
                                           do[None, None], causal=causal)
    want = _terms_loop(q, k, v, do, 1 / math.sqrt(3), causal)
    for g, w in zip(got, want):
        np.testing.assert_allclose(g[0, 0], w, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("causal,lens,window,hkv", [(False, None, 0, 2), (True, [9, 4], 0, 1),
                                                    (True, None, 3, 2)])
def test_gradient_magnitudes_bound_the_gradients(causal, lens, window, hkv):
    rng = np.random.default_rng(5)
    q, do = (rng.normal(size=(2, 2, 9, 4)) * s for s in (3.0, 1.0))
    k, v = (rng.normal(size=(2, hkv, 9, 4)) * s for s in (3.0, 1.0))
    grads = oracle.attention_grad(q, k, v, do, causal=causal, seq_lens=lens, window=window)
    mags = oracle.attention_grad_magnitudes(q, k, v, do, causal=causal, seq_lens=lens, window=window)
    for g, a in zip(grads, mags):
        assert g.shape == a.shape
        assert np.all(np.abs(g) <= a * (1 + 1e-12) + 1e-15)


def test_gradient_magnitudes_equality_cases():
    rng = np.random.default_rng(6)
    q, k, v = (rng.normal(size=(1, 1, 6, 4)) for _ in range(3))
    do = np.abs(rng.normal(size=(1, 1, 6, 4)))           # dO >= 0: dV has no cancellation
    _, _, dv = oracle.attention_grad(q, k, v, do)
    _, _, av = oracle.attention_grad_magnitudes(q, k, v, do)
    np.testing.assert_allclose(av, dv, rtol=1e-13)
    # one admitted key per row (causal row 0): |dV|_0 gets |dO_0| from row 0 alone
    q1, k1, v1, do1 = (rng.normal(size=(1, 1, 1, 4)) for _ in range(4))
    aq, ak, av = oracle.attention_grad_magnitudes(q1, k1, v1, do1, causal=True)
    np.testing.assert_allclose(av[0, 0, 0], np.abs(do1[0, 0, 0]), rtol=1e-15)
    # P = 1, dP = <dO, V>, D+ = sum |dO * V|: |dQ| = scale (|<dO,V>| + D+) |K|
    dp = float(do1[0, 0, 0] @ v1[0, 0, 0])
    dplus = float(np.abs(do1[0, 0, 0] * v1[0, 0, 0]).sum())
    np.testing.assert_allclose(aq[0, 0, 0], 0.5 * (abs(dp) + dplus) * np.abs(k1[0, 0, 0]), rtol=1e-14)
    np.testing.assert_allclose(ak[0, 0, 0], 0.5 * (abs(dp) + dplus) * np.abs(q1[0, 0, 0]), rtol=1e-14)
