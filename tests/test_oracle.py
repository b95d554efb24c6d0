"""Pins of the fp64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it checks.  Together they are chosen so that a plausible slip
in the oracle (a dropped rescale, a wrong sign, a transposed operand, a causal off-by-one,
a forgotten scale) fails at least one of them.
"""

import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _worked():
    with open(os.path.join(GOLDEN, "p5_worked_example.json")) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example (el-ai.com §3)
def test_worked_example_scalar_recurrence_matches_page_table():
    ex = _worked()
    tol = 0.5 * 10 ** -ex["printed_decimals"] + 1e-15
    o, steps = oracle.online_softmax_scalar(ex["scores"], ex["values"])
    assert len(steps) == len(ex["steps"])
    for got, want in zip(steps, ex["steps"]):
        m, l, ot = got
        assert m == want["m"]
        assert abs(l - want["l"]) <= tol
        np.testing.assert_allclose(ot, want["o"], rtol=0, atol=tol)
    np.testing.assert_allclose(o, ex["output"], rtol=0, atol=tol)


def test_worked_example_wrong_variant_is_detected():
    """Rescaling l but not u gives the page's wrong first component; the second one stays
    right, so a check of one component alone would miss the flaw (el-ai.com §3)."""
    ex = _worked()
    tol = 0.5 * 10 ** -ex["printed_decimals"] + 1e-15
    o_bad, _ = oracle.online_softmax_scalar(ex["scores"], ex["values"], rescale_numerator=False)
    assert abs(o_bad[0] - ex["wrong_first_component"]) <= tol
    assert abs(o_bad[1] - ex["output"][1]) <= tol
    o_good, _ = oracle.online_softmax_scalar(ex["scores"], ex["values"])
    assert abs(o_good[0] - o_bad[0]) > 0.4


def test_worked_example_materialised_attention():
    """Same row through the materialised definition: d=1, q=1, keys = the scores, scale 1."""
    ex = _worked()
    tol = 0.5 * 10 ** -ex["printed_decimals"] + 1e-15
    S = np.array([ex["scores"]])
    O, lse = oracle.attend(S, np.array(ex["values"]))
    np.testing.assert_allclose(O[0], ex["output"], rtol=0, atol=tol)
    # LSE closed form: 1001 + log(1 + e^-1 + e^-2)
    assert abs(lse[0] - (1001 + math.log(1 + math.exp(-1) + math.exp(-2)))) < 1e-12
    k = np.array(ex["scores"]).reshape(1, 1, 3, 1)
    v = np.array(ex["values"]).reshape(1, 1, 3, 2)
    # attention() needs the same n for q and k: use a 3-row query block, check the last row
    q3 = np.ones((1, 1, 3, 1))
    O3, _ = oracle.attention(q3, k, v, scale=1.0)
    np.testing.assert_allclose(O3[0, 0, 2], ex["output"], rtol=0, atol=tol)


# ---------------------------------------------------------------- mpmath brute force
mpmath.mp.dps = 50


def _mp_attention_row(q, K, V, scale, admitted):
    """Direct definition at 50 digits: no max subtraction, no blocking."""
    num = [mpmath.mpf(0)] * V.shape[1]
    den = mpmath.mpf(0)
    for j in admitted:
        s = mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(q, K[j]))
        w = mpmath.exp(s)
        den += w
        for c in range(V.shape[1]):
            num[c] += w * mpmath.mpf(float(V[j, c]))
    if den == 0:
        return [0.0] * V.shape[1], -math.inf
    return [float(x / den) for x in num], float(mpmath.log(den))


@pytest.mark.parametrize("case", range(12))
def test_attention_against_mpmath_brute_force(case):
    rng = np.random.default_rng(1000 + case)
    B, H = 2, 2
    n = int(rng.integers(1, 9))
    d = int(rng.integers(1, 5))
    causal = bool(case % 2)
    spread = [1.0, 10.0, 300.0][case % 3]
    q = rng.normal(size=(B, H, n, d)) * spread
    k = rng.normal(size=(B, H, n, d)) * spread
    v = rng.uniform(-3, 3, size=(B, H, n, d))
    lens = [int(rng.integers(1, n + 1)), n] if case % 4 >= 2 else None
    scale = 1.0 / math.sqrt(d)
    O, LSE = oracle.attention(q, k, v, causal=causal, seq_lens=lens)
    for b in range(B):
        L = n if lens is None else lens[b]
        for h in range(H):
            for i in range(n):
                if i >= L:
                    admitted = []
                else:
                    admitted = [j for j in range(L) if (not causal or j <= i)]
                want, want_lse = _mp_attention_row(q[b, h, i], k[b, h], v[b, h], scale, admitted)
                np.testing.assert_allclose(O[b, h, i], want, rtol=1e-13, atol=1e-14)
                if admitted:
                    assert abs(LSE[b, h, i] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))
                else:
                    assert LSE[b, h, i] == -math.inf


@pytest.mark.parametrize("case", range(6))
def test_attention_chunk_against_mpmath(case):
    """A chunk of queries at an offset into the key sequence: the causal mask and the window
    compare key positions with the chunk's query positions q_start + i."""
    rng = np.random.default_rng(2500 + case)
    H, Hkv, nk, d = 4, 2, 9, 3
    nq = int(rng.integers(1, nk + 1))
    q_start = int(rng.integers(0, nk - nq + 1))
    causal = case % 3 != 0
    window = 3 if case % 3 == 2 else 0
    q = rng.normal(size=(1, H, nq, d)) * 5
    k = rng.normal(size=(1, Hkv, nk, d)) * 5
    v = rng.normal(size=(1, Hkv, nk, d))
    O, LSE = oracle.attention_chunk(q, k, v, q_start, causal=causal, window=window)
    for h in range(H):
        for i in range(nq):
            p = q_start + i
            admitted = [j for j in range(nk) if (not causal or j <= p) and (not window or j > p - window)]
            want, want_lse = _mp_attention_row(q[0, h, i], k[0, h // 2], v[0, h // 2], 1 / math.sqrt(d), admitted)
            np.testing.assert_allclose(O[0, h, i], want, rtol=1e-13, atol=1e-14)
            assert abs(LSE[0, h, i] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))


@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 37)])
def test_attention_chunk_is_the_rows_of_whole_sequence_attention(causal, window):
    """Chunk i of a sequence equals rows q_start .. of attention over the whole sequence
    (the square-mask computation), for every chunk of an uneven cut; the whole sequence as
    one chunk is plain attention."""
    rng = np.random.default_rng(2600 + window + int(causal))
    B, H, Hkv, n, d = 2, 4, 2, 150, 8
    q = rng.normal(size=(B, H, n, d)) * 3
    k = rng.normal(size=(B, Hkv, n, d)) * 3
    v = rng.normal(size=(B, Hkv, n, d))
    ro, rl = oracle.attention(q, k, v, causal=causal, window=window)
    cuts = [0, 1, 40, 64, 129, 150]
    for a, c in zip(cuts[:-1], cuts[1:]):
        o, l = oracle.attention_chunk(q[:, :, a:c], k, v, a, causal=causal, window=window)
        np.testing.assert_allclose(o, ro[:, :, a:c], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, rl[:, :, a:c], rtol=1e-14, atol=1e-13)


@pytest.mark.parametrize("case", range(4))
def test_attention_rows_against_mpmath(case):
    rng = np.random.default_rng(2000 + case)
    H, n, d = 3, 9, 3
    q = rng.normal(size=(1, H, n, d))
    k = rng.normal(size=(1, H, n, d))
    v = rng.normal(size=(1, H, n, d))
    rows = np.stack([rng.permutation(n)[:4] for _ in range(H)])
    causal = bool(case % 2)
    O, LSE = oracle.attention_rows(q, k, v, rows, causal=causal)
    for h in range(H):
        for r_i, i in enumerate(rows[h]):
            admitted = [j for j in range(n) if (not causal or j <= i)]
            want, want_lse = _mp_attention_row(q[0, h, i], k[0, h], v[0, h], 1 / math.sqrt(d), admitted)
            np.testing.assert_allclose(O[0, h, r_i], want, rtol=1e-13, atol=1e-14)
            assert abs(LSE[0, h, r_i] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))


def test_decode_against_mpmath():
    rng = np.random.default_rng(7)
    B, H, d = 3, 2, 4
    lens = [1, 5, 11]
    q = rng.normal(size=(B, H, d)) * 3
    ks = [rng.normal(size=(H, L, d)) * 3 for L in lens]
    vs = [rng.normal(size=(H, L, d)) for L in lens]
    O, LSE = oracle.decode(q, ks, vs)
    for b in range(B):
        for h in range(H):
            want, want_lse = _mp_attention_row(q[b, h], ks[b][h], vs[b][h], 1 / math.sqrt(d), range(lens[b]))
            np.testing.assert_allclose(O[b, h], want, rtol=1e-13, atol=1e-14)
            assert abs(LSE[b, h] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))


@pytest.mark.parametrize("case", range(8))
def test_grouped_heads_and_window_against_mpmath(case):
    """Query head h reads K/V head h // (H / H_kv); a window w admits keys i - w < j <= i."""
    rng = np.random.default_rng(2500 + case)
    H, Hkv = [(4, 1), (4, 2), (6, 3), (2, 2)][case % 4]
    n, d = int(rng.integers(3, 10)), int(rng.integers(1, 4))
    window = [1, 2, 3, 100][case % 4] if case < 6 else 0
    causal = window > 0 or case % 2 == 1
    q = rng.normal(size=(2, H, n, d)) * 2
    k = rng.normal(size=(2, Hkv, n, d)) * 2
    v = rng.normal(size=(2, Hkv, n, d))
    lens = [n, int(rng.integers(1, n + 1))]
    O, LSE = oracle.attention(q, k, v, causal=causal, seq_lens=lens, window=window)
    G = H // Hkv
    for b in range(2):
        for h in range(H):
            for i in range(lens[b]):
                admitted = [j for j in range(lens[b])
                            if (not causal or j <= i) and (not window or j > i - window)]
                want, want_lse = _mp_attention_row(q[b, h, i], k[b, h // G], v[b, h // G],
                                                   1 / math.sqrt(d), admitted)
                np.testing.assert_allclose(O[b, h, i], want, rtol=1e-13, atol=1e-14)
                assert abs(LSE[b, h, i] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))
            rows = rng.permutation(n)[:3]
            Or, Lr = oracle.attention_rows(q, k, v, np.broadcast_to(rows, (2, H, 3)), causal=causal,
                                           seq_lens=lens, window=window)
            np.testing.assert_array_equal(Or[b, h], np.where((rows < lens[b])[:, None], O[b, h, rows], 0))


def test_window_of_one_returns_own_value_and_wide_window_is_causal():
    rng = np.random.default_rng(8)
    q, k, v = (rng.normal(size=(1, 2, 7, 3)) for _ in range(3))
    O, LSE = oracle.attention(q, k, v, causal=True, window=1)
    np.testing.assert_allclose(O, v, rtol=0, atol=1e-15)
    np.testing.assert_allclose(LSE, np.einsum("bhnd,bhnd->bhn", q, k) / math.sqrt(3), atol=1e-14)
    Ow, Lw = oracle.attention(q, k, v, causal=True, window=7)
    Oc, Lc = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(Ow, Oc)
    np.testing.assert_array_equal(Lw, Lc)


def test_grouped_heads_reject_a_non_divisor():
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 3, 2, 1)), np.zeros((1, 2, 2, 1)), np.zeros((1, 2, 2, 1)))


def test_decode_grouped_heads_and_window_against_mpmath():
    rng = np.random.default_rng(9)
    B, H, Hkv, d = 3, 4, 2, 3
    lens = [1, 6, 13]
    q = rng.normal(size=(B, H, d)) * 3
    ks = [rng.normal(size=(Hkv, L, d)) * 3 for L in lens]
    vs = [rng.normal(size=(Hkv, L, d)) for L in lens]
    for window in (0, 1, 4):
        O, LSE = oracle.decode(q, ks, vs, window=window)
        for b in range(B):
            for h in range(H):
                lo = lens[b] - window if window else 0
                want, want_lse = _mp_attention_row(q[b, h], ks[b][h // 2], vs[b][h // 2],
                                                   1 / math.sqrt(d), range(max(lo, 0), lens[b]))
                np.testing.assert_allclose(O[b, h], want, rtol=1e-13, atol=1e-14)
                assert abs(LSE[b, h] - want_lse) <= 1e-13 * max(1.0, abs(want_lse))


# ---------------------------------------------------------------- invariants
def test_rows_are_distributions_and_outputs_in_convex_hull():
    """Rows of A lie in (0,1) and sum to 1; each output is a convex combination of values
    (pierluigilucio.it, Formulazione Algebrica, step 3-4; el-ai.com §1)."""
    rng = np.random.default_rng(11)
    n, d = 40, 8
    S = rng.normal(size=(n, n)) * 20
    V = rng.uniform(-2, 2, size=(n, d))
    valid = np.tril(np.ones((n, n), dtype=bool))
    # weights as the oracle forms them: attend applied to identity values gives A itself
    A, _ = oracle.attend(S, np.eye(n), valid)
    assert np.all(A[valid] > 0) and np.all(A[valid] <= 1)
    assert np.all(A[~valid] == 0)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    O, _ = oracle.attend(S, V, valid)
    for i in range(n):
        lo = V[: i + 1].min(axis=0)
        hi = V[: i + 1].max(axis=0)
        assert np.all(O[i] >= lo - 1e-15) and np.all(O[i] <= hi + 1e-15)


def test_row_constant_shift_leaves_output_unchanged():
    """Adding the same constant to every score of a row changes nothing (el-ai.com §1)."""
    rng = np.random.default_rng(12)
    n, d = 30, 5
    S = rng.normal(size=(n, n)) * 50
    V = rng.normal(size=(n, d))
    c = rng.normal(size=(n, 1)) * 1e3
    O1, l1 = oracle.attend(S, V)
    O2, l2 = oracle.attend(S + c, V)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2 - l1, c[:, 0], rtol=1e-12)


def test_key_shift_and_value_shift_closed_forms():
    """K + 1 w^T shifts row i's scores by scale <q_i, w>: output unchanged.
    V + 1 c^T shifts every output by c (rows sum to one)."""
    rng = np.random.default_rng(13)
    q = rng.normal(size=(1, 2, 16, 4))
    k = rng.normal(size=(1, 2, 16, 4))
    v = rng.normal(size=(1, 2, 16, 4))
    w = rng.normal(size=4) * 5
    c = rng.normal(size=4) * 7
    for causal in (False, True):
        O, _ = oracle.attention(q, k, v, causal=causal)
        O_k, _ = oracle.attention(q, k + w, v, causal=causal)
        O_v, _ = oracle.attention(q, k, v + c, causal=causal)
        np.testing.assert_allclose(O_k, O, atol=1e-12)
        np.testing.assert_allclose(O_v, O + c, atol=1e-12)


def test_key_permutation_invariance_non_causal():
    rng = np.random.default_rng(14)
    q = rng.normal(size=(1, 1, 12, 3))
    k = rng.normal(size=(1, 1, 12, 3))
    v = rng.normal(size=(1, 1, 12, 3))
    p = rng.permutation(12)
    O, _ = oracle.attention(q, k, v)
    O_p, _ = oracle.attention(q, k[:, :, p], v[:, :, p])
    np.testing.assert_allclose(O_p, O, atol=1e-14)


def test_scale_default_is_inverse_sqrt_d():
    rng = np.random.default_rng(15)
    q = rng.normal(size=(1, 1, 6, 16))
    k = rng.normal(size=(1, 1, 6, 16))
    v = rng.normal(size=(1, 1, 6, 16))
    O, _ = oracle.attention(q, k, v)
    O4, _ = oracle.attention(q, k, v, scale=0.25)
    np.testing.assert_allclose(O, O4, atol=0)
    O1, _ = oracle.attention(q, k, v, scale=1.0)
    assert np.abs(O1 - O).max() > 1e-3


# ---------------------------------------------------------------- closed forms
def test_zero_queries_give_prefix_means():
    """Q = 0: all admitted scores are equal, so o_i is the mean of the admitted values —
    the prefix mean v_0..v_i under the causal mask."""
    rng = np.random.default_rng(16)
    n, d = 50, 6
    q = np.zeros((1, 1, n, d))
    k = rng.normal(size=(1, 1, n, d))
    v = rng.normal(size=(1, 1, n, d))
    O, LSE = oracle.attention(q, k, v, causal=True)
    want = np.cumsum(v[0, 0], axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(O[0, 0], want, atol=1e-14)
    np.testing.assert_allclose(LSE[0, 0], np.log(np.arange(1, n + 1)), atol=1e-14)
    O2, _ = oracle.attention(q, k, v, causal=False, seq_lens=[17])
    np.testing.assert_allclose(O2[0, 0, :17], np.broadcast_to(v[0, 0, :17].mean(axis=0), (17, d)), atol=1e-14)
    assert np.all(O2[0, 0, 17:] == 0)


def test_single_key_returns_its_value_and_padding_rows_are_zero():
    """n_b = 1: the only key gets weight 1 (el-ai.com §2 starts the state at u = v_1);
    padding queries have no admitted key: output 0, lse -inf (el-ai.com §5 convention)."""
    rng = np.random.default_rng(17)
    q = rng.normal(size=(2, 2, 5, 3)) * 40
    k = rng.normal(size=(2, 2, 5, 3)) * 40
    v = rng.normal(size=(2, 2, 5, 3))
    O, LSE = oracle.attention(q, k, v, seq_lens=[1, 5])
    np.testing.assert_array_equal(O[0, :, 0], v[0, :, 0])
    assert np.all(O[0, :, 1:] == 0)
    assert np.all(LSE[0, :, 1:] == -np.inf)
    assert np.all(np.isfinite(LSE[1]))


def test_dominant_key_takes_all_the_weight():
    n, d = 20, 4
    rng = np.random.default_rng(18)
    S = rng.normal(size=(n, n))
    j = rng.integers(0, n, size=n)
    S[np.arange(n), j] = S.max(axis=1) + 60.0
    V = rng.normal(size=(n, d))
    O, _ = oracle.attend(S, V)
    # the other weights are below e^-60 relative to the dominant one
    np.testing.assert_allclose(O, V[j], rtol=0, atol=1e-15)


def test_overflowing_scores_stay_finite():
    """Scores near 1000 overflow a naive exp (el-ai.com §3); the oracle must not."""
    S = np.array([[1000.0, 1001.0, 999.0, -1000.0]])
    V = np.array([[1.0], [2.0], [3.0], [4.0]])
    O, lse = oracle.attend(S, V)
    assert np.all(np.isfinite(O)) and np.isfinite(lse[0])


# ---------------------------------------------------------------- merge of blocks (el-ai.com §4)
@pytest.mark.parametrize("a", [1.0, 10.0, 1000.0])
def test_block_merge_experiment_design(a):
    """The page's experiment: 257 keys, 4-component values U[-2,2], scores U[-a,a], blocks
    of 1, 7, 32 and 257 against the materialised stable softmax; the page reports a max
    error of about 6.66e-16 in Python floats.  Own draws (the page's archive is not here)."""
    rng = np.random.default_rng(20260924)
    s = rng.uniform(-a, a, size=257)
    V = rng.uniform(-2, 2, size=(257, 4))
    ref, _ = oracle.attend(s[None, :], V)
    for block in (1, 7, 32, 257):
        o = oracle.blocked_softmax(s, V, block)
        assert np.abs(o - ref[0]).max() <= 4e-15


def test_merge_is_commutative_and_associative_up_to_rounding():
    rng = np.random.default_rng(21)
    s = rng.normal(size=30) * 30
    V = rng.normal(size=(30, 3))
    A = oracle.summarize(s[:7], V[:7])
    Bs = oracle.summarize(s[7:19], V[7:19])
    C = oracle.summarize(s[19:], V[19:])
    whole = oracle.summarize(s, V)
    ab, ba = oracle.merge(A, Bs), oracle.merge(Bs, A)
    assert ab[0] == ba[0]
    assert abs(ab[1] - ba[1]) <= 1e-15 * ab[1]
    np.testing.assert_allclose(ab[2], ba[2], rtol=1e-15, atol=0)
    x = oracle.merge(oracle.merge(A, Bs), C)
    y = oracle.merge(A, oracle.merge(Bs, C))
    z = oracle.merge(C, oracle.merge(Bs, A))
    for m, l, u in (x, y, z):
        assert m == whole[0]
        assert abs(l - whole[1]) <= 1e-14 * whole[1]
        np.testing.assert_allclose(u / l, whole[2] / whole[1], rtol=0, atol=1e-14)


def test_scalar_recurrence_rejects_empty_and_nonfinite():
    with pytest.raises(ValueError):
        oracle.online_softmax_scalar([], [])
    with pytest.raises(ValueError):
        oracle.online_softmax_scalar([1.0, float("inf")], [[0.0], [1.0]])


def test_scalar_recurrence_equals_materialised_on_random_rows():
    rng = np.random.default_rng(22)
    for a in (1.0, 100.0, 1000.0):
        s = rng.uniform(-a, a, size=64)
        V = rng.normal(size=(64, 3))
        o, _ = oracle.online_softmax_scalar(s, V)
        ref, _ = oracle.attend(s[None, :], V)
        np.testing.assert_allclose(o, ref[0], atol=1e-14)
