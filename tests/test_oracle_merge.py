"""Pins of oracle.merge_outputs (the merge of attention results over disjoint key sets).

el-ai.com "Attenzione: softmax online, riscalamento e memoria", section 4: the summaries of
two disjoint key sets combine into the summary of their union.  Here a part is an output
normalised over its own keys plus that set's log-sum-exp; the pins check the merged result
against attention computed directly over the union (oracle.attend on the full score
matrix), which is a different computation, and against closed forms.
"""

import math

import numpy as np
import pytest

import oracle


def _parts(S, V, sets, valid=None):
    """Output and LSE of each key set, computed directly on its columns."""
    outs, lses = [], []
    for cols in sets:
        vs = None if valid is None else valid[:, cols]
        o, l = oracle.attend(S[:, cols], V[cols], vs)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("scale", [1.0, 40.0])
def test_merge_of_disjoint_key_sets_is_attention_over_the_union(scale):
    rng = np.random.default_rng(11)
    nq, nk, d = 6, 29, 5
    S = scale * rng.standard_normal((nq, nk)) * 25.0  # scores up to ~+-1000 at scale 40
    V = rng.standard_normal((nk, d))
    perm = rng.permutation(nk)
    sets = [perm[:3], perm[3:4], perm[4:17], perm[17:]]  # uneven, non-contiguous sets
    outs, lses = _parts(S, V, sets)
    o, lse = oracle.merge_outputs(outs, lses)
    ro, rl = oracle.attend(S, V)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=0)


def test_causal_sequence_from_query_and_key_chunks():
    # a causal sequence cut into C chunks: query chunk i against key chunks j < i (all pairs
    # admitted) and the diagonal chunk (causal inside), merged, is causal attention
    rng = np.random.default_rng(12)
    n, C, d = 24, 4, 8
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    S = q @ k.T / math.sqrt(d)
    valid = np.tril(np.ones((n, n), dtype=bool))
    ro, rl = oracle.attend(S, v, valid)
    c = n // C
    for i in range(C):
        rows = slice(i * c, (i + 1) * c)
        outs, lses = [], []
        for j in range(i + 1):
            cols = slice(j * c, (j + 1) * c)
            vb = np.tril(np.ones((c, c), dtype=bool)) if j == i else None
            o, l = oracle.attend(S[rows, cols], v[cols], vb)
            outs.append(o)
            lses.append(l)
        o, l = oracle.merge_outputs(np.stack(outs), np.stack(lses))
        np.testing.assert_allclose(o, ro[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l, rl[rows], rtol=1e-14, atol=0)


def test_part_order_does_not_matter():
    rng = np.random.default_rng(13)
    outs = rng.standard_normal((5, 7, 3))
    lses = rng.standard_normal((5, 7)) * 30.0
    o1, l1 = oracle.merge_outputs(outs, lses)
    p = [3, 0, 4, 1, 2]
    o2, l2 = oracle.merge_outputs(outs[p], lses[p])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-15, atol=0)


def test_empty_parts_are_ignored_and_all_empty_rows_give_zero():
    rng = np.random.default_rng(14)
    outs = rng.standard_normal((3, 4, 2))
    lses = rng.standard_normal((3, 4))
    lses[1, :] = -np.inf            # part 1 admits no key of any row
    outs[1, :] = np.nan             # and whatever it holds is never read
    lses[:, 3] = -np.inf            # row 3 has no admitted key at all
    o, l = oracle.merge_outputs(outs, lses)
    o_ref, l_ref = oracle.merge_outputs(outs[[0, 2]], lses[[0, 2]])
    np.testing.assert_array_equal(o[:3], o_ref[:3])
    np.testing.assert_array_equal(l[:3], l_ref[:3])
    assert np.all(o[3] == 0.0) and l[3] == -np.inf


def test_two_parts_of_equal_lse_average_their_outputs():
    a = np.array([[1.0, -2.0, 0.5]])
    b = np.array([[3.0, 4.0, -0.5]])
    o, l = oracle.merge_outputs(np.stack([a, b]), np.array([[7.25], [7.25]]))
    np.testing.assert_allclose(o, (a + b) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(l, [7.25 + math.log(2.0)], rtol=1e-15, atol=0)
