"""Pins of the oracle's FP8 (E4M3) path (CPU only): the format decoded from its bit fields,
nearest rounding by brute force, torch's float8_e4m3fn cast, block quantisation identities,
and closed forms of the tiled FP8 loop."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def grid_from_bits():
    """Every finite E4M3 value with its code: sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); exponent 15 with mantissa 7
    is NaN (no infinities)."""
    codes, vals = [], []
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        codes.append(c)
        vals.append(-v if s else v)
    return np.array(codes, dtype=np.uint8), np.array(vals)


def test_grid_is_fixed_by_rounding_and_encoding():
    codes, vals = grid_from_bits()
    assert vals.max() == 448.0 and len(vals) == 254
    np.testing.assert_array_equal(fp8.e4m3_round(vals), vals)
    np.testing.assert_array_equal(fp8.e4m3_encode(vals), codes)


def test_rounding_is_nearest_with_ties_to_even():
    codes, vals = grid_from_bits()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(0)
    xs = np.concatenate([mids, -mids, rng.uniform(-448, 448, 4000), rng.uniform(-0.05, 0.05, 4000)])
    got = fp8.e4m3_round(xs)
    for x, g in zip(xs, got):
        dist = np.abs(vals - x)
        best = vals[dist == dist.min()]
        if len(best) > 1:  # a tie: the value whose mantissa field is even
            best = [b for b in best if fp8.e4m3_encode(b) % 2 == 0]
        assert g == best[0] or (g == 0 and best[0] == 0), (x, g, best)


def test_rounding_matches_torch_float8_cast():
    rng = np.random.default_rng(1)
    xs = np.concatenate([rng.normal(size=5000) * 30, rng.normal(size=2000) * 0.01]).astype(np.float32)
    xs = np.clip(xs, -448, 448)
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(fp8.e4m3_round(xs), want)


def test_rounding_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_round([449.0])
    with pytest.raises(ValueError):
        fp8.e4m3_round([np.nan])


def test_block_quantisation_identities():
    rng = np.random.default_rng(2)
    x = rng.normal(size=(2, 3, 150, 16)).astype(np.float32) * np.array([1, 100, 0.01])[None, :, None, None]
    x[1, 2, 64:128] = 0.0                                   # an all-zero block
    vals, sc = fp8.quantize_blocks(x, seq_lens=[150, 100])
    assert sc.shape == (2, 3, 3) and sc.dtype == np.float32
    for b, L in ((0, 150), (1, 100)):
        for h in range(3):
            for t in range(3):
                r0, r1 = 64 * t, min(64 * t + 64, L)
                if r1 <= r0:
                    assert sc[b, h, t] == 0 and np.all(vals[b, h, r0:] == 0)
                    continue
                blk = x[b, h, r0:r1]
                amax = np.abs(blk).max()
                assert sc[b, h, t] == np.float32(amax) / np.float32(448)
                if amax == 0:
                    assert np.all(vals[b, h, r0:r1] == 0)
                    continue
                # the largest entry lands on +-448; dequantised values within half a spacing
                assert np.abs(vals[b, h, r0:r1]).max() == 448
                deq = vals[b, h, r0:r1] * sc[b, h, t]
                assert np.all(np.abs(deq - blk) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** -10 * sc[b, h, t])
        assert np.all(vals[b, :, L:] == 0)                  # padding rows


def quantized(q, k, v, lens=None):
    (q8, sq), (k8, sk), (v8, sv) = (fp8.quantize_blocks(t, seq_lens=lens) for t in (q, k, v))
    return q8, k8, v8, sq, sk, sv


def test_zero_queries_give_prefix_means_of_dequantised_values():
    rng = np.random.default_rng(3)
    q = np.zeros((1, 2, 200, 8), np.float32)
    k = rng.normal(size=(1, 2, 200, 8)).astype(np.float32)
    v = rng.normal(size=(1, 2, 200, 8)).astype(np.float32)
    q8, k8, v8, sq, sk, sv = quantized(q, k, v)
    O, LSE = fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=0.3, causal=True)
    deq = v8 * np.repeat(sv.astype(np.float64), 64, axis=2)[:, :, :200, None]
    want = np.cumsum(deq, axis=2) / np.arange(1, 201)[None, None, :, None]
    np.testing.assert_allclose(O, want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(LSE, np.broadcast_to(np.log(np.arange(1, 201)), (1, 2, 200)), atol=1e-12)
    # row 0 admits one key: its dequantised value exactly
    np.testing.assert_array_equal(O[:, :, 0], deq[:, :, 0])


def test_two_key_example_rounds_the_weight_and_the_normaliser():
    """q = (1, 0); keys (0, 0) and (x, 0) with scale * x = ln 0.3, so the weights are
    (1, 0.3).  0.3 is not on the E4M3 grid: its neighbours are 0.296875 and 0.3125 (spacing
    2^-5 in [0.25, 0.5)), and 0.3 rounds to 0.3125.  With v = (1, 0), (0, 1) the output is
    (1, 0.3125) / 1.3125; an unrounded weight would give (1, 0.3) / 1.3, and rounding the
    weight but not the normaliser (1, 0.3125) / 1.3."""
    scale = 0.5
    x = math.log(0.3) / scale
    q = np.array([[[[1.0, 0.0], [1.0, 0.0]]]], np.float32)
    k = np.array([[[[0.0, 0.0], [x, 0.0]]]], np.float32)
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    q8, k8, v8, sq, sk, sv = quantized(q, k, v)
    O, LSE = fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=scale)
    s_v = float(sv[0, 0, 0]) * 448                               # the dequantised 1.0
    want = np.array([1.0, 0.3125]) / 1.3125 * s_v
    np.testing.assert_allclose(O[0, 0, 0], want, rtol=1e-6)
    np.testing.assert_allclose(O[0, 0, 1], want, rtol=1e-6)
    assert abs(LSE[0, 0, 0] - math.log(1.3125)) < 1e-6


def test_running_maximum_moves_once_per_tile():
    """Two admitted keys in different tiles (the other keys of tile 0 score so low that
    their weights round to 0 in E4M3).
    (a) Scores 0 then ln 0.3: the second tile's weight is taken against the first tile's
        maximum, 0.3 -> 0.3125 on the E4M3 grid, output (v_a + 0.3125 v_b) / 1.3125.
    (b) Scores c0 < 0 then 0: the first tile's weight was 1 against its own maximum and is
        later multiplied by exp(c0) outside the rounding: output (e^c0 v_a + v_b) /
        (e^c0 + 1).  Key a shares its block with the -200 keys (block scale 200/448), so
        it is placed on that block's grid: k_a = -5.5 * 200/448, c0 = scale * k_a."""
    scale, n = 0.5, 65
    x = math.log(0.3) / scale
    ka = -5.5 * 200 / 448
    c0 = math.exp(scale * ka)
    q = np.zeros((1, 1, n, 2), np.float32)
    q[..., 0] = 1.0
    v = np.zeros((1, 1, n, 2), np.float32)
    v[0, 0, 0] = (1.0, 0.0)
    v[0, 0, 64] = (0.0, 1.0)
    for first, second, want in ((0.0, x, np.array([1.0, 0.3125]) / 1.3125),
                                (ka, 0.0, np.array([c0, 1.0]) / (c0 + 1))):
        k = np.zeros((1, 1, n, 2), np.float32)
        k[0, 0, 1:64, 0] = -200.0                      # weights exp(-100) -> 0 in E4M3
        k[0, 0, 0, 0], k[0, 0, 64, 0] = first, second
        q8, k8, v8, sq, sk, sv = quantized(q, k, v)
        O, _ = fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=scale)
        s_v = float(sv[0, 0, 0]) * 448
        np.testing.assert_allclose(O[0, 0, 0], want * s_v, rtol=1e-6)


def test_key_order_inside_a_tile_does_not_matter():
    """The running maximum moves once per tile, so permuting keys (with their values)
    inside one tile of a non-causal row changes nothing but summation order."""
    rng = np.random.default_rng(4)
    q, k, v = (rng.normal(size=(1, 1, 128, 16)).astype(np.float32) for _ in range(3))
    perm = np.concatenate([rng.permutation(64), 64 + rng.permutation(64)])
    a = fp8.attention_fp8(*quantized(q, k, v), scale=0.25)
    q8, k8, v8, sq, sk, sv = quantized(q, k, v)
    b = fp8.attention_fp8(q8, k8[:, :, perm], v8[:, :, perm], sq, sk, sv, scale=0.25)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_error_against_exact_attention_is_within_e4m3_precision():
    """Each operand and weight is within a relative 2^-4 of its exact value, so the FP8
    output stays within a few 2^-4 of the exact one; gross mistakes (a dropped scale, a
    transposed block) are far outside."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.normal(size=(1, 2, 300, 64)).astype(np.float32) for _ in range(3))
    for causal in (False, True):
        O, _ = fp8.attention_fp8(*quantized(q, k, v), scale=0.125, causal=causal)
        Oe, _ = oracle.attention(q, k, v, scale=0.125, causal=causal)
        err = np.abs(O - Oe)
        assert err.mean() <= 2.0 ** -4 * np.abs(v).mean(), err.mean()
        assert err.max() <= 2.0 ** -1, err.max()


def test_grouped_heads_and_lengths():
    rng = np.random.default_rng(6)
    q = rng.normal(size=(2, 4, 100, 8)).astype(np.float32)
    k = rng.normal(size=(2, 2, 100, 8)).astype(np.float32)
    v = rng.normal(size=(2, 2, 100, 8)).astype(np.float32)
    lens = [100, 37]
    O, LSE = fp8.attention_fp8(*quantized(q, k, v, lens), scale=0.3, causal=True, seq_lens=lens)
    assert np.all(O[1, :, 37:] == 0) and np.all(LSE[1, :, 37:] == -np.inf)
    # head h reads K/V head h // 2: the same as running the group's heads one by one
    q8, k8, v8, sq, sk, sv = quantized(q, k, v, lens)
    for h in range(4):
        o1, _ = fp8.attention_fp8(q8[:, h:h + 1], k8[:, h // 2:h // 2 + 1], v8[:, h // 2:h // 2 + 1],
                                  sq[:, h:h + 1], sk[:, h // 2:h // 2 + 1], sv[:, h // 2:h // 2 + 1],
                                  scale=0.3, causal=True, seq_lens=lens)
        np.testing.assert_array_equal(o1[:, 0], O[:, h])


def test_near_tie_slack_covers_the_other_rounding():
    """A weight placed next to the E4M3 midpoint 0.328125 (between 0.3125, mantissa even, and
    0.34375): the loop rounds it to 0.3125; rounding it up instead gives
    (v0 + 0.34375 v1) / 1.34375.  The reported slack must cover that difference, and rows
    without a near-tie report none."""
    scale = 0.5
    x = math.log(0.328125) / scale
    q = np.array([[[[1.0, 0.0], [1.0, 0.0]]]], np.float32)
    k = np.array([[[[0.0, 0.0], [x, 0.0]]]], np.float32)
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]], np.float32)
    q8, k8, v8, sq, sk, sv = quantized(q, k, v)
    O, LSE, Os, Ls = fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=scale, tie_rel=2.0 ** -16)
    s_v = float(sv[0, 0, 0]) * 448
    np.testing.assert_allclose(O[0, 0, 0], np.array([1.0, 0.3125]) / 1.3125 * s_v, rtol=1e-6)
    alt = np.array([1.0, 0.34375]) / 1.34375 * s_v
    diff = np.abs(alt - O[0, 0, 0])
    assert np.all(diff <= Os[0, 0, 0]) and np.all(Os[0, 0, 0] <= 2 * diff + 1e-12), (diff, Os[0, 0, 0])
    assert abs(math.log(1.34375) - LSE[0, 0, 0]) <= Ls[0, 0, 0]
    # the same inputs with tie_rel 0: identical outputs; far from a tie: no slack
    O2, L2 = fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=scale)
    np.testing.assert_array_equal(O, O2)
    rng = np.random.default_rng(7)
    qq, kk, vv = (rng.normal(size=(1, 1, 64, 8)).astype(np.float32) for _ in range(3))
    _, _, Os3, Ls3 = fp8.attention_fp8(*quantized(qq, kk, vv), scale=0.3, tie_rel=1e-30)
    assert np.all(Os3 == 0) and np.all(Ls3 == 0)
