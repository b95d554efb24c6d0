"""The FP8 parity check (tests/fp8_check.py), on the CPU: it passes the oracle's own output
and rejects typical mistakes of an FP8 attention kernel, each planted in an evaluation of
the FP8 loop (pierluigilucio.it "Sviluppo AI ed Algebra Lineare", FP8 part,
"Quantizzazione a Blocchi e Scaling Algebrico" and "Integrazione nel ciclo Online
Softmax") and run through the exact check the GPU test applies, with its committed
TIE_REL / ACC_REL window and slack-use bounds.

The mutated evaluations below restate the loop's steps with one mistake each; they are
test aids, not references: the reference is oracle.fp8.attention_fp8."""

import math

import numpy as np
import pytest

import workloads
from fp8_check import ACC_REL, TIE_REL, as_bf16, check, slack_use
from oracle import fp8

SCALE = float(np.float32(1 / math.sqrt(128)))


def quantized(q, k, v, lens=None):
    return [fp8.quantize_blocks(t, seq_lens=lens) for t in (q, k, v)]


def reference(ops, causal, lens=None):
    (q8, sq), (k8, sk), (v8, sv) = ops
    return fp8.attention_fp8(q8, k8, v8, sq, sk, sv, scale=SCALE, causal=causal, seq_lens=lens,
                             tie_rel=TIE_REL, acc_rel=ACC_REL)


def truncate_e4m3(x):
    """E4M3 grid value of x rounded toward zero (a planted rounding mistake)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.trunc(x / q) * q


def mutated_loop(ops, causal, mistake, lens=None):
    """The tiled FP8 loop with one planted mistake; returns (o as the kernel would store it,
    i.e. bf16, and lse as fp32)."""
    (q8, sq), (k8, sk), (v8, sv) = ops
    B, H, n, d = q8.shape
    f32 = np.float32
    blk = fp8.BLOCK
    lens_ = [n] * B if lens is None else list(lens)
    O = np.zeros((B, H, n, d))
    LSE = np.full((B, H, n), -np.inf)
    for b in range(B):
        L = lens_[b]
        rows = np.arange(L)
        for h in range(H):
            s_q = sq[b, h, rows // blk].astype(f32)
            m = np.full(L, -np.inf, dtype=f32)
            l = np.zeros(L)
            u = np.zeros((L, d))
            for t in range(-(-L // blk)):
                j0, j1 = t * blk, min((t + 1) * blk, L)
                keys = np.arange(j0, j1)
                shift = 1 if mistake == "causal_off_by_one" else 0
                ok = (keys[None, :] <= rows[:, None] + shift) if causal else np.ones((L, j1 - j0), bool)
                live = ok.any(axis=1)
                alpha = ((f32(SCALE) * s_q) * f32(sk[b, h, t])).astype(f32)
                S = (alpha[:, None] * (q8[b, h, :L] @ k8[b, h, j0:j1].T).astype(f32)).astype(f32)
                S = np.where(ok, S, -np.inf).astype(f32)
                m_tile = np.where(live, S.max(axis=1), -np.inf).astype(f32)
                m_new = np.where(live, np.maximum(m, m_tile), m).astype(f32)
                ref_m = m_tile if mistake == "per_tile_max" else m_new
                P = np.where(ok, np.exp((S - np.where(live, ref_m, 0)[:, None]).astype(f32)), 0).astype(f32)
                if mistake == "p_unrounded":
                    P8 = P.astype(np.float64)
                elif mistake == "p_truncated":
                    P8 = truncate_e4m3(P)
                else:
                    P8 = fp8.e4m3_round(P)
                if mistake == "per_tile_max":  # bring the tile's weights to the running max after rounding
                    P8 = P8 * np.exp(np.where(live, ref_m.astype(np.float64) - m_new, 0.0))[:, None]
                c = np.where(m == -np.inf, 0.0, np.exp(m.astype(np.float64) - m_new.astype(np.float64)))
                c = np.where(live, c, 1.0)
                l = l * c + (P.astype(np.float64).sum(axis=1) if mistake == "l_unrounded" else P8.sum(axis=1))
                tv = min(t + 1, sv.shape[2] - 1) if mistake == "v_scale_next_block" else t
                s_v = 1.0 if mistake == "no_v_scale" else float(sv[b, h, tv])
                u = u * c[:, None] + s_v * (P8 @ v8[b, h, j0:j1])
                m = m_new
            O[b, h, :L] = u / l[:, None]
            LSE[b, h, :L] = (np.log(l) if mistake == "lse_without_max" else
                             m.astype(np.float64) + np.log(l))
    return as_bf16(O), LSE.astype(np.float32).astype(np.float64)


def causal_case():
    q, k, v = workloads.prefill(1, 2, 256, 128, seed=321)
    return q, k, v


def test_check_passes_the_oracle_output_as_a_kernel_stores_it():
    q, k, v = causal_case()
    ops = quantized(q, k, v)
    ref = reference(ops, causal=True)
    o, lse = mutated_loop(ops, causal=True, mistake=None)
    np.testing.assert_allclose(o, as_bf16(ref[0]), atol=2.0 ** -8)
    check(o, lse, ref)


@pytest.mark.parametrize("mistake", ["l_unrounded", "p_unrounded", "p_truncated", "no_v_scale",
                                     "per_tile_max", "v_scale_next_block", "causal_off_by_one",
                                     "lse_without_max"])
def test_check_rejects_a_planted_mistake_in_the_loop(mistake):
    q, k, v = causal_case()
    ops = quantized(q, k, v)
    ref = reference(ops, causal=True)
    o, lse = mutated_loop(ops, causal=True, mistake=mistake)
    with pytest.raises(AssertionError):
        check(o, lse, ref)
    # the element-wise bound itself, widened by the tie slack, is exceeded (the slack-use
    # bounds are not what catches it); the LSE mistake shows in the LSE alone
    if mistake != "lse_without_max":
        assert slack_use(o, ref)[0] > 0


@pytest.mark.parametrize("largest", [240.0, 256.0])
def test_check_rejects_a_quantiser_with_the_wrong_largest_magnitude(largest, monkeypatch):
    """Operands quantised with s = max|X| / 240 (or 256) instead of / 448, then the correct
    loop: the check against the correctly quantised reference must fail.  (A divisor off by a
    power of two, 224, is no mistake: the E4M3 grid is invariant under it outside the
    subnormals, so the dequantised operands are the same.)"""
    q, k, v = causal_case()
    ref = reference(quantized(q, k, v), causal=True)
    monkeypatch.setattr(fp8, "E4M3_MAX", largest)
    ops = quantized(q, k, v)
    monkeypatch.undo()
    o, lse = mutated_loop(ops, causal=True, mistake=None)
    with pytest.raises(AssertionError):
        check(o, lse, ref)


def test_check_rejects_a_quantiser_rounding_with_the_exponent_off_by_one(monkeypatch):
    """Quantisation onto a grid one binade finer (the exponent taken one too small): the
    codes are not the E4M3 codes, and the check must see it in the output."""
    q, k, v = causal_case()
    ref = reference(quantized(q, k, v), causal=True)

    def finer(x):
        x = np.asarray(x, dtype=np.float64)
        _, e = np.frexp(x)
        qq = np.ldexp(1.0, np.maximum(e - 2, -7) - 3)
        return np.rint(x / qq) * qq

    monkeypatch.setattr(fp8, "e4m3_round", finer)
    ops = quantized(q, k, v)
    monkeypatch.undo()
    o, lse = mutated_loop(ops, causal=True, mistake=None)
    with pytest.raises(AssertionError):
        check(o, lse, ref)
