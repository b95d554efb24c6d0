"""FP8 (E4M3) block-scaled attention, step by step — TEST INFRASTRUCTURE.

Source: pierluigilucio.it "Sviluppo AI ed Algebra Lineare", the part on FP8 quantisation and
mixed-precision accumulation in FlashAttention-3:
  * format: E4M3 = 1 sign bit, 4 exponent bits, 3 mantissa bits, largest magnitude 448
    (section "I Due Formati FP8").  The exponent bias (7), the subnormals (m * 2^-9) and the
    absence of infinities are the OCP "E4M3FN" definition the page names; rounding is to
    nearest, ties to even.
  * block quantisation (section "Quantizzazione a Blocchi e Scaling Algebrico"): for a block
    X of rows, s_X = max|X| / 448 and X_fp8 = clip(round(X / s_X), -448, 448); the scales
    leave the products algebraically, S = (scale * s_Q * s_K) * (Q_fp8 K_fp8^T), the factor
    applied once, in fp32, to the fp32 accumulator.
  * the online-softmax loop (section "Integrazione nel ciclo Online Softmax"): scores in
    fp32, the maximum, S - m and exp(S - m) in fp32; the weights P~ are rounded to E4M3
    before the second product P~_fp8 V_fp8, accumulated in fp32; the division by l happens
    once at the end, then the cast to bf16.

Readings (where the page is silent): blocks are 64 rows of one (batch, head) for Q, K and V
(the key block is the tile of the online loop); a block whose entries are all 0 has s = 0
and codes 0; rows past a sequence's length are padding (treated as 0, never admitted); the
normaliser l sums the same E4M3-rounded weights that enter P~ V (as the bf16 path sums its
bf16-rounded weights); the running maximum is updated once per key tile, exactly (no
headroom), so P~ of tile t is taken against the maximum over tiles 0..t.  Since the E4M3
rounding of P~ depends on that maximum, this function follows the tiled loop in the page's
order rather than a closed form.

Pinned in tests/test_oracle_fp8.py: the E4M3 grid decoded from its bit fields, brute-force
nearest rounding with ties to even, torch's float8_e4m3fn cast; block quantisation
identities; the Q = 0 closed form (prefix means of the dequantised V), single-key rows, a
hand-computed two-key example of the weight rounding, invariance to key order inside a
tile, and the E4M3 error bound against exact attention.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import _group, to_f64

E4M3_MAX = 448.0
BLOCK = 64  # rows per quantisation block; also the key tile of the online loop


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value (ties to even) of finite x with |x| <= 448, as float64.

    Normal numbers 2^E * (1 + f/8), E in [-6, 8]: spacing 2^(E-3).  Subnormals f/8 * 2^-6:
    spacing 2^-9.  So the spacing at x is 2^(max(E, -6) - 3) with E = floor(log2|x|).
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_round takes finite values within +-448")
    _, e = np.frexp(x)                       # x = mant * 2^e, mant in [0.5, 1)
    E = np.maximum(e - 1, -6)
    q = np.ldexp(1.0, E - 3)
    return np.rint(x / q) * q                # np.rint rounds half to even


def e4m3_encode(v) -> np.ndarray:
    """uint8 codes of E4M3 values (as produced by e4m3_round): sign | exponent | mantissa."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.uint8) << 7
    a = np.abs(v)
    _, e = np.frexp(a)
    E = e - 1
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, E + 7, 0)
    mant = np.where(normal, a / np.ldexp(1.0, E) - 1.0, a / 2.0 ** -6) * 8
    if np.any(mant != np.rint(mant)):
        raise ValueError("value not on the E4M3 grid")
    code = sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)
    return np.where(a == 0, sign, code).astype(np.uint8)


def quantize_blocks(x, *, seq_lens=None, block: int = BLOCK):
    """Per-block E4M3 quantisation of [B, H, n, d] (any float dtype).

    Returns (values, scales): values float64 [B, H, n, d] on the E4M3 grid, scales float32
    [B, H, ceil(n / block)].  s = max|X| / 448 and X / s are fp32 operations; rows at or past
    a sequence's length count as 0.
    """
    x32 = np.asarray(to_f64(x), dtype=np.float32)
    B, H, n, d = x32.shape
    nb = -(-n // block)
    vals = np.zeros(x32.shape, dtype=np.float64)
    scales = np.zeros((B, H, nb), dtype=np.float32)
    lens = [n] * B if seq_lens is None else [int(v) for v in seq_lens]
    for b in range(B):
        for h in range(H):
            for t in range(nb):
                r0, r1 = t * block, min((t + 1) * block, lens[b])
                if r1 <= r0:
                    continue
                X = x32[b, h, r0:r1]
                s = np.float32(np.abs(X).max()) / np.float32(E4M3_MAX)
                scales[b, h, t] = s
                if s == 0:
                    continue
                y = np.clip(X / s, -E4M3_MAX, E4M3_MAX)          # fp32 division, then clip
                vals[b, h, r0:r1] = e4m3_round(y)
    return vals, scales


def _near_ties(P, window):
    """E4M3 spacing at each weight that lies within window * p of a rounding midpoint (either
    rounding is then a correct outcome of an evaluation that precise), else 0."""
    P = np.asarray(P, dtype=np.float64)
    _, e = np.frexp(P)
    q = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    mid = (np.floor(P / q) + 0.5) * q
    return np.where((P > 0) & (np.abs(P - mid) <= window * P), q, 0.0)


def attention_fp8(q8, k8, v8, q_scale, k_scale, v_scale, *, scale: float, causal: bool = False,
                  seq_lens=None, block: int = BLOCK, tie_rel: float = 0.0, acc_rel: float = 0.0):
    """The FP8 online-softmax loop over key tiles of `block` keys (rows in parallel).

    q8 [B, H, n, d], k8 / v8 [B, H_kv, n, d]: E4M3 values (float64); *_scale: fp32 block
    scales [B, heads, ceil(n / block)].  Returns (O float64 [B, H, n, d] before the output
    cast, LSE float64 [B, H, n]); rows with no admitted key give 0 / -inf.

    The weights are rounded to E4M3 from fp32 values, and another correct evaluation (a
    different summation order, exponential or scale folding, or a product unit that sums
    its terms with less than fp32 precision) can land on the other side of a rounding
    midpoint.  With tie_rel > 0 the function also returns (O_slack, LSE_slack): for every
    weight within `window` * p of a midpoint, the largest change of the row's output and LSE
    that rounding it the other way makes (first order, summed over such weights); rows
    without near-ties have zero slack.  window = tie_rel + 2 * acc_rel * alpha * 2 * 448^2:
    acc_rel bounds the error of one 64-term block of the score sum relative to its largest
    term (at most 448^2 in code units; two blocks per 128-dim score, alpha = scale s_Q s_K
    converts to score units, and a weight exp(S - m) moves by the error of S and of m).
    """
    q8, k8, v8 = (np.asarray(a, dtype=np.float64) for a in (q8, k8, v8))
    B, H, n, d = q8.shape
    G = _group(H, k8.shape[1])
    lens = [n] * B if seq_lens is None else [int(v) for v in seq_lens]
    O = np.zeros((B, H, n, d))
    LSE = np.full((B, H, n), -math.inf)
    O_slack = np.zeros((B, H, n, d))
    LSE_slack = np.zeros((B, H, n))
    f32 = np.float32
    for b in range(B):
        L = lens[b]
        if L <= 0:
            continue
        rows = np.arange(L)
        for h in range(H):
            hk = h // G
            s_q = q_scale[b, h, rows // block].astype(f32)
            m = np.full(L, -np.inf, dtype=f32)   # running maximum per row (fp32, natural units)
            l = np.zeros(L)
            u = np.zeros((L, d))
            ties = []                           # (tile, spacing per weight, tile maximum)
            for t in range(-(-L // block)):
                j0, j1 = t * block, min((t + 1) * block, L)
                keys = np.arange(j0, j1)
                ok = (keys[None, :] <= rows[:, None]) if causal else np.ones((L, j1 - j0), bool)
                live = ok.any(axis=1)           # rows that admit a key of this tile
                alpha = ((f32(scale) * s_q) * f32(k_scale[b, hk, t])).astype(f32)
                raw = q8[b, h, :L] @ k8[b, hk, j0:j1].T                 # exact in fp64
                S = (alpha[:, None] * raw.astype(f32)).astype(f32)     # fp32 scores
                S = np.where(ok, S, -np.inf).astype(f32)
                m_new = np.where(live, np.maximum(m, S.max(axis=1)), m).astype(f32)
                P = np.where(ok, np.exp((S - np.where(live, m_new, 0)[:, None]).astype(f32)), 0)
                P8 = e4m3_round(P.astype(f32))
                c = np.where(m == -np.inf, 0.0, np.exp(m.astype(np.float64) - m_new.astype(np.float64)))
                c = np.where(live, c, 1.0)
                l = l * c + P8.sum(axis=1)
                u = u * c[:, None] + float(v_scale[b, hk, t]) * (P8 @ v8[b, hk, j0:j1])
                m = m_new
                if tie_rel > 0:
                    window = tie_rel + 2 * acc_rel * alpha.astype(np.float64) * 2 * E4M3_MAX ** 2
                    ties.append((t, _near_ties(P.astype(f32), window[:, None]), m_new.astype(np.float64)))
            o = u / l[:, None]
            O[b, h, :L] = o
            LSE[b, h, :L] = m.astype(np.float64) + np.log(l)
            if tie_rel > 0:
                mf = m.astype(np.float64)
                dw_tot = np.zeros(L)
                for t, sp, mt in ties:
                    ri, kj = np.nonzero(sp)                       # the near-tie weights
                    if len(ri) == 0:
                        continue
                    w = sp[ri, kj] * np.exp(mt[ri] - mf[ri])      # spacing at the row's end
                    dv = float(v_scale[b, hk, t]) * v8[b, hk, t * block + kj]
                    np.add.at(O_slack[b, h], ri, w[:, None] * np.abs(dv - o[ri]))
                    np.add.at(dw_tot, ri, w)
                denom = np.maximum(l - dw_tot, 1e-300)
                O_slack[b, h, :L] /= denom[:, None]
                LSE_slack[b, h, :L] = dw_tot / denom
    if tie_rel > 0:
        return O, LSE, O_slack, LSE_slack
    return O, LSE
