"""fp64 CPU oracle for exact scaled dot-product attention — TEST INFRASTRUCTURE.

This package is the slow, obviously correct reference that the GPU library is checked
against.  Only the test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import it; the product path (``online_softmax_attn_amd``) never
does, and the two share no code.  Everything here is plain NumPy in float64 (mpmath only
in the tests that pin it).

Sources (the pages' own text; formulas there are partly garbled by HTML extraction):
  * pierluigilucio.it "Sviluppo AI ed Algebra Lineare", section "Formulazione Algebrica
    della Self-Attention" — the definition S = QK^T/sqrt(d_k), row softmax, Y = AV.
  * maeste.it "attention matrix deep" page — the formula softmax(Q K^T / sqrt(d_head)) V,
    the causal mask (future keys set to -inf before the softmax), decode as a 1 x n row.
  * el-ai.com "Attenzione: softmax online, riscalamento e memoria" — section 1 (the
    object computed, max subtraction), section 2 (the (m, l, u) invariant), section 3
    (worked example), section 4 (merge of disjoint blocks), section 5 (fully masked rows
    need an explicit convention).

Functions and their pins (tests/test_oracle.py):
  attention / attend / attention_rows / decode
      pinned by 50-digit mpmath brute force on tiny inputs (also with grouped K/V heads and
      causal windows), the worked example, row sums, convex hull, shift invariance, closed
      forms (Q = 0 prefix means, single key, dominant key, a window of one returns the
      token's own value, a window as long as the sequence is plain causal).
  online_softmax_scalar / merge / summarize / blocked_softmax
      pinned by the worked example's step table (and its wrong variant), the block-merge
      experiment design of el-ai.com section 4, and merge associativity/commutativity.
  attention_chunk
      pinned by the rows q_start .. of attention over the whole sequence (a square-mask
      computation) for causal, windowed and unmasked chunks, grouped heads, and the whole
      sequence as one chunk; by a 50-digit brute force of a tiny offset chunk.
  merge_outputs
      pinned by attention over the union of disjoint key sets (plain and causal, key sets
      of uneven size and scores up to ~+-1000), the causal decomposition of a sequence into
      query/key chunks, part-order invariance, empty parts, and the closed form for two
      parts of equal LSE (mean of the outputs, LSE + ln 2).
  attention_grad_magnitudes (backward.py)
      pinned by the triangle inequality against the gradients (every magnitude at least
      the gradient element), its equality cases (dO >= 0 gives |dV| = dV; a single admitted
      key gives |dV| = |dO| and |dQ|, |dK| as written out for P = 1), and by sums of
      absolute values over an explicit loop of the terms on tiny inputs.
  attention_grad (backward.py)
      pinned by 50-digit central differences of the forward definition (masks, padding)
      (also two query heads sharing one K/V head under a causal window) and by closed forms
      (sum of dK is zero; sum of dV is the sum of dO; Q = 0 gives dK = 0; single-key rows
      send no gradient to q or k).
  fp8.e4m3_round / e4m3_encode / quantize_blocks / attention_fp8 (fp8.py)
      pinned in tests/test_oracle_fp8.py by the E4M3 grid decoded from its bit fields,
      brute-force nearest rounding with ties to even, torch's float8_e4m3fn cast, block
      quantisation identities, the Q = 0 closed form, hand-computed two-key examples of the
      weight rounding and of the once-per-tile running maximum, key-order invariance inside
      a tile, and the E4M3 error bound against exact attention.
No function here is "parity unpinned".
"""

from . import fp8
from .attention import attend, attention, attention_chunk, attention_rows, decode, to_f64
from .backward import attention_grad, attention_grad_magnitudes
from .online import blocked_softmax, merge, merge_outputs, online_softmax_scalar, summarize

__all__ = [
    "fp8",
    "attend",
    "attention",
    "attention_chunk",
    "attention_rows",
    "decode",
    "to_f64",
    "attention_grad",
    "attention_grad_magnitudes",
    "online_softmax_scalar",
    "merge",
    "merge_outputs",
    "summarize",
    "blocked_softmax",
]
