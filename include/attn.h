/*
 * attn.h — C ABI of the MI355X (gfx950) exact-attention library (libattn.so).
 *
 * What the library computes is exact scaled dot-product attention,
 *     O = softmax(Q K^T * scale) V,     scale normally 1/sqrt(d_head),
 * as defined on pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (section "Formulazione
 * Algebrica della Self-Attention") and on the maeste.it attention-matrix page (the formula
 * softmax(Q K^T / sqrt(d_head)) V and the causal mask).  It is evaluated tile by tile with
 * the running (m, l, u) summary of el-ai.com "Attenzione: softmax online, riscalamento e
 * memoria" (section 2: maximum, normaliser and unnormalised accumulator rescaled together),
 * so the n x n score matrix never exists in device memory; disjoint key ranges are joined
 * with the merge of its section 4.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller; the library never
 *     allocates, frees, synchronises, prints or aborts.  Work is enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) and the call returns once it is enqueued.
 *   - Tensors are dense and row-major with the last dimension fastest.  bf16 is the
 *     bfloat16 bit pattern (1-8-7), f32 is IEEE binary32.
 *   - Host-visible arguments are validated before anything is enqueued; on any error
 *     nothing is enqueued and a status other than ATTN_OK is returned.  Values that live
 *     in device memory (lengths, block ids) cannot be checked without a synchronisation;
 *     they are preconditions, stated per function.
 *   - Unsupported combinations fail loudly with ATTN_ERR_UNSUPPORTED; there is no
 *     fallback path (the-ai.news fused-kernel page, "Attenzione di tipo FlashAttention e
 *     attenzione paginata": forcing a backend that cannot take the input must fail).
 *   - Grouped key/value heads and a sliding window, the two complements of exact attention
 *     the aimpact.prandi.net FlashAttention page lists ("Impatto pratico"), are taken in
 *     their plainest form: `heads` query heads share `kv_heads` K/V heads (heads a multiple
 *     of kv_heads; query head h reads K/V head h / (heads / kv_heads); kv_heads == heads is
 *     ordinary multi-head attention), and a window w > 0 limits query i to the keys
 *     i - w < j <= i (it requires the causal mask; w = 0 means no window).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 5

/* The enumerations are int-sized.  C++ gets the underlying type spelled out, so that any int
 * a caller passes (ctypes, C) is a valid value there too and is rejected by the checks. */
#ifdef __cplusplus
#define ATTN_INT_ENUM : int
#else
#define ATTN_INT_ENUM
#endif

typedef enum attn_status ATTN_INT_ENUM {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, size <= 0, scale not finite or <= 0, bad block size */
  ATTN_ERR_UNSUPPORTED = 2, /* dtype / head_dim / option combination this build has no kernel for */
  ATTN_ERR_WORKSPACE = 3,   /* workspace null or smaller than the matching *_workspace_bytes() */
  ATTN_ERR_LAUNCH = 4       /* the HIP runtime refused the launch (hipGetLastError after it) */
} attn_status;

typedef enum attn_dtype ATTN_INT_ENUM {
  ATTN_F32 = 0,  /* fp32 in, fp32 out */
  ATTN_BF16 = 1  /* bf16 in, bf16 out, fp32 accumulation */
} attn_dtype;

/*
 * attn_fwd — prefill attention of every query of every (batch, head).
 *
 * q, o       : [batch, heads, seq_len, head_dim] of `dtype`, contiguous.  o is written
 *              in full (padding rows included) and may not alias q, k or v.
 * k, v       : [batch, kv_heads, seq_len, head_dim] of `dtype`, contiguous.
 * lse        : optional (NULL allowed) fp32 [batch, heads, seq_len]; receives the natural
 *              log of sum_j exp(scale * <q_i, k_j>) over the admitted keys — the saved
 *              statistic the pages' backward pass recomputes from.
 * seq_lens   : optional (NULL = every row has seq_len) DEVICE int32 [batch].  Positions
 *              >= seq_lens[b] are padding: they are never read as keys or values, and their
 *              query rows get o = 0 and lse = -inf (a row with no admitted key has no
 *              distribution; this is the explicit convention el-ai.com section 5 asks for).
 *              Precondition: 1 <= seq_lens[b] <= seq_len.
 * causal     : nonzero => query i admits keys j <= i only (maeste.it: future keys are set
 *              to -inf before the softmax).  Combines with seq_lens.
 * window     : 0, or w > 0 with causal: query i admits keys i - w < j <= i only.
 * scale      : the factor applied to <q, k>; pass 1/sqrt(head_dim) for the pages' form.
 * Errors     : ATTN_ERR_INVALID also for kv_heads <= 0, heads % kv_heads != 0, window < 0
 *              or a window without causal.
 * Supported  : ATTN_F32 with head_dim 64 or 128 (scores accumulated in fp64);
 *              ATTN_BF16 with head_dim 128 or 64 (MFMA, fp32 accumulation).
 */
attn_status attn_fwd(attn_dtype dtype, const void* q, const void* k, const void* v, void* o,
                     float* lse, const int32_t* seq_lens, int batch, int heads, int kv_heads,
                     int seq_len, int head_dim, int causal, int window, float scale,
                     void* stream);

/*
 * attn_fwd_chunk — prefill attention of a contiguous chunk of queries against a longer key
 * sequence: the q_len query rows are positions q_start .. q_start + q_len - 1 of a sequence
 * whose kv_len keys and values are k and v, and the causal mask and window count those
 * positions (maeste.it: future keys are set to -inf before the softmax).  This is the
 * per-device step of sequence-parallel attention once the K/V shards are gathered (the
 * maeste.it page leaves contexts past one GPU to sequence parallelism over several), and a
 * prefill chunk against a cached prefix; each query block is independent work, as in the
 * query-outer loop of pierluigilucio.it ("I Due Pilastri di FlashAttention", FA2).
 *
 * q, o       : [batch, heads, q_len, head_dim] bf16, contiguous; o written in full.
 * k, v       : [batch, kv_heads, kv_len, head_dim] bf16, contiguous (head_dim 128 or 64).
 * lse        : optional fp32 [batch, heads, q_len], as in attn_fwd.
 * causal     : nonzero => query row i admits keys j <= q_start + i.
 * window     : 0, or w > 0 with causal: row i admits keys q_start + i - w < j <= q_start + i.
 * Errors     : ATTN_ERR_INVALID for null q/k/v/o, sizes <= 0, q_start < 0,
 *              q_start + q_len > kv_len, kv_heads <= 0 or not dividing heads, window < 0 or
 *              without causal, scale not finite or <= 0; ATTN_ERR_UNSUPPORTED for a dtype
 *              other than ATTN_BF16, head_dim not 128 or 64, or sizes past the 32-bit
 *              offsets.
 * With q_start = 0 and q_len = kv_len it computes what attn_fwd computes (no seq_lens).
 */
attn_status attn_fwd_chunk(attn_dtype dtype, const void* q, const void* k, const void* v,
                           void* o, float* lse, int batch, int heads, int kv_heads, int q_len,
                           int kv_len, int q_start, int head_dim, int causal, int window,
                           float scale, void* stream);

/*
 * attn_bwd_workspace_bytes — device bytes attn_bwd needs as `workspace` (one fp32 per query
 * row: D_i = <dO_i, O_i>).  Returns 0 for sizes attn_bwd would reject.
 */
size_t attn_bwd_workspace_bytes(int batch, int heads, int seq_len);

/*
 * attn_bwd — gradients of L = sum(O * dO) with respect to q, k and v, by recomputation: the
 * backward pass of pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (section "Ricalcolo
 * nel Backward Pass"), which keeps only the forward's per-row normalisation statistics and
 * recomputes the weight blocks P_ij = exp(scale <q_i, k_j> - lse_i) from q, k, v.
 *
 * q, o, dout : [batch, heads, seq_len, head_dim] of `dtype`, contiguous; o and lse are
 *              the outputs attn_fwd produced for these q, k, v, mask and scale.
 * k, v       : [batch, kv_heads, seq_len, head_dim] of `dtype`, contiguous.
 * lse        : fp32 [batch, heads, seq_len] (required).
 * seq_lens, kv_heads, causal, window, scale : as in attn_fwd (same values as the forward).
 * dq         : fp32 [batch, heads, seq_len, head_dim], written in full (padding rows 0).
 * dk, dv     : fp32 [batch, kv_heads, seq_len, head_dim], written in full; a shared K/V
 *              head receives the sum over the query heads that read it.
 * workspace  : DEVICE buffer of at least attn_bwd_workspace_bytes() bytes, owned by the
 *              caller; contents on entry do not matter.
 * Supported  : ATTN_BF16 with head_dim 128.
 */
attn_status attn_bwd(attn_dtype dtype, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse,
                     const int32_t* seq_lens, float* dq, float* dk, float* dv, int batch,
                     int heads, int kv_heads, int seq_len, int head_dim, int causal,
                     int window, float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * attn_decode_workspace_bytes — device bytes attn_decode_paged needs as `workspace` for
 * these sizes, this window and this split length (kv_split tokens per partial; 0 = the
 * library's default).  Returns 0 for arguments attn_decode_paged would reject.
 */
size_t attn_decode_workspace_bytes(int batch, int heads, int kv_heads, int head_dim,
                                   int max_seq_len, int window, int kv_split);

/*
 * attn_decode_paged — one new query per sequence against that sequence's paged K/V cache
 * (the decode step of the maeste.it page: a 1 x n score row, bound by reading the cache).
 *
 * q           : [batch, heads, head_dim] bf16.
 * k_cache,
 * v_cache     : [num_blocks, kv_heads, block_size, head_dim] bf16 pools of fixed-size
 *               blocks; one (block, K/V head) is block_size * head_dim contiguous elements.
 *               The query heads that share a K/V head are served together, so each cached
 *               block is read once per K/V head, not once per query head.
 * block_table : DEVICE int32 [batch, max_blocks_per_seq]; entry i of row b is the pool
 *               block holding tokens [i*block_size, (i+1)*block_size) of sequence b (the
 *               block table of the-ai.news page, "attenzione paginata").  Entries past a
 *               sequence's last block are never read.
 * seq_lens    : DEVICE int32 [batch]; the query of sequence b sits at position
 *               seq_lens[b]-1 and admits its tokens 0 .. seq_lens[b]-1 (no mask inside the
 *               cache), or with window w > 0 only the last w of them.  Slots outside that
 *               range are never used, whatever they hold.
 *               Preconditions: 1 <= seq_lens[b] <= max_seq_len, every referenced table
 *               entry in [0, num_blocks).
 * o           : [batch, heads, head_dim] bf16 output.
 * lse         : optional fp32 [batch, heads] natural-log normaliser (see attn_fwd).
 * kv_split    : tokens per split-KV partial, a positive multiple of block_size, or 0 for
 *               the library's default.  Each (sequence, head, split) produces a partial
 *               (m, l, u) that a second kernel merges (el-ai.com section 4); the result
 *               does not depend on kv_split beyond rounding.  Splits start at the first
 *               admitted token.
 * workspace   : DEVICE buffer of at least attn_decode_workspace_bytes(batch, heads,
 *               kv_heads, head_dim, max_seq_len, window, kv_split) bytes, owned by the
 *               caller; its contents on entry do not matter.  Concurrent calls must not
 *               share one workspace.
 * Errors      : ATTN_ERR_INVALID also for kv_heads <= 0, heads % kv_heads != 0 or
 *               window < 0.
 * Supported   : ATTN_BF16, head_dim 128, block_size 16.
 */
attn_status attn_decode_paged(attn_dtype dtype, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int batch,
                              int heads, int kv_heads, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, int max_seq_len,
                              int window, float scale, int kv_split, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged_noalloc — attn_decode_paged for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without `workspace` / `workspace_bytes`, the same kernels and results.
 * The split partials go to a device array of ATTN_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; the call allocates and frees
 * nothing.  Its contents on entry do not matter.
 * Errors     : those of attn_decode_paged; ATTN_ERR_WORKSPACE when
 *              attn_decode_workspace_bytes(...) for these arguments exceeds
 *              ATTN_NOALLOC_SCRATCH_BYTES (nothing is enqueued); ATTN_ERR_LAUNCH when the
 *              array's device address cannot be obtained.
 * Concurrency: calls on one GPU share its array; calls that overlap in time on one GPU (on
 *              different streams or from different host threads) race on it — serialise
 *              them.  Calls on different GPUs are independent.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
attn_status attn_decode_paged_noalloc(attn_dtype dtype, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_table,
                                      const int32_t* seq_lens, void* o, float* lse, int batch,
                                      int heads, int kv_heads, int head_dim, int block_size,
                                      int num_blocks, int max_blocks_per_seq, int max_seq_len,
                                      int window, float scale, int kv_split, void* stream);

/*
 * attn_quantize_fp8 — block quantisation of a bf16 tensor to FP8 E4M3, the operand format of
 * attn_fwd_fp8.  The FP8 part of pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (section
 * "Quantizzazione a Blocchi e Scaling Algebrico") gives each block X the scale
 * s = max|X| / 448 and the codes clip(round(X / s), -448, 448); here a block is 64 rows of
 * one (batch, head), X / s is a correctly rounded fp32 division, and rounding is to nearest,
 * ties to even.  A block that is all 0 gets s = 0 and codes 0.
 *
 * x         : bf16 [batch, heads, seq_len, head_dim], contiguous.
 * x8        : E4M3 codes (OCP E4M3: 1-4-3, bias 7, no infinities), written in full:
 *             transpose = 0: [batch, heads, seq_len, head_dim] (Q and K);
 *             transpose = 1: [batch, heads, head_dim, n_pad] with n_pad = 64*ceil(seq_len/64)
 *             (V, the layout attn_fwd_fp8 reads; the padding columns are 0).
 * scales    : fp32 [batch, heads, ceil(seq_len / 64)].
 * seq_lens  : optional DEVICE int32 [batch]; rows at or past a length count as 0 (code 0).
 * Supported : head_dim 128.
 */
attn_status attn_quantize_fp8(const void* x, void* x8, float* scales, const int32_t* seq_lens,
                              int batch, int heads, int seq_len, int head_dim, int transpose,
                              void* stream);

/*
 * attn_fwd_fp8 — prefill attention on E4M3 operands with per-block scales (pierluigilucio.it
 * "Sviluppo AI ed Algebra Lineare", FP8 part, "Integrazione nel ciclo Online Softmax"): scores (scale * s_Q * s_K) * (Q8 K8^T) accumulated
 * in fp32; maximum, differences and exponentials in fp32; the weights rounded to E4M3 before
 * the P.V product (fp32 accumulation); l sums the rounded weights; o = u / l cast to bf16.
 * The running maximum moves once per 64-key tile (the quantisation block), exactly.
 *
 * q8, q_scale : [batch, heads, seq_len, head_dim] codes and fp32 [batch, heads, nb] scales,
 *               nb = ceil(seq_len / 64), as attn_quantize_fp8 writes them (transpose = 0).
 * k8, k_scale : [batch, kv_heads, seq_len, head_dim] and [batch, kv_heads, nb] (transpose = 0).
 * vt8, v_scale: [batch, kv_heads, head_dim, n_pad] and [batch, kv_heads, nb] (transpose = 1).
 * o           : bf16 [batch, heads, seq_len, head_dim], written in full.
 * lse         : optional fp32 [batch, heads, seq_len]: m + ln(l) of the rounded weights.
 * seq_lens, kv_heads, causal, scale : as in attn_fwd (no window); the lengths must be the
 *               ones the operands were quantised with.
 * Supported   : head_dim 128.
 */
attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale,
                         const float* k_scale, const float* v_scale, void* o, float* lse,
                         const int32_t* seq_lens, int batch, int heads, int kv_heads,
                         int seq_len, int head_dim, int causal, float scale, void* stream);

/*
 * attn_merge — attention over the union of disjoint key sets from each set's own result
 * (el-ai.com "Attenzione: softmax online, riscalamento e memoria", section 4: summaries of
 * disjoint blocks of keys combine by bringing them to the larger maximum and adding).  A
 * part is an output o_s normalised over its own keys and that set's log-sum-exp lse_s, as
 * attn_fwd writes them; the merged row is
 *     lse = ln sum_s exp(lse_s),     o = sum_s exp(lse_s - lse) o_s.
 * It joins the pieces of one query block computed against different key ranges — the
 * per-device step of attention over a sequence whose keys are spread over devices.
 *
 * o_parts   : [parts, rows, head_dim] (dtype), the parts stacked; rows is any row count
 *             (for example batch * heads * seq_len).
 * lse_parts : fp32 [parts, rows], natural log; -inf where a part admits no key of the row
 *             (its output values are then never used: they may hold anything).
 * o         : [rows, head_dim] (dtype), written in full; must not overlap o_parts.  Rows no
 *             part admits get 0.
 * lse       : optional fp32 [rows]; -inf where no part admits the row.
 * Supported : dtype bf16 or f32 (merged in fp32, o rounded to nearest even for bf16),
 *             head_dim 64 or 128, 1 <= parts <= 1024.
 */
attn_status attn_merge(attn_dtype dtype, const void* o_parts, const float* lse_parts, void* o,
                       float* lse, int parts, int64_t rows, int head_dim, void* stream);

/* attn_status_str — static, NUL-terminated name of a status code (never NULL). */
const char* attn_status_str(attn_status status);

/* attn_abi_version — ATTN_ABI_VERSION of the built library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
