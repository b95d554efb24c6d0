// Host-side sizing shared by the C ABI layer and the launchers: the decode's split length,
// split count and partial-summary workspace, and the backward's workspace.  Plain C++ with
// no HIP types, so the validation layer can be built and checked on a host without a GPU.
#pragma once

#include <stddef.h>

constexpr int kDecodeBlock = 16;                    // tokens per cache page
constexpr int kDecodeMaxSplit = 64 * kDecodeBlock;  // one table entry per lane of a wave

// Groups of at least this many query heads per K/V head run on the matrix cores
// (decode_gqa_kernel); single heads (plain multi-head attention) on the vector units
// (decode_split_kernel, one query head per wave).  Measured on 32 sequences of 1024..8192
// tokens, 8 K/V heads, a 1 GiB write before each call: the matrix-core kernel reads 5.8 /
// 5.6 / 5.4 / 5.0 TB/s at 2 / 4 / 8 / 16 heads per group, the vector kernel (one wave
// serving 2 or 4 heads of a group) 5.5 / 4.6 TB/s at 2 / 4.
constexpr int kDecodeMfmaGroup = 2;

// Pages a sequence's admitted tokens can touch: all of them, or under a window of w the w
// tokens [L - w, L), which straddle at most ceil((w + 15) / 16) pages.
int decode_span_blocks(int max_seq_len, int window);
// Splits of `split` tokens over that span.
int decode_max_splits(int max_seq_len, int window, int split);
// Default split length of attn_decode_paged (kv_split = 0).
int decode_default_split(int batch, int heads, int kv_heads, int max_seq_len, int window);
// Bytes of the split partials (m, l, u per query head and split); 0 if that does not fit in
// size_t.
size_t decode_workspace_bytes(int batch, int heads, int head_dim, int max_seq_len, int window,
                              int split);
// Bytes of the backward's workspace (D = rowsum(dO * O), one float per query row).
size_t bwd_workspace_bytes(int batch, int heads, int n);
