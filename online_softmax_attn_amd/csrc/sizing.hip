// Host-side sizing (sizing.h): host code only, no kernels.
#include "sizing.h"

namespace {

// waves per (sequence, split): decode_gqa_kernel takes up to 32 heads of a group per wave,
// decode_split_kernel one head
long long waves_per_split(int heads, int kv_heads) {
  const int G = heads / kv_heads;
  if (G >= kDecodeMfmaGroup) return (long long)kv_heads * ((G + 31) / 32);
  return heads;
}

}  // namespace

int decode_span_blocks(int max_seq_len, int window) {
  const int all = (int)(((long long)max_seq_len + kDecodeBlock - 1) / kDecodeBlock);
  if (!window) return all;
  const int w = (int)(((long long)window + 2 * kDecodeBlock - 2) / kDecodeBlock);
  return all < w ? all : w;
}

int decode_max_splits(int max_seq_len, int window, int split) {
  const int split_blocks = split / kDecodeBlock;
  return (decode_span_blocks(max_seq_len, window) + split_blocks - 1) / split_blocks;
}

// Split length: as long as possible (each split wave streams its blocks back to back) while
// the grid still offers enough waves to keep every CU's memory pipeline full.  Measured on
// the decode workload (B=32, H=32, lengths up to 8192): 128 tokens 407 us, 256: 390 us,
// 512: 376 us, 768: 376 us, 1024: 378 us.
int decode_default_split(int batch, int heads, int kv_heads, int max_seq_len, int window) {
  const long long wave_heads = waves_per_split(heads, kv_heads);
  const long long span = (long long)decode_span_blocks(max_seq_len, window) * kDecodeBlock;
  if (heads / kv_heads >= kDecodeMfmaGroup) {
    // the matrix-core kernel: its waves start with two dependent memory round trips (page
    // numbers, then the first tiles), so it takes the longest split (at most 1024 tokens)
    // that still gives 2048 waves.  Measured with 8 K/V heads x 8 query heads, 32 sequences
    // of 1024..8192 tokens: 128 tokens 4.2 TB/s, 256: 4.6, 512: 4.9, 1024: 5.5.
    for (int split : {1024, 512, 256, 128}) {
      const long long waves = (long long)batch * wave_heads * ((span + split - 1) / split);
      if (waves >= 2048) return split;
    }
    return 64;
  }
  constexpr long long kTargetWaves = 8192;
  for (int split : {512, 256, 128}) {
    const long long waves = (long long)batch * wave_heads * ((span + split - 1) / split);
    if (waves >= kTargetWaves) return split;
  }
  return 64;
}

size_t decode_workspace_bytes(int batch, int heads, int head_dim, int max_seq_len, int window,
                              int split) {
  size_t n_part = 0, bytes = 0;
  if (__builtin_mul_overflow((size_t)batch, (size_t)heads, &n_part) ||
      __builtin_mul_overflow(n_part, (size_t)decode_max_splits(max_seq_len, window, split), &n_part) ||
      __builtin_mul_overflow(n_part, (2 + (size_t)head_dim) * sizeof(float), &bytes))
    return 0;  // does not fit
  return bytes;
}

size_t bwd_workspace_bytes(int batch, int heads, int n) {
  return (size_t)batch * heads * n * sizeof(float);
}
