// C ABI of libattn.so: argument validation, kernel selection, launch on the caller's stream.
// The contract of every entry point is documented in include/attn.h.
#include "attn.h"

#include <climits>
#include <cmath>

#include "common.h"

namespace {

bool finite_positive(float x) { return std::isfinite(x) && x > 0.f; }

// a * b * c for factors >= 0, or LLONG_MAX when the product does not fit in 64 bits (the
// size checks below compare such products against the 32-bit limits of offsets and grids)
long long mul3(long long a, long long b, long long c) {
  long long ab = 0, abc = 0;
  if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc)) return LLONG_MAX;
  return abc;
}

// number of `tile`-row tiles covering n rows
long long tiles(int n, int tile) { return ((long long)n + tile - 1) / tile; }

attn_status launch_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

// grouped heads and window: heads a positive multiple of kv_heads, window >= 0
bool heads_window_ok(int heads, int kv_heads, int window) {
  return kv_heads > 0 && heads % kv_heads == 0 && window >= 0;
}

// the split length attn_decode_paged will use, or 0 if `kv_split` is not acceptable
int resolve_split(int batch, int heads, int kv_heads, int max_seq_len, int window, int kv_split) {
  if (kv_split == 0) return decode_default_split(batch, heads, kv_heads, max_seq_len, window);
  if (kv_split < 0 || kv_split % kDecodeBlock != 0 || kv_split > kDecodeMaxSplit) return 0;
  return kv_split;
}

}  // namespace

attn_status decode_paged_check(attn_dtype dtype, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const void* o, int batch, int heads,
                               int kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, int window, float scale,
                               int kv_split, int* split, size_t* need) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || head_dim <= 0 || num_blocks <= 0 || max_seq_len <= 0)
    return ATTN_ERR_INVALID;
  if (block_size <= 0 || max_blocks_per_seq <= 0) return ATTN_ERR_INVALID;
  if (!heads_window_ok(heads, kv_heads, window)) return ATTN_ERR_INVALID;
  if (!finite_positive(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 || head_dim != 128 || block_size != kDecodeBlock)
    return ATTN_ERR_UNSUPPORTED;
  if ((long long)max_blocks_per_seq * block_size < max_seq_len) return ATTN_ERR_INVALID;
  if (batch > 65535 || heads > 65535) return ATTN_ERR_UNSUPPORTED;  // grid.y / grid.z limits
  *split = resolve_split(batch, heads, kv_heads, max_seq_len, window, kv_split);
  if (*split == 0) return ATTN_ERR_INVALID;
  *need = decode_workspace_bytes(batch, heads, head_dim, max_seq_len, window, *split);
  if (*need == 0) return ATTN_ERR_UNSUPPORTED;  // the partials' size does not fit in size_t
  return ATTN_OK;
}

extern "C" {

int attn_abi_version(void) { return ATTN_ABI_VERSION; }

const char* attn_status_str(attn_status status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID: return "ATTN_ERR_INVALID";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
    case ATTN_ERR_LAUNCH: return "ATTN_ERR_LAUNCH";
  }
  return "ATTN_ERR_UNKNOWN";
}

attn_status attn_fwd(attn_dtype dtype, const void* q, const void* k, const void* v, void* o,
                     float* lse, const int32_t* seq_lens, int batch, int heads, int kv_heads,
                     int seq_len, int head_dim, int causal, int window, float scale,
                     void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (!heads_window_ok(heads, kv_heads, window) || (window > 0 && !causal)) return ATTN_ERR_INVALID;
  if (!finite_positive(scale)) return ATTN_ERR_INVALID;
  // 32-bit byte offsets inside one (batch, head) slice
  const long long elem = dtype == ATTN_F32 ? 4 : 2;
  if (mul3(seq_len, head_dim, elem) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  if (mul3(batch, heads, tiles(seq_len, 128)) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == ATTN_F32) {
    if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
    if ((long long)batch * heads >= 65536) return ATTN_ERR_UNSUPPORTED;  // grid.y limit
    return launch_status(launch_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                        static_cast<const float*>(v), static_cast<float*>(o), lse,
                                        seq_lens, batch, heads, kv_heads, seq_len, head_dim,
                                        causal != 0, window, scale, s));
  }
  if (dtype == ATTN_BF16) {
    if (head_dim != 128 && head_dim != 64) return ATTN_ERR_UNSUPPORTED;
    return launch_status(launch_fwd_bf16(static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                                         static_cast<const bf16*>(v), static_cast<bf16*>(o), lse,
                                         seq_lens, batch, heads, kv_heads, seq_len, seq_len, 0,
                                         head_dim, causal != 0, window, scale, s));
  }
  return ATTN_ERR_UNSUPPORTED;
}

attn_status attn_fwd_chunk(attn_dtype dtype, const void* q, const void* k, const void* v,
                           void* o, float* lse, int batch, int heads, int kv_heads, int q_len,
                           int kv_len, int q_start, int head_dim, int causal, int window,
                           float scale, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || q_len <= 0 || kv_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (q_start < 0 || (long long)q_start + q_len > kv_len) return ATTN_ERR_INVALID;
  if (!heads_window_ok(heads, kv_heads, window) || (window > 0 && !causal)) return ATTN_ERR_INVALID;
  if (!finite_positive(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 || (head_dim != 128 && head_dim != 64)) return ATTN_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside one (batch, head) slice
  if (mul3(kv_len, head_dim, 2) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  if (mul3(batch, heads, tiles(q_len, 128)) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  return launch_status(launch_fwd_bf16(static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                                       static_cast<const bf16*>(v), static_cast<bf16*>(o), lse,
                                       nullptr, batch, heads, kv_heads, q_len, kv_len, q_start,
                                       head_dim, causal != 0, window, scale,
                                       reinterpret_cast<hipStream_t>(stream)));
}

size_t attn_bwd_workspace_bytes(int batch, int heads, int seq_len) {
  if (batch <= 0 || heads <= 0 || seq_len <= 0) return 0;
  if (mul3(batch, heads, tiles(seq_len, 128)) >= (1LL << 31)) return 0;  // attn_bwd rejects it
  return bwd_workspace_bytes(batch, heads, seq_len);
}

attn_status attn_bwd(attn_dtype dtype, const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse,
                     const int32_t* seq_lens, float* dq, float* dk, float* dv, int batch,
                     int heads, int kv_heads, int seq_len, int head_dim, int causal,
                     int window, float scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (!heads_window_ok(heads, kv_heads, window) || (window > 0 && !causal)) return ATTN_ERR_INVALID;
  if (!finite_positive(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 || head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside one (batch, head) slice; one fp32 gradient row is 512 bytes
  if (mul3(seq_len, head_dim, 4) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  if (mul3(batch, heads, tiles(seq_len, 128)) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < bwd_workspace_bytes(batch, heads, seq_len))
    return ATTN_ERR_WORKSPACE;
  return launch_status(launch_bwd_bf16(
      static_cast<const bf16*>(q), static_cast<const bf16*>(k), static_cast<const bf16*>(v),
      static_cast<const bf16*>(o), static_cast<const bf16*>(dout), lse, seq_lens, dq, dk, dv,
      batch, heads, kv_heads, seq_len, causal != 0, window, scale, workspace,
      reinterpret_cast<hipStream_t>(stream)));
}

attn_status attn_quantize_fp8(const void* x, void* x8, float* scales, const int32_t* seq_lens,
                              int batch, int heads, int seq_len, int head_dim, int transpose,
                              void* stream) {
  if (!x || !x8 || !scales) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)batch * heads > 65535) return ATTN_ERR_UNSUPPORTED;  // grid.y limit
  return launch_status(launch_quantize_fp8(static_cast<const bf16*>(x), static_cast<uint8_t*>(x8),
                                           scales, seq_lens, batch, heads, seq_len, transpose != 0,
                                           reinterpret_cast<hipStream_t>(stream)));
}

attn_status attn_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale,
                         const float* k_scale, const float* v_scale, void* o, float* lse,
                         const int32_t* seq_lens, int batch, int heads, int kv_heads,
                         int seq_len, int head_dim, int causal, float scale, void* stream) {
  if (!q8 || !k8 || !vt8 || !q_scale || !k_scale || !v_scale || !o) return ATTN_ERR_INVALID;
  if (batch <= 0 || heads <= 0 || seq_len <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (!heads_window_ok(heads, kv_heads, 0)) return ATTN_ERR_INVALID;
  if (!finite_positive(scale)) return ATTN_ERR_INVALID;
  if (head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside one (batch, head) slice, also of the transposed V
  if (mul3(tiles(seq_len, 64), 64, head_dim) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  if (mul3(batch, heads, tiles(seq_len, 128)) >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;
  return launch_status(launch_fwd_fp8(
      static_cast<const uint8_t*>(q8), static_cast<const uint8_t*>(k8),
      static_cast<const uint8_t*>(vt8), q_scale, k_scale, v_scale, static_cast<bf16*>(o), lse,
      seq_lens, batch, heads, kv_heads, seq_len, causal != 0, scale,
      reinterpret_cast<hipStream_t>(stream)));
}

attn_status attn_merge(attn_dtype dtype, const void* o_parts, const float* lse_parts, void* o,
                       float* lse, int parts, int64_t rows, int head_dim, void* stream) {
  if (!o_parts || !lse_parts || !o) return ATTN_ERR_INVALID;
  if (parts <= 0 || rows <= 0 || head_dim <= 0) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return ATTN_ERR_UNSUPPORTED;
  if (parts > 1024) return ATTN_ERR_UNSUPPORTED;
  if ((rows - 1) / 16 + 1 >= (1LL << 31)) return ATTN_ERR_UNSUPPORTED;  // grid: 16 rows per workgroup
  return launch_status(launch_merge(dtype == ATTN_BF16, o_parts, lse_parts, o, lse, parts,
                                    (long long)rows, head_dim,
                                    reinterpret_cast<hipStream_t>(stream)));
}

size_t attn_decode_workspace_bytes(int batch, int heads, int kv_heads, int head_dim,
                                   int max_seq_len, int window, int kv_split) {
  if (batch <= 0 || heads <= 0 || head_dim != 128 || max_seq_len <= 0) return 0;
  if (!heads_window_ok(heads, kv_heads, window)) return 0;
  if (batch > 65535 || heads > 65535) return 0;  // attn_decode_paged rejects these grids
  const int split = resolve_split(batch, heads, kv_heads, max_seq_len, window, kv_split);
  if (split == 0) return 0;
  return decode_workspace_bytes(batch, heads, head_dim, max_seq_len, window, split);
}

attn_status attn_decode_paged(attn_dtype dtype, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int batch,
                              int heads, int kv_heads, int head_dim, int block_size,
                              int num_blocks, int max_blocks_per_seq, int max_seq_len,
                              int window, float scale, int kv_split, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int split = 0;
  size_t need = 0;
  const attn_status st = decode_paged_check(dtype, q, k_cache, v_cache, block_table, seq_lens,
                                            o, batch, heads, kv_heads, head_dim, block_size,
                                            num_blocks, max_blocks_per_seq, max_seq_len, window,
                                            scale, kv_split, &split, &need);
  if (st != ATTN_OK) return st;
  if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  return launch_status(launch_decode_paged(
      static_cast<const bf16*>(q), static_cast<const bf16*>(k_cache),
      static_cast<const bf16*>(v_cache), block_table, seq_lens, static_cast<bf16*>(o), lse,
      batch, heads, kv_heads, num_blocks, max_blocks_per_seq, max_seq_len, window, scale, split,
      workspace, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
