// Shared device types and launch declarations of the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn.h"
#include "sizing.h"

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));

#define ATTN_LOG2E 1.4426950408889634f
#define ATTN_LN2 0.6931471805599453f

// Launchers (host side).  Arguments are already validated by the C ABI layer; each returns
// the HIP status of its launch(es).  `kv_heads` divides `heads` (query head h reads K/V head
// h / (heads / kv_heads)); `window` is 0 or a causal window length.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const int32_t* seq_lens, int batch, int heads, int kv_heads, int n,
                          int head_dim, int causal, int window, float scale, hipStream_t stream);

// bf16 prefill: n query rows at positions q_start .. q_start + n - 1 of a key sequence of
// n_kv rows (the plain call: n_kv = n, q_start = 0; seq_lens only with the plain call);
// head_dim 128 or 64.
hipError_t launch_fwd_bf16(const bf16* q, const bf16* k, const bf16* v, bf16* o, float* lse,
                           const int32_t* seq_lens, int batch, int heads, int kv_heads, int n,
                           int n_kv, int q_start, int head_dim, int causal, int window,
                           float scale, hipStream_t stream);

// Backward pass (bf16 in, fp32 gradients): D = rowsum(dO * O) into `workspace`, then dQ
// and dK/dV kernels that recompute the weights from the saved log-sum-exp.
hipError_t launch_bwd_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o,
                           const bf16* dout, const float* lse, const int32_t* seq_lens,
                           float* dq, float* dk, float* dv, int batch, int heads, int kv_heads,
                           int n, int causal, int window, float scale, void* workspace,
                           hipStream_t stream);

// Split-KV paged decode: partials into `workspace`, then the merge pass writes o / lse.
hipError_t launch_decode_paged(const bf16* q, const bf16* k_cache, const bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, bf16* o,
                               float* lse, int batch, int heads, int kv_heads, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, int window, float scale,
                               int split, void* workspace, hipStream_t stream);

// Every host-visible check of attn_decode_paged (include/attn.h); on ATTN_OK also the split
// length the call will use and the workspace bytes it needs.
attn_status decode_paged_check(attn_dtype dtype, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_table,
                               const int32_t* seq_lens, const void* o, int batch, int heads,
                               int kv_heads, int head_dim, int block_size, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, int window, float scale,
                               int kv_split, int* split, size_t* need);

// Grouped-head decode on the matrix cores (partials in the layout decode_merge_kernel reads);
// launch_decode_paged picks it for groups of 8 or more query heads per K/V head.
hipError_t launch_decode_gqa(const bf16* q, const bf16* k_cache, const bf16* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int batch,
                             int heads, int kv_heads, int num_blocks, int max_blocks_per_seq,
                             int max_seq_len, int window, float scale, int split, int max_splits,
                             void* workspace, size_t n_part, hipStream_t stream);

// FP8 E4M3 path: 64-row block quantisation, then attention on the codes.
hipError_t launch_quantize_fp8(const bf16* x, uint8_t* x8, float* scales, const int32_t* seq_lens,
                               int batch, int heads, int n, int transpose, hipStream_t stream);
hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          bf16* o, float* lse, const int32_t* seq_lens, int batch, int heads,
                          int kv_heads, int n, int causal, float scale, hipStream_t stream);

// Merge of results over disjoint key sets: parts [n_parts, rows, head_dim] (bf16 or fp32)
// with their fp32 lse [n_parts, rows] into out [rows, head_dim] and lse_out [rows].
hipError_t launch_merge(bool bf16_data, const void* parts, const float* lse_parts, void* out,
                        float* lse_out, int n_parts, long long rows, int head_dim,
                        hipStream_t stream);

// ---------------------------------------------------------------------------------------
// Launch order of a causal grid: `n_tiles` work tiles per (batch, head), `HB` (batch, head)s,
// one workgroup each.  Workgroups are dealt round-robin to the 8 XCDs (block % 8), so XCD x
// receives blocks x, x+8, ...  Each XCD gets a contiguous range of HB/8 (batch, head)s, taken
// eight at a time: all tiles of eight heads, heaviest first, before the next eight.  About 64
// workgroups are resident per XCD (32 CUs, two each), so few heads are in flight on one XCD
// and their K/V are mostly re-read from its 4 MiB L2, while the heavy tiles of a group still
// start early enough to keep the tail short.  Measured on the causal prefill [4,32,2048,128]
// (16 heads per XCD): reads from MALL/HBM of 353 MB per launch against 599 MB when all 16
// heads of an XCD run at once, 1-3% faster; groups of four read only the compulsory 202 MB
// but run 1-5% slower (their last group's heavy tiles lengthen the tail).  `rank` is the
// tile's place in heaviness order (0 = most work).
struct GridSlot {
  int rank;
  int bh;
};
__device__ __forceinline__ GridSlot causal_grid_slot(int block, int HB, int n_tiles) {
  constexpr int kGroup = 8;
  if (HB % (8 * kGroup) == 0) {
    const int x = block % 8, i = block / 8, span = kGroup * n_tiles;
    return {(i % span) / kGroup, x * (HB / 8) + (i / span) * kGroup + i % kGroup};
  }
  const int j = block % HB;  // all tiles of one rank, then the next
  return {block / HB, (HB % 8 == 0) ? (j % 8) * (HB / 8) + j / 8 : j};
}

// ---------------------------------------------------------------------------------------
// Buffer resources: loads through a buffer descriptor return 0 for any byte offset at or
// past `bytes`, which is how out-of-range rows (ragged tails, padding) are zero-filled
// without branches.  The fourth descriptor word is the gfx9-family default format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
typedef __attribute__((address_space(3))) void lds_void;
// 16 bytes per lane from global (buffer offset `voff`) straight into LDS: lane i of the
// wave writes lds_base + 16 * i.  lds_base must be wave-uniform.
__device__ __forceinline__ void load_lds16(rsrc_t r, lds_void* lds_base, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 load_b128(rsrc_t r, int voff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
