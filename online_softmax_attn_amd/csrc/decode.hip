// Split-KV paged decode on gfx950: one bf16 query per sequence, head_dim 128, 16-token blocks.
//
// The decode step reads a sequence's whole K/V cache for one query (maeste.it attention-
// matrix page: a 1 x n score row, bound by memory reads), through the block table of the
// paged cache (the-ai.news fused-kernel page, "attenzione paginata": fixed-size blocks and
// a table from logical position to physical block).  Each (sequence, head) is cut into
// splits of `split` tokens; each split is one wave that keeps the running (m, l, u) summary
// of el-ai.com "Attenzione: softmax online, riscalamento e memoria" (section 2) over its
// blocks and writes it to the workspace.  A second kernel merges the summaries of one
// (sequence, head) as in that page's section 4: bring every partial to the largest maximum
// and add.  There is no data reuse (a GEMV), so the matrix cores are not involved: the
// kernel is shaped for HBM bandwidth — 128-bit loads, the next block's K/V requested before
// the current one is consumed, the table slice fetched once per split.
//
// Lane layout inside a 16 x 128 block (4 KiB for K, 4 KiB for V): one load instruction
// reads 1 KiB contiguous — lane l takes 16-byte chunk l % 16 (dims 8 (l%16) .. +7) of token
// 4 i + l / 16 for i = 0..3.  A token's score is a dot2 chain over the lane's 8 dims and a
// 16-lane DPP reduction; its weight scales the same lane's 8 values of V, so the
// accumulator is 8 floats per lane, reduced over the four 16-lane groups once per split.
#include "common.h"

namespace {
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// K/V are read exactly once: non-temporal loads keep them from displacing useful cache
// lines (measured: +6% bandwidth on the decode workload).
__device__ __forceinline__ uint4 load_stream(const bf16* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

constexpr int kD = 128;
constexpr int kBlock = 16;
#ifndef ATTN_DECODE_DEPTH
#define ATTN_DECODE_DEPTH 2
#endif
constexpr int kDepth = ATTN_DECODE_DEPTH;  // blocks requested ahead of the one being consumed

struct Partials {  // workspace views; index p = (b * H + h) * max_splits + split
  float* m;        // running max, log2 units
  float* l;        // normaliser
  float* u;        // [p][128] unnormalised accumulator
};

__device__ __forceinline__ Partials partial_views(void* ws, size_t n_part) {
  float* f = reinterpret_cast<float*>(ws);
  return Partials{f, f + n_part, f + 2 * n_part};
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), kCtrl,
                                                            0xF, 0xF, true));
}
// sum over the 16 lanes of a row: swaps within pairs, quads, half-rows, rows
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}
__device__ __forceinline__ float xor16(float x) {  // own + lane ^ 16
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32(float x) {  // own + lane ^ 32
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct Block {
  uint4 k[4], v[4];  // token 4 i + lane/16, dims 8 (lane%16) .. +7
};

// One wave per (sequence, K/V head, split, group of GQ query heads sharing that K/V head:
// every block loaded is scored and accumulated GQ times).  Launched with GQ = 1 (plain
// multi-head attention); groups of kDecodeMfmaGroup or more query heads go to decode_gqa_kernel.
// Tokens [kbeg, L) are admitted (kbeg > 0 under a window); splits count blocks from the one
// holding kbeg.
template <int GQ>
__global__ __launch_bounds__(64) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, void* __restrict__ ws,
    int H, int Hkv, int num_blocks, int max_blocks_per_seq, int max_seq_len, int window,
    int max_splits, int split_blocks, float c_log2, size_t n_part) {
  // heads fastest: waves dispatched together read neighbouring 4 KiB pieces of one block
  const int chunks = H / Hkv / GQ;  // query-head groups per K/V head
  const int hk = blockIdx.x / chunks;
  const int h0 = hk * (H / Hkv) + (blockIdx.x % chunks) * GQ;  // first query head served
  const int split = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = min(max(lens[b], 0), max_seq_len);  // out-of-contract lengths stay in bounds
  const int kbeg = window ? max(L - window, 0) : 0;
  const int nblk = (L + kBlock - 1) / kBlock;
  const int blk0 = kbeg / kBlock + split * split_blocks;
  if (blk0 >= nblk) return;  // beyond this sequence: the merge never reads it
  const int count = min(blk0 + split_blocks, nblk) - blk0;
  const int grp = lane >> 4, dc = lane & 15;

  // this lane's 8 dims of each served query, as bf16 pairs
  uint4 qv[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g)
    qv[g] = *reinterpret_cast<const uint4*>(q + ((size_t)b * H + h0 + g) * kD + 8 * dc);
  // table slice for this split: lane j holds entry blk0 + j
  const int tbl = (lane < count) ? table[(size_t)b * max_blocks_per_seq + blk0 + lane] : 0;

  const size_t blk_stride = (size_t)Hkv * kBlock * kD;
  const size_t lane_off = (size_t)hk * kBlock * kD + (size_t)grp * kD + 8 * dc;
  auto fetch = [&](int j, Block& d) {
    // out-of-contract block ids are clamped into the pool rather than read out of bounds
    const int phys = min(max(__builtin_amdgcn_readlane(tbl, j), 0), num_blocks - 1);
    const bf16* kp = kc + (size_t)phys * blk_stride + lane_off;
    const bf16* vp = vc + (size_t)phys * blk_stride + lane_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) d.k[i] = load_stream(kp + 4 * i * kD);
#pragma unroll
    for (int i = 0; i < 4; ++i) d.v[i] = load_stream(vp + 4 * i * kD);
  };

  float m_run[GQ], l_run[GQ], acc[GQ][8];
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
  }

  auto consume = [&](int j, const Block& d) {
    const int tok0 = (blk0 + j) * kBlock + grp;  // token of score i is tok0 + 4 i
    const bool edge = (blk0 + j + 1) * kBlock > L || (blk0 + j) * kBlock < kbeg;
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ok[i] = !edge || (tok0 + 4 * i < L && tok0 + 4 * i >= kbeg);
    float vf[4][8];  // V as fp32, shared by the served heads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(&d.v[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[i][2 * e] = bf_lo(vw[e]);
        vf[i][2 * e + 1] = bf_hi(vw[e]);
      }
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      float s[4];
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qv[g]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* kw = reinterpret_cast<const uint32_t*>(&d.k[i]);
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]),
                                              __builtin_bit_cast(bf16x2, qw[e]), x, false);
        s[i] = row_sum16(x);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = ok[i] ? s[i] * c_log2 : -INFINITY;
        mx = __builtin_fmaxf(mx, s[i]);
      }
      mx = max32(max16(mx));
      // every block holds at least one admitted token, so mx and m_new are finite
      const float m_new = __builtin_fmaxf(m_run[g], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[g] - m_new);
      m_run[g] = m_new;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = ok[i] ? __builtin_amdgcn_exp2f(s[i] - m_new) : 0.f;
      l_run[g] = fmaf(l_run[g], alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= alpha;
      // a slot outside the admitted range has p = 0 by selection, so whatever it holds
      // (NaN included) is never multiplied in
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!ok[i]) continue;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[g][c] = fmaf(p[i], vf[i][c], acc[g][c]);
      }
    }
  };

  // software pipeline: kDepth + 1 register buffers, loads kDepth blocks ahead
  constexpr int kDep = kDepth;
  Block buf[kDep + 1];
#pragma unroll
  for (int j = 0; j < kDep; ++j)
    if (j < count) fetch(j, buf[j]);
  int j = 0;
  for (; j + kDep + 1 <= count; j += kDep + 1) {
#pragma unroll
    for (int r = 0; r <= kDep; ++r) {
      if (j + r + kDep < count) fetch(j + r + kDep, buf[(r + kDep) % (kDep + 1)]);
      consume(j + r, buf[r]);
    }
  }
#pragma unroll
  for (int r = 0; r <= kDep; ++r)
    if (j + r < count) consume(j + r, buf[r]);

  const Partials P = partial_views(ws, n_part);
#pragma unroll
  for (int g = 0; g < GQ; ++g) {
    // reduce over the four 16-lane groups (each lane summed its own tokens)
    const float l_tot = xor32(xor16(l_run[g]));
    float a[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) a[c] = xor32(xor16(acc[g][c]));
    const size_t p = ((size_t)b * H + h0 + g) * max_splits + split;
    if (lane < 16) {
      float* u = P.u + p * kD + 8 * dc;
      floatx4 lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo[c] = a[c];
        hi[c] = a[4 + c];
      }
      // streamed past the caches (the sixteen lanes write the head's whole 512-byte row):
      // 1.2% faster on the decode workload with a cache flush before each call
      __builtin_nontemporal_store(lo, reinterpret_cast<floatx4*>(u));
      __builtin_nontemporal_store(hi, reinterpret_cast<floatx4*>(u + 4));
      if (lane == 0) {
        __builtin_nontemporal_store(m_run[g], P.m + p);
        __builtin_nontemporal_store(l_tot, P.l + p);
      }
    }
  }
}

// merge of the partial summaries of one (sequence, head): one wave, lane = 2 dimensions.
// The partials of the first kMergePre splits (lane s: split s's m and l; every lane: its
// two dimensions of each u row) are loaded together with the sequence length, before the
// split count is known: they lie inside this (sequence, head)'s rows of the workspace, and
// only the first ns of them are used.  The merge then waits for one memory round trip
// instead of three (length, then maxima, then the rows): 7.1 -> 5.3 us on the decode
// workload.  The arithmetic and its order are those of a plain loop over the splits.
constexpr int kMergePre = 16;
__global__ __launch_bounds__(64) void decode_merge_kernel(
    const void* __restrict__ ws, const int32_t* __restrict__ lens, bf16* __restrict__ o,
    float* __restrict__ lse, int H, int max_seq_len, int window, int max_splits,
    int split_blocks, size_t n_part) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const Partials P = partial_views(const_cast<void*>(ws), n_part);
  const size_t p0 = ((size_t)b * H + h) * max_splits;
  float m_lane = -INFINITY, l_lane = 0.f;
  if (lane < max_splits) {
    m_lane = P.m[p0 + lane];
    l_lane = P.l[p0 + lane];
  }
  floatx2 up[kMergePre];
#pragma unroll
  for (int s = 0; s < kMergePre; ++s)
    up[s] = s < max_splits ? *reinterpret_cast<const floatx2*>(P.u + (p0 + s) * kD + 2 * lane)
                           : floatx2{0.f, 0.f};
  const int L = min(max(lens[b], 0), max_seq_len);
  const int kbeg = window ? max(L - window, 0) : 0;
  const int nblk = (L + kBlock - 1) / kBlock - kbeg / kBlock;  // blocks the splits cover
  const int ns = (nblk + split_blocks - 1) / split_blocks;
  const size_t out = ((size_t)b * H + h) * kD + 2 * lane;
  if (ns == 0) {  // no admitted key (out of contract): the empty-row convention
    o[out] = (bf16)0.f;
    o[out + 1] = (bf16)0.f;
    if (lse && lane == 0) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  float mstar = lane < ns ? m_lane : -INFINITY;
  for (int s = lane + 64; s < ns; s += 64) mstar = __builtin_fmaxf(mstar, P.m[p0 + s]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mstar = __builtin_fmaxf(mstar, __shfl_xor(mstar, off));
  const float w_lane = __builtin_amdgcn_exp2f(m_lane - mstar);  // split `lane`'s weight
  float lsum = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
  for (int s = 0; s < kMergePre; ++s) {
    if (s < ns) {
      const float w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(w_lane), s));
      const float l = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(l_lane), s));
      lsum = fmaf(w, l, lsum);
      u0 = fmaf(w, up[s][0], u0);
      u1 = fmaf(w, up[s][1], u1);
    }
  }
#pragma unroll 8
  for (int s = kMergePre; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(P.m[p0 + s] - mstar);
    const floatx2 uu = *reinterpret_cast<const floatx2*>(P.u + (p0 + s) * kD + 2 * lane);
    lsum = fmaf(w, P.l[p0 + s], lsum);
    u0 = fmaf(w, uu[0], u0);
    u1 = fmaf(w, uu[1], u1);
  }
  const float inv = 1.0f / lsum;
  floatx2 r;
  r[0] = u0 * inv;
  r[1] = u1 * inv;
  *reinterpret_cast<bf16x2*>(o + out) = __builtin_convertvector(r, bf16x2);
  if (lse && lane == 0) lse[(size_t)b * H + h] = mstar * ATTN_LN2 + __logf(lsum);
}

}  // namespace

hipError_t launch_decode_paged(const bf16* q, const bf16* k_cache, const bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, bf16* o,
                               float* lse, int batch, int heads, int kv_heads, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, int window, float scale,
                               int split, void* workspace, hipStream_t stream) {
  const int max_splits = decode_max_splits(max_seq_len, window, split);
  const size_t n_part = (size_t)batch * heads * max_splits;
  if (heads / kv_heads >= kDecodeMfmaGroup) {
    const hipError_t e = launch_decode_gqa(q, k_cache, v_cache, block_table, seq_lens, batch, heads,
                                           kv_heads, num_blocks, max_blocks_per_seq, max_seq_len,
                                           window, scale, split, max_splits, workspace, n_part,
                                           stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_merge_kernel, dim3(heads, batch), dim3(64), 0, stream, workspace,
                       seq_lens, o, lse, heads, max_seq_len, window, max_splits, split / kBlock,
                       n_part);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)heads, (unsigned)max_splits, (unsigned)batch);
  hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(64), 0, stream, q, k_cache, v_cache,
                     block_table, seq_lens, workspace, heads, kv_heads, num_blocks,
                     max_blocks_per_seq, max_seq_len, window, max_splits, split / kBlock,
                     scale * ATTN_LOG2E, n_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(heads, batch), dim3(64), 0, stream, workspace,
                     seq_lens, o, lse, heads, max_seq_len, window, max_splits, split / kBlock,
                     n_part);
  return hipGetLastError();
}
