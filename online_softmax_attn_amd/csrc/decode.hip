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
// Lane layout inside a 16 x 128 block (4 KiB for K, 4 KiB for V): lane l owns token l / 4
// and the four 16-byte chunks (l % 4) + 4 i, i = 0..3, i.e. 32 of the 128 dimensions.  A
// token's score is a dot2 chain over those 32 dims plus a 4-lane reduction; its weight then
// scales the same lane's 32 values of V, so the accumulator is per lane and is reduced over
// the 16 token slots only once, at the end of the split.
#include "common.h"

namespace {

constexpr int kD = 128;
constexpr int kBlock = 16;
constexpr int kDefaultSplit = 256;

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

__global__ __launch_bounds__(64) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, void* __restrict__ ws,
    int H, int num_blocks, int max_blocks_per_seq, int max_seq_len, int max_splits,
    int split_blocks, float c_log2, size_t n_part) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = min(max(lens[b], 0), max_seq_len);  // out-of-contract lengths stay in bounds
  const int nblk = (L + kBlock - 1) / kBlock;
  const int blk0 = split * split_blocks;
  if (blk0 >= nblk) return;  // beyond this sequence: the merge never reads it
  const int blk1 = min(blk0 + split_blocks, nblk);
  const int tok = lane >> 2, qq = lane & 3;

  // this lane's 32 query dims as bf16 pairs
  uint4 qv[4];
  const bf16* qrow = q + ((size_t)b * H + h) * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) qv[i] = *reinterpret_cast<const uint4*>(qrow + 8 * (qq + 4 * i));

  // table slice for this split: lane j holds entry blk0 + j
  const int tbl = (lane < blk1 - blk0) ? table[(size_t)b * max_blocks_per_seq + blk0 + lane] : 0;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;

  const size_t head_off = (size_t)h * kBlock * kD + (size_t)tok * kD;
  const size_t blk_stride = (size_t)H * kBlock * kD;

  uint4 kb[4], vb[4], kn[4], vn[4];
  auto fetch = [&](int j, uint4* kd, uint4* vd) {
    // out-of-contract block ids are clamped into the pool rather than read out of bounds
    const int phys = min(max(__builtin_amdgcn_readlane(tbl, j), 0), num_blocks - 1);
    const bf16* kp = kc + (size_t)phys * blk_stride + head_off;
    const bf16* vp = vc + (size_t)phys * blk_stride + head_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kd[i] = *reinterpret_cast<const uint4*>(kp + 8 * (qq + 4 * i));
      vd[i] = *reinterpret_cast<const uint4*>(vp + 8 * (qq + 4 * i));
    }
  };

  fetch(0, kb, vb);
  for (int j = 0; j < blk1 - blk0; ++j) {
    if (j + 1 < blk1 - blk0) fetch(j + 1, kn, vn);
    // score of this lane's token
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(&kb[i]);
      const uint32_t* qw = reinterpret_cast<const uint32_t*>(&qv[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw[e]),
                                            __builtin_bit_cast(bf16x2, qw[e]), s, false);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    const int key = (blk0 + j) * kBlock + tok;
    const bool ok = key < L;
    s = ok ? s * c_log2 : -INFINITY;
    float mx = s;
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    mx = fmaxf(mx, __shfl_xor(mx, 8));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // every block holds at least one admitted token, so mx and m_new are finite
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = __builtin_amdgcn_exp2f(s - m_new);
    m_run = m_new;
    l_run = fmaf(l_run, alpha, p);
    if (ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* vw = reinterpret_cast<const uint32_t*>(&vb[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[8 * i + 2 * e] = fmaf(p, bf_lo(vw[e]), acc[8 * i + 2 * e] * alpha);
          acc[8 * i + 2 * e + 1] = fmaf(p, bf_hi(vw[e]), acc[8 * i + 2 * e + 1] * alpha);
        }
      }
    } else {  // slot past the sequence end: its value is never read (it may be anything)
#pragma unroll
      for (int i = 0; i < 32; ++i) acc[i] *= alpha;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kb[i] = kn[i];
      vb[i] = vn[i];
    }
  }

  // reduce over the 16 token slots (lanes with equal lane % 4)
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) {
    l_run += __shfl_xor(l_run, off);
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] += __shfl_xor(acc[i], off);
  }
  const Partials P = partial_views(ws, n_part);
  const size_t p = ((size_t)b * H + h) * max_splits + split;
  if (lane < 4) {
    float* u = P.u + p * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx4 lo, hi;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        lo[c] = acc[8 * i + c];
        hi[c] = acc[8 * i + 4 + c];
      }
      *reinterpret_cast<floatx4*>(u + 8 * (lane + 4 * i)) = lo;
      *reinterpret_cast<floatx4*>(u + 8 * (lane + 4 * i) + 4) = hi;
    }
    if (lane == 0) {
      P.m[p] = m_run;
      P.l[p] = l_run;
    }
  }
}

// merge of the partial summaries of one (sequence, head); thread = one dimension
__global__ __launch_bounds__(kD) void decode_merge_kernel(
    const void* __restrict__ ws, const int32_t* __restrict__ lens, bf16* __restrict__ o,
    float* __restrict__ lse, int H, int max_seq_len, int max_splits, int split_tokens,
    size_t n_part) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(max(lens[b], 0), max_seq_len);
  const int ns = (L + split_tokens - 1) / split_tokens;
  if (ns == 0) {  // no admitted key (out of contract): the empty-row convention
    o[((size_t)b * H + h) * kD + d] = (bf16)0.f;
    if (lse && d == 0) lse[(size_t)b * H + h] = -INFINITY;
    return;
  }
  const Partials P = partial_views(const_cast<void*>(ws), n_part);
  const size_t p0 = ((size_t)b * H + h) * max_splits;
  float mstar = -INFINITY;
  for (int s = 0; s < ns; ++s) mstar = fmaxf(mstar, P.m[p0 + s]);
  float lsum = 0.f, usum = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(P.m[p0 + s] - mstar);
    lsum = fmaf(w, P.l[p0 + s], lsum);
    usum = fmaf(w, P.u[(p0 + s) * kD + d], usum);
  }
  o[((size_t)b * H + h) * kD + d] = (bf16)(usum / lsum);
  if (lse && d == 0) lse[(size_t)b * H + h] = mstar * ATTN_LN2 + __logf(lsum);
}

}  // namespace

int decode_default_split(int batch, int heads, int max_seq_len) {
  (void)batch;
  (void)heads;
  (void)max_seq_len;
  return kDefaultSplit;
}

size_t decode_workspace_bytes(int batch, int heads, int head_dim, int max_seq_len, int split) {
  const size_t max_splits = (size_t)((max_seq_len + split - 1) / split);
  const size_t n_part = (size_t)batch * heads * max_splits;
  return n_part * (2 + (size_t)head_dim) * sizeof(float);
}

hipError_t launch_decode_paged(const bf16* q, const bf16* k_cache, const bf16* v_cache,
                               const int32_t* block_table, const int32_t* seq_lens, bf16* o,
                               float* lse, int batch, int heads, int num_blocks,
                               int max_blocks_per_seq, int max_seq_len, float scale, int split,
                               void* workspace, hipStream_t stream) {
  const int max_splits = (max_seq_len + split - 1) / split;
  const size_t n_part = (size_t)batch * heads * max_splits;
  hipLaunchKernelGGL(decode_split_kernel, dim3(max_splits, heads, batch), dim3(64), 0, stream,
                     q, k_cache, v_cache, block_table, seq_lens, workspace, heads, num_blocks,
                     max_blocks_per_seq, max_seq_len, max_splits, split / kBlock,
                     scale * ATTN_LOG2E, n_part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(heads, batch), dim3(kD), 0, stream, workspace,
                     seq_lens, o, lse, heads, max_seq_len, max_splits, split, n_part);
  return hipGetLastError();
}
