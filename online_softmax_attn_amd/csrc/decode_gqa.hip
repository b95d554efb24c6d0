// Split-KV paged decode for grouped K/V heads on gfx950 matrix cores (bf16, head_dim 128).
//
// Same computation as decode_split_kernel (the decode step of the maeste.it page through the
// paged cache of the-ai.news page, partial (m, l, u) summaries of el-ai.com "Attenzione:
// softmax online, riscalamento e memoria" section 2, merged by decode_merge_kernel as in
// its section 4), for the case where several query heads share a K/V head (grouped heads,
// named by aimpact.prandi.net "Impatto pratico").  The G query heads of a group read the
// same cache, so their scores form a real matrix product: a wave takes up to 32 of them as
// the columns of S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 — the register
// layouts of the bf16 prefill kernel, with the group's heads in place of its 32 queries.
// The cache is read once per K/V head; the matrix cores have ample headroom (at most 32
// columns of a 32-token tile per 16 KiB read), so the kernel stays bound by HBM.
//
// Tiles are 32 tokens = two 16-token pages.  Each wave owns a 3-slot LDS ring (K and V,
// 8 KiB each per slot) filled by direct global->LDS loads, two tiles ahead.  Every page gets
// its own buffer descriptor (64-bit page address), whose range ends at the sequence length
// in the last page, so slots past it read as 0; a missing second page of a split's last
// tile has an empty range (zeros).  Tokens before the window read their real cache rows;
// their V rows are cleared in LDS so whatever they hold never meets a zero weight.
#include "common.h"

namespace {

constexpr int kD = 128;
constexpr int kBlock = 16;
constexpr int kTile = 32;                   // tokens per tile (two pages)
constexpr int kCols = 32;                   // query heads per wave (MFMA columns)
constexpr int kStages = 3;
constexpr int kTileElems = kTile * kD;      // 8 KiB of bf16

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

struct Partials {  // workspace views (the layout decode_merge_kernel reads)
  float* m;
  float* l;
  float* u;
};

// LDS element offsets of logical 16-byte chunk c of tile row r (the prefill swizzles: K rows
// read whole, V rows read transposed)
__device__ __forceinline__ int k_slot(int r, int c) { return r * kD + ((c ^ (r & 15)) << 3); }
__device__ __forceinline__ int v_slot(int r, int c) { return r * kD + ((c ^ ((r & 3) << 2)) << 3); }

__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A fill of 16 bytes per lane marked non-temporal: the cache is read once, and loads that
// allocate in the caches evict (and write back) whatever the caches hold; with the caches
// full of dirty lines from earlier work, the normal policy halves the read rate here
// (measured: 3.1 vs 4.5 TB/s, 8 K/V heads with 8 query heads each)
__device__ __forceinline__ void load_lds16_nt(rsrc_t r, lds_void* lds_base, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, voff, 0, 0, 2);
}

// s_waitcnt immediate (gfx9 encoding): vector-memory count <= n, the other counts unconstrained
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

__global__ __launch_bounds__(64) void decode_gqa_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc,
    const int32_t* __restrict__ table, const int32_t* __restrict__ lens, void* __restrict__ ws,
    int H, int Hkv, int num_blocks, int max_blocks_per_seq, int max_seq_len, int window,
    int max_splits, int split_blocks, float c_log2, size_t n_part) {
  // K ring slots 0-2, V ring slots 3-5 (one LDS object: the compiler then keeps the
  // non-aliasing of the slots declared below)
  __shared__ __attribute__((aligned(1024))) bf16 tiles[2 * kStages][kTileElems];

  const int G = H / Hkv;
  const int chunks = (G + kCols - 1) / kCols;
  const int hk = blockIdx.x / chunks;
  const int col0 = (blockIdx.x % chunks) * kCols;
  const int ncols = min(kCols, G - col0);
  const int split = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x, hl = lane >> 5, lq = lane & 31;
  const int L = min(max(lens[b], 0), max_seq_len);
  const int kbeg = window ? max(L - window, 0) : 0;
  const int nblk = (L + kBlock - 1) / kBlock;
  const int blk0 = kbeg / kBlock + split * split_blocks;
  if (blk0 >= nblk) return;  // beyond this sequence: the merge never reads it
  const int count = min(blk0 + split_blocks, nblk) - blk0;  // pages in this split (<= 64)
  const int n_tiles = (count + 1) / 2;
  const int tok0 = blk0 * kBlock;                       // first token of the split
  const int tok_end = min(L, tok0 + count * kBlock);    // past its last token
  const bool col_ok = lq < ncols;
  const int head = hk * G + col0 + lq;  // query head of this lane's column

  // Q^T operand: lane (column lq, half hl) holds dims 16 ks + 8 hl .. +7 of its head
  bf16x8 qop[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (col_ok) {
      qop[ks] = *reinterpret_cast<const bf16x8*>(q + ((size_t)b * H + head) * kD + 16 * ks + 8 * hl);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[ks][e] = (bf16)0.f;
    }
  }
  const int tbl = (lane < count) ? table[(size_t)b * max_blocks_per_seq + blk0 + lane] : 0;

  // direct fills: slice j (1 KiB) = tile rows 4j .. 4j+3; lane i -> row 4j + i/16, chunk slot
  // i%16 holding the logical chunk the swizzle puts there
  const size_t page_stride = (size_t)Hkv * kBlock * kD;  // elements between pool pages
  const size_t head_off = (size_t)hk * kBlock * kD;
  constexpr int kFillOps = 16;  // vector-memory instructions per fill

  floatx16 acc[4];  // O^T: lane holds d = 32 db + 8 (r/4) + 4 hl + r%4 of its column
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // l_run: this lane's half of the normaliser
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  const int g16 = lane >> 4, s16 = lane & 15;
  const int tr_row = 4 * (g16 >> 1) + (s16 >> 2);
  const int tr_col = 16 * (g16 & 1) + 4 * (s16 & 3);

  // one tile: tile t is in (Kt, Vt); tile t+2 is fetched into (Kf, Vf), the slot of t-1
  // The slots are addressed at an offset the optimiser cannot see (zero at run time): with
  // constant arguments it would substitute the constants into the ring function below
  // before inlining it, and the non-aliasing of its parameters would be lost.
  int hidden_zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
  lds_bf16* k0 = (lds_bf16*)(tiles[0] + hidden_zero);
  lds_bf16* k1 = (lds_bf16*)(tiles[1] + hidden_zero);
  lds_bf16* k2 = (lds_bf16*)(tiles[2] + hidden_zero);
  lds_bf16* v0 = (lds_bf16*)(tiles[3] + hidden_zero);
  lds_bf16* v1 = (lds_bf16*)(tiles[4] + hidden_zero);
  lds_bf16* v2 = (lds_bf16*)(tiles[5] + hidden_zero);
  // The whole ring runs inside one function whose slot pointers are declared non-aliasing:
  // the compiler then knows that a fill of one slot does not touch the slot being read and
  // leaves the wait for tile t to the explicit vmcnt below (it would otherwise drain every
  // outstanding fill before each LDS read).
  auto pipeline = [&](lds_bf16* __restrict__ k0, lds_bf16* __restrict__ k1,
                      lds_bf16* __restrict__ k2, lds_bf16* __restrict__ v0,
                      lds_bf16* __restrict__ v1, lds_bf16* __restrict__ v2) {
    auto fill = [&](int t, lds_bf16* Kd, lds_bf16* Vd) {
  #pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int p = 2 * t + jb;  // page within the split
        uint32_t bytes = 0;
        size_t base = 0;
        if (p < count) {
          const int phys = min(max(__builtin_amdgcn_readlane(tbl, p), 0), num_blocks - 1);
          base = (size_t)phys * page_stride + head_off;
          bytes = (uint32_t)min(L - (blk0 + p) * kBlock, kBlock) * kD * 2;  // ends at the length
        }
        const rsrc_t rk = make_rsrc(kc + base, bytes);
        const rsrc_t rv = make_rsrc(vc + base, bytes);
  #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * jb + i;
          const int r = 4 * j + (lane >> 4), pc = lane & 15, rr = r & 15;
          load_lds16_nt(rk, (lds_void*)&Kd[j * 512], (rr * kD + 8 * (pc ^ (r & 15))) * 2);
          load_lds16_nt(rv, (lds_void*)&Vd[j * 512], (rr * kD + 8 * (pc ^ ((r & 3) << 2))) * 2);
        }
      }
    };
    auto step = [&](int t, lds_bf16* Kt, lds_bf16* Vt, lds_bf16* Kf, lds_bf16* Vf) {
      if (t + 2 < n_tiles) fill(t + 2, Kf, Vf);
      // tile t has landed once at most the fills issued after it are outstanding
      if (t + 2 < n_tiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kFillOps));
      else if (t + 1 < n_tiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kFillOps));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const int t0 = tok0 + kTile * t;  // first token of the tile
      if (t0 < kbeg) {
        // tokens before the window: clear their V rows (at most 15, all in the first page)
        const int nz = kbeg - t0;
        for (int r = lane >> 4; r < nz; r += 4)
          *reinterpret_cast<lds_u32x4*>(&Vt[r * kD + 8 * (lane & 15)]) = u32x4_t{0u, 0u, 0u, 0u};
      }
      // ---- S^T = K Q^T: s[r] is the score of token t0 + 8 (r/4) + 4 hl + r%4
      floatx16 s;
  #pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
  #pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kop = *reinterpret_cast<const lds_bf16x8*>(&Kt[k_slot(lq, 2 * ks + hl)]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s, 0, 0, 0);
      }
      // ---- mask (end of the split or sequence, window start), online update
      // (one wave-uniform branch around the whole tile: a test per element compiles into a
      // branch per element)
      if ((t0 + kTile > tok_end) || (t0 < kbeg)) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = t0 + 8 * (r >> 2) + 4 * hl + (r & 3);
          s[r] = (tok < tok_end && tok >= kbeg) ? s[r] : -INFINITY;
        }
      }
      float mx = -INFINITY;
  #pragma unroll
      for (int r = 0; r < 16; ++r) mx = __builtin_fmaxf(mx, s[r]);
      mx = other_half_max(mx) * c_log2;
      // The reference m_run follows the running maximum lazily: it is raised (l and u
      // rescaled by 2^(old - new)) only when a score exceeds it by more than 2^8, so weights
      // stay <= 2^8 and the rescale is mostly skipped; on the first tile (l = u = 0) it is
      // just set.  Every tile holds an admitted token, so mx is finite.
      if (t == 0) {
        m_run = mx;
      } else if (__any(mx > m_run + 8.0f)) {
        const float m_new = __builtin_fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
  #pragma unroll
        for (int db = 0; db < 4; ++db)
  #pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
        m_run = m_new;
      }
      const float m_new = m_run;
      // ---- P^T operand (bf16) and the normaliser from the same rounded weights
      bf16x8 pop[2];
  #pragma unroll
      for (int g = 0; g < 2; ++g)
  #pragma unroll
        for (int e = 0; e < 8; e += 2) {
          floatx2 pp;
          pp[0] = __builtin_amdgcn_exp2f(fmaf(s[8 * g + e], c_log2, -m_new));
          pp[1] = __builtin_amdgcn_exp2f(fmaf(s[8 * g + e + 1], c_log2, -m_new));
          const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_run, false);
          pop[g][e] = pb[0];
          pop[g][e + 1] = pb[1];
        }
      // ---- O^T += V^T P^T, V^T read transposed from the row-major tile
  #pragma unroll
      for (int g = 0; g < 2; ++g)
  #pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int col = 32 * db + tr_col;
          const int r_lo = 16 * g + tr_row;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4*)(&Vt[v_slot(r_lo, col >> 3) + (col & 7)]));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_shortx4*)(&Vt[v_slot(r_lo + 8, col >> 3) + (col & 7)]));
          const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                     __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4,
                                                     5, 6, 7);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[g], acc[db], 0, 0, 0);
        }
    };

    fill(0, k0, v0);
    if (n_tiles > 1) fill(1, k1, v1);
    // two turns of the ring per iteration: the compiler's tracking of which slot a pending
    // fill targets does not survive the loop's back edge, so the first step of an iteration
    // still waits for all fills; two turns halve how often that happens
    for (int t = 0; t < n_tiles; t += 2 * kStages) {
      step(t, k0, v0, k2, v2);
      if (t + 1 < n_tiles) step(t + 1, k1, v1, k0, v0);
      if (t + 2 < n_tiles) step(t + 2, k2, v2, k1, v1);
      if (t + 3 < n_tiles) step(t + 3, k0, v0, k2, v2);
      if (t + 4 < n_tiles) step(t + 4, k1, v1, k0, v0);
      if (t + 5 < n_tiles) step(t + 5, k2, v2, k1, v1);
    }
  };
  pipeline(k0, k1, k2, v0, v1, v2);

  // ---- partial summary of this split for each served head
  const float l_tot = other_half_sum(l_run);
  if (!col_ok) return;
  const Partials P{reinterpret_cast<float*>(ws), reinterpret_cast<float*>(ws) + n_part,
                   reinterpret_cast<float*>(ws) + 2 * n_part};
  const size_t p = ((size_t)b * H + head) * max_splits + split;
  float* u = P.u + p * kD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      floatx4 x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = acc[db][4 * a + c];
      *reinterpret_cast<floatx4*>(u + 32 * db + 8 * a + 4 * hl) = x;
    }
  if (hl == 0) {
    P.m[p] = m_run;
    P.l[p] = l_tot;
  }
}

}  // namespace

hipError_t launch_decode_gqa(const bf16* q, const bf16* k_cache, const bf16* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, int batch,
                             int heads, int kv_heads, int num_blocks, int max_blocks_per_seq,
                             int max_seq_len, int window, float scale, int split, int max_splits,
                             void* workspace, size_t n_part, hipStream_t stream) {
  const int G = heads / kv_heads;
  const int chunks = (G + kCols - 1) / kCols;
  hipLaunchKernelGGL(decode_gqa_kernel, dim3((unsigned)(kv_heads * chunks), (unsigned)max_splits,
                                             (unsigned)batch),
                     dim3(64), 0, stream, q, k_cache, v_cache, block_table, seq_lens, workspace,
                     heads, kv_heads, num_blocks, max_blocks_per_seq, max_seq_len, window,
                     max_splits, split / kBlock, scale * ATTN_LOG2E, n_part);
  return hipGetLastError();
}
