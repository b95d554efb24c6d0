// FP8 (E4M3) prefill attention on gfx950 matrix cores, head_dim 128, bf16 output.
//
// The FP8 variant of pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (its part on FP8 in
// FlashAttention-3, sections "Quantizzazione a Blocchi e Scaling Algebrico" and
// "Integrazione nel ciclo Online Softmax"): Q, K, V arrive as E4M3 codes with one fp32 scale per 64-row block
// (s = max|X| / 448, produced by quantize_fp8_kernel); the score block is
// (scale s_Q s_K) (Q8 K8^T), the factor applied once in fp32 to the fp32 accumulator; the
// maximum, S - m and exp(S - m) are fp32; the weights are rounded to E4M3 (v_cvt_pk_fp8_f32)
// before the P.V product, accumulated in fp32, and l sums those rounded weights; V's block
// scale multiplies its tile's P.V product; one division by l at the end, cast to bf16.
// The running maximum moves once per 64-key tile, exactly, since the E4M3 rounding of P
// depends on it (no lazily raised reference as in the bf16 kernel).
//
// Mapping onto CDNA4 (v_mfma_f32_32x32x64_f8f6f4, E4M3 x E4M3 -> fp32):
//   * workgroup = 4 waves = 128 queries of one (batch, head); wave = 32 queries.
//   * S^T = K Q^T: a lane (query lq, half hl) holds 32 of its query's 64 tile scores.  The K
//     rows are placed in LDS in an order that makes those 32 keys two runs of 16 consecutive
//     keys (32 kb + 16 hl + 0..15), so the rounded weights form the B operand of the P.V
//     product straight from the score registers, and the matching A operand (V^T) is two
//     16-byte reads of a transposed V tile (V is stored [128][n_pad] per (batch, head)).
//   * l = the row sum of the rounded weights, computed by one more MFMA against a block of
//     ones (exact: E4M3 values summed in fp32).
//   * K tile 64 x 128 B and V^T tile 128 x 64 B (8 KiB each) double-buffered in LDS, filled
//     by direct global->LDS loads with XOR-swizzled 16-byte chunks (conflict-free reads).
#include "common.h"

namespace {

constexpr int kD = 128;
constexpr int kBM = 128;    // queries per workgroup
constexpr int kBN = 64;     // keys per tile (= the quantisation block)
constexpr int kThreads = 256;
constexpr int kTileBytes = kBN * kD;  // 8 KiB, for K and for V^T
constexpr float kSlack = 8.0f;        // log2 headroom of the accumulation reference

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint4 lds_uint4;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// LDS byte offset of 16-byte chunk c (0..7) of K-tile row R (128 B per row)
__device__ __forceinline__ int k_off(int R, int c) { return R * 128 + ((c ^ (R & 7)) << 4); }
// LDS byte offset of 16-byte chunk c (0..3) of V^T-tile row D (64 B per row; two rows per
// 128-byte line, chunk slots XORed with the line index so 8 consecutive rows hit 8 slots)
__device__ __forceinline__ int v_off(int D, int c) {
  return (D >> 1) * 128 + (D & 1) * 64 + ((c ^ ((D >> 1) & 3)) << 4);
}
// key held by LDS row R of a K tile: rows are permuted inside each 32-row group so that MFMA
// row 8a + 4h + b (a, b < 4, h < 2) carries key 16h + 4a + b
__device__ __forceinline__ int k_row_key(int R) {
  const int i = R & 31;
  return (R & 32) + 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

__device__ __forceinline__ intx8 read32(const uint8_t* base, int off0, int off1) {
  const uint4 a = *reinterpret_cast<const uint4*>(base + off0);
  const uint4 b = *reinterpret_cast<const uint4*>(base + off1);
  return intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__global__ __launch_bounds__(kThreads, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8, const uint8_t* __restrict__ VT8,
    const float* __restrict__ q_scale, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, bf16* __restrict__ O, float* __restrict__ LSE,
    const int32_t* __restrict__ lens, int B, int H, int Hkv, int n, int n_qtiles, int n_blocks,
    int causal, float scale) {
  // K tiles in slots 0 and 1, V^T tiles in slots 2 and 3 (one LDS object: the compiler then
  // keeps the non-aliasing of the four slots declared below)
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[4][kTileBytes];

  const int HB = H * B;
  const GridSlot slot = causal_grid_slot((int)blockIdx.x, HB, n_qtiles);  // heaviest first
  const int qt = n_qtiles - 1 - slot.rank;
  const int bh = slot.bh;
  const int b = bh / H;
  const int bhk = b * Hkv + (bh % H) / (H / Hkv);
  int L = lens ? lens[b] : n;
  L = L < 0 ? 0 : (L > n ? n : L);
  const int m0 = qt * kBM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5, lq = lane & 31;
  const int qi = m0 + 32 * w + lq;
  const size_t o_base = (size_t)bh * n * kD;

  if (m0 >= L) {  // the whole tile is padding: o = 0, lse = -inf
    for (int i = tid; i < kBM * kD / 8; i += kThreads) {
      const int r = m0 + (i * 8) / kD;
      if (r < n) {
        bf16x8 z;
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = (bf16)0.f;
        *reinterpret_cast<bf16x8*>(O + o_base + (size_t)r * kD + (i * 8) % kD) = z;
      }
    }
    if (LSE)
      for (int r = m0 + tid; r < min(m0 + kBM, n); r += kThreads) LSE[(size_t)bh * n + r] = -INFINITY;
    return;
  }

  const size_t n_pad = (size_t)n_blocks * kBN;
  const rsrc_t rq = make_rsrc(Q8 + (size_t)bh * n * kD, (uint32_t)L * kD);

  // Q^T operand: lane (query lq, half hl) holds dims 64 ks + 32 hl .. +31 for ks = 0, 1
  intx8 qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const uint4 a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qi * kD + 64 * ks + 32 * hl, 0, 0));
    const uint4 c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, qi * kD + 64 * ks + 32 * hl + 16, 0, 0));
    qop[ks] = intx8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)c.x, (int)c.y, (int)c.z, (int)c.w};
  }
  // the wave's 32 queries lie in one 64-row quantisation block (clamped: a wave whose
  // queries are all past n reads the last block's scale and writes nothing)
  const float sq = q_scale[(size_t)bh * n_blocks + min((m0 + 32 * w) / kBN, n_blocks - 1)];
  const float c_q = scale * sq * ATTN_LOG2E;
  const float* ks_row = k_scale + (size_t)bhk * n_blocks;
  const float* vs_row = v_scale + (size_t)bhk * n_blocks;

  const int kend = causal ? min(L, m0 + kBM) : L;
  const int n_tiles = (kend + kBN - 1) / kBN;
  const int wave_q_first = m0 + 32 * w, wave_q_last = wave_q_first + 31;
  const int wave_tiles = causal ? min(n_tiles, wave_q_last / kBN + 1) : n_tiles;

  // direct global->LDS fills: wave w writes 1 KiB slices 2w, 2w+1 of each tile
  int k_src[2], v_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int sl = 2 * w + i, p = lane & 7;
    const int R = 8 * sl + (lane >> 3);                        // K: LDS row, chunk slot p
    k_src[i] = k_row_key(R) * kD + 16 * (p ^ (R & 7));
    const int ln = 8 * sl + (lane >> 3);                       // V^T: 128-byte line, slot p
    const int D = 2 * ln + (p >> 2);
    v_src[i] = D * (int)n_pad + 16 * ((p & 3) ^ (ln & 3));
  }
  // Each tile is read through a descriptor whose base is the tile's first key (K: row
  // t * 64; V^T: column t * 64), with the range ending at row L (K) or at the matrix end
  // (V^T, whose padding columns are zeros), and each wave's 2 KiB slice of a tile sits at a
  // scalar LDS offset: a fill costs no vector instruction.
  const uint8_t* k_head = K8 + (size_t)bhk * n * kD;
  const uint8_t* v_head = VT8 + (size_t)bhk * kD * n_pad;
  const int lds_w = __builtin_amdgcn_readfirstlane(w * 2 * 1024);
  auto issue_k = [&](int t, uint8_t* Kd) __attribute__((always_inline)) {
    const int first = t * kBN;
    const rsrc_t r = make_rsrc(k_head + (size_t)first * kD, (uint32_t)max(L - first, 0) * kD);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      load_lds16(r, (lds_void*)((lds_char*)(lds_void*)Kd + lds_w + i * 1024), k_src[i]);
  };
  auto issue_v = [&](int t, uint8_t* Vd) __attribute__((always_inline)) {
    const int first = t * kBN;
    const rsrc_t r = make_rsrc(v_head + first, (uint32_t)(kD * n_pad - first));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      load_lds16(r, (lds_void*)((lds_char*)(lds_void*)Vd + lds_w + i * 1024), v_src[i]);
  };

  floatx16 acc[4];  // O^T: lane holds d = 32 db + 8 (r/4) + 4 hl + r%4 of query qi
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // m_cur: the exact running maximum (log2 units) through the last scored tile — the weights
  // of a tile are taken against it.  m_ref: the reference acc and l_acc are kept in; it
  // follows m_cur lazily (raised when m_cur exceeds it by more than kSlack), so a tile's
  // contribution enters with the factor 2^(m_cur - m_ref) and the rescale of acc is rare.
  float m_cur = -INFINITY, m_ref = -INFINITY, l_acc = 0.f;
  const intx8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  const floatx16 zero16 = {};

  struct Tile {
    floatx16 s[2];  // raw scores: s[kb][r] is key k0 + 32 kb + 16 hl + r (masked: -inf)
  };
  auto compute_s = [&](Tile& T, const uint8_t* Kt) __attribute__((always_inline)) {  // S^T = K Q^T, 4 MFMA
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) T.s[kb] = zero16;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int R = 32 * kb + lq, c0 = 4 * ks + 2 * hl;
        const intx8 a = read32(Kt, k_off(R, c0), k_off(R, c0 + 1));
        T.s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qop[ks], T.s[kb], 0, 0, 0, 0, 0, 0);
      }
  };
  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int k0 = t * kBN;
    return (k0 + kBN > L) || (causal && k0 + kBN - 1 > wave_q_first);
  };
  auto apply_mask = [&](Tile& T, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * kb + 16 * hl + r;
        T.s[kb][r] = (key < L && (!causal || key <= qi)) ? T.s[kb][r] : -INFINITY;
      }
  };
  // tile maximum in log2 units; c > 0, so max(raw) * c is the max of the rounded products
  auto row_max = [&](const Tile& T, float c) __attribute__((always_inline)) {
    float mx = __builtin_fmaxf(T.s[0][0], T.s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, T.s[0][r]), T.s[0][r + 1]);
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, T.s[1][r]), T.s[1][r + 1]);
    return other_half_max(mx) * c;
  };
  auto weights = [&](const Tile& T, float c, float m_use, intx8& pop) __attribute__((always_inline)) {  // byte e = 16 kb + r
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      const int kb = wd >> 2, r0 = 4 * (wd & 3);
      const float p0 = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0], c, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0 + 1], c, -m_use));
      const float p2 = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0 + 2], c, -m_use));
      const float p3 = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0 + 3], c, -m_use));
      const int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
      pop[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
    }
  };
  auto raise_ref = [&]() __attribute__((always_inline)) {
    if (__any(m_cur > m_ref + kSlack)) {
      const float m_new = __builtin_fmaxf(__builtin_fmaxf(m_ref, m_cur), -1e30f);
      const float alpha = __builtin_amdgcn_exp2f(__builtin_fmaxf(m_ref, -1e30f) - m_new);  // 0 from empty
      m_ref = m_new;
      l_acc *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
  };

  // One pipelined step: the weights of tile t (in `cur`) are formed while the matrix cores
  // compute the scores of tile t+1 (into `nxt`); then P(t) V(t) runs while the maximum of
  // tile t+1 is taken and the previous products enter acc.  K loads run two tiles ahead,
  // V loads one.  Every wave runs these steps up to the workgroup's last tile, so the step
  // is straight-line code; a wave whose diagonal lies before the last tile scores that tile
  // needlessly (its maximum then moves m_cur past any use: the last step skips the wave).
  // Block scales of K (tiles t and t+1) and V (tile t), read one step ahead: a scalar load
  // inside the step would make the wave wait for every LDS read in flight as well.
  float ks_cur = 0.f, ks_nxt = 0.f, vs_cur = 0.f;
  const int t_last = n_tiles - 1;
  auto pv_update = [&](const intx8& pop, const uint8_t* Vt, float fv, auto&& between)
      __attribute__((always_inline)) {
    // P.V in two halves of 64 dimensions (keeps 32 product registers live), the row sum of
    // the rounded weights, and `between` (the next tile's mask and maximum) in between
    floatx16 lsum;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      floatx16 tmp[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int D = 64 * half + 32 * i + lq;
        const intx8 a = read32(Vt, v_off(D, hl), v_off(D, 2 + hl));
        tmp[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pop, zero16, 0, 0, 0, 0, 0, 0);
      }
      if (half == 0) {
        lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pop, zero16, 0, 0, 0, 0, 0, 0);
        between();
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[2 * half + i][r] = fmaf(tmp[i][r], fv, acc[2 * half + i][r]);
    }
    return lsum[0];
  };
  auto step = [&](int t, Tile& cur, Tile& nxt, uint8_t* Kf, uint8_t* Vf, const uint8_t* Kr,
                  const uint8_t* Vr) __attribute__((always_inline)) {
    if (t + 2 < n_tiles) issue_k(t + 2, Kf);
    issue_v(t + 1, Vf);
    raise_ref();
    const float m_use = __builtin_fmaxf(m_cur, -1e30f);
    const float f = __builtin_amdgcn_exp2f(m_use - __builtin_fmaxf(m_ref, -1e30f));
    intx8 pop;
    compute_s(nxt, Kr);
    weights(cur, c_q * ks_cur, m_use, pop);
    const float lsum = pv_update(pop, Vr, f * vs_cur, [&]() __attribute__((always_inline)) {
      // tile t+1 is used unless it is the last tile and lies past this wave's diagonal
      if ((t + 1 < wave_tiles || t + 1 < t_last) && need_mask(t + 1)) apply_mask(nxt, (t + 1) * kBN);
      m_cur = __builtin_fmaxf(m_cur, row_max(nxt, c_q * ks_nxt));
    });
    l_acc = fmaf(lsum, f, l_acc);
    ks_cur = ks_nxt;
    ks_nxt = ks_row[min(t + 2, n_blocks - 1)];
    vs_cur = vs_row[min(t + 1, n_blocks - 1)];
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of the next tiles (and scales) landed
    __syncthreads();
  };
  // the last tile: the rest of its work, no loads, no barrier
  auto step_last = [&](int t, Tile& cur, const uint8_t* Vr) __attribute__((always_inline)) {
    if (t < wave_tiles) {
      raise_ref();
      const float m_use = __builtin_fmaxf(m_cur, -1e30f);
      const float f = __builtin_amdgcn_exp2f(m_use - __builtin_fmaxf(m_ref, -1e30f));
      intx8 pop;
      weights(cur, c_q * ks_cur, m_use, pop);
      const float lsum = pv_update(pop, Vr, f * vs_cur, []() {});
      l_acc = fmaf(lsum, f, l_acc);
    }
  };

  // The sweep runs inside one function whose four tile slots are declared non-aliasing: the
  // compiler then knows that the fills a step issues do not touch the tiles it reads, and
  // leaves the wait for them to the step's closing waitcnt (it would otherwise wait for the
  // fills just issued before the first LDS read after them).  Tile t lives in slot t & 1.
  auto sweep = [&](uint8_t* __restrict__ k0, uint8_t* __restrict__ k1, uint8_t* __restrict__ v0,
                   uint8_t* __restrict__ v1) {
    // ---- prologue: K(0), V(0), K(1) in flight; scores and maximum of tile 0
    issue_k(0, k0);
    issue_v(0, v0);
    if (n_tiles > 1) issue_k(1, k1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    Tile ta, tb;
    compute_s(ta, k0);
    if (need_mask(0)) apply_mask(ta, 0);
    m_cur = row_max(ta, c_q * ks_row[0]);
    ks_cur = ks_row[0];
    ks_nxt = ks_row[min(1, n_blocks - 1)];
    vs_cur = vs_row[0];
    __syncthreads();  // every wave is done with K(0) before K(2) overwrites its buffer

    for (int t = 0; t < t_last; t += 2) {
      step(t, ta, tb, k0, v1, k1, v0);
      if (t + 1 < t_last) step(t + 1, tb, ta, k1, v0, k0, v1);
    }
    if ((t_last & 1) == 0)
      step_last(t_last, ta, v0);
    else
      step_last(t_last, tb, v1);
  };
  // The slots are passed at an offset the optimiser cannot see (zero at run time): with
  // constant arguments it would substitute the constants into the body before inlining it,
  // and the non-aliasing of the parameters would be lost.
  int hidden_zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
  sweep(tiles[0] + hidden_zero, tiles[1] + hidden_zero, tiles[2] + hidden_zero, tiles[3] + hidden_zero);

  // ---- epilogue: o = u / l (l is the whole row's sum: every lane of the MFMA column has it),
  // staged through LDS so that each store writes four whole 256-byte rows of O: once every
  // wave is past its last tile the four slots (32 KiB) are free, and wave w takes 32 rows,
  // the 16-byte chunks of row r XOR-swizzled by r % 16.
  __syncthreads();
  const bool valid = qi < L;
  const float inv = 1.0f / l_acc;
  bf16* stage = reinterpret_cast<bf16*>(&tiles[0][0]) + w * (32 * kD);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      floatx4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = valid ? acc[db][4 * a + e] * inv : 0.f;
      const int chunk = (4 * db + a) ^ (lq & 15);
      *reinterpret_cast<bf16x4*>(stage + lq * kD + 8 * chunk + 4 * hl) = __builtin_convertvector(x, bf16x4);
    }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 4 * j + lane / 16, c = lane % 16;
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(stage + r * kD + 8 * (c ^ (r & 15)));
    const int row = m0 + 32 * w + r;
    // written once and never read here: streamed past the caches, which keep K and V
    if (row < n) __builtin_nontemporal_store(y, reinterpret_cast<bf16x8*>(O + o_base + (size_t)row * kD + 8 * c));
  }
  if (LSE && hl == 0 && qi < n)
    LSE[(size_t)bh * n + qi] = valid ? (m_ref * ATTN_LN2 + __logf(l_acc)) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8,
                          const float* q_scale, const float* k_scale, const float* v_scale,
                          bf16* o, float* lse, const int32_t* seq_lens, int batch, int heads,
                          int kv_heads, int n, int causal, float scale, hipStream_t stream) {
  const int n_qtiles = (n + kBM - 1) / kBM;
  const int n_blocks = (n + kBN - 1) / kBN;
  hipLaunchKernelGGL(fwd_fp8_kernel, dim3((unsigned)n_qtiles * batch * heads), dim3(kThreads), 0,
                     stream, q8, k8, vt8, q_scale, k_scale, v_scale, o, lse, seq_lens, batch, heads,
                     kv_heads, n, n_qtiles, n_blocks, causal, scale);
  return hipGetLastError();
}
