// bf16 prefill attention on gfx950 matrix cores, head_dim 128 (and 64).
//
// Method: the score matrix is produced and consumed one 64-key tile at a time with the
// running (m, l, u) summary of el-ai.com "Attenzione: softmax online, riscalamento e
// memoria", section 2 (new maximum m' = max(m, rowmax); l and u both multiplied by
// 2^(m - m'); then the tile's weights and weighted values added), and u is divided by l
// once at the end (the deferred normalisation pierluigilucio.it "Sviluppo AI ed Algebra
// Lineare" credits to FlashAttention-2).  Scores never leave registers.
//
// Mapping onto CDNA4:
//   * workgroup = 4 waves = 128 queries of one (batch, head); each wave owns 32 queries.
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the
//     query is the MFMA column (lane % 32), so a lane holds 32 of one query's 64 tile
//     scores and the other 32 sit in lane ^ 32.  Row max = in-lane max + one cross-half
//     exchange; the normaliser stays a per-lane partial until the epilogue.
//   * the output is accumulated transposed too, O^T += V^T P^T: its column is again the
//     query, so the rescale factor of a query multiplies that lane's registers only.  The
//     bf16 weights P^T feed the MFMA B operand straight from the score registers; V^T is
//     read from a row-major V tile with ds_read_b64_tr_b16, whose 16-lane transpose hands
//     each lane 4 consecutive keys of one dimension.
//   * K/V tiles (64 x 128 bf16 = 16 KiB each; 8 KiB at head_dim 64) are double-buffered in
//     LDS and filled by 16-byte-per-lane buffer loads that write LDS directly (no register
//     staging), each lane fetching the chunk an XOR swizzle puts in its slot; the swizzle
//     keeps the K row reads and the transposed V reads free of bank conflicts (at head_dim
//     64 the transposed reads keep a 2-way conflict).  K runs two tiles ahead of its use, V
//     one.  One barrier per tile.
//   * the output tile is staged through the then idle K buffers so that every store writes
//     whole rows (four of 256 bytes; eight of 128 at head_dim 64).
//   * exp is v_exp_f32 (2^x): scores are scaled by scale*log2(e) inside one FMA.
//   * the normaliser sums the bf16-ROUNDED weights that enter the P.V product (dot2 with
//     ones), so rounding of P cancels in u/l to first order.
//   * causal: the key loop ends at the workgroup's diagonal; a wave whose own diagonal lies
//     a tile earlier scores that last tile along with the others but skips its weights and
//     P.V (one straight-line step for all waves keeps the loop free of per-wave branches,
//     and the compiler interleaves the weights' FMAs and exps with the score products).
//     Every query tile of one (batch, head) lands on the same XCD, eight heads at a time,
//     heaviest tiles first (causal_grid_slot), so K/V are re-read from that XCD's L2.
//     Consecutive heads share an XCD, so the query heads of one K/V group (grouped heads)
//     read their shared K/V from one L2 as well.
//   * causal window w: the key loop starts at the first tile any query of the workgroup
//     admits (query i admits keys i - w < j <= i); tiles that cross a window edge are
//     masked like the diagonal ones.
#include "common.h"

namespace {

constexpr int kBM = 128;     // queries per workgroup
constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kSlack = 8.0f;  // log2 headroom of the lazily raised reference maximum

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) char lds_char;

// Tile swizzles, per head dim D (rows of D bf16, 16-byte chunks c = 0 .. D/8 - 1).
// D = 128 (256-byte rows, one row spans all LDS banks): a K row's chunk index is XORed with
// r % 16, so the 16 rows one MFMA operand read touches hit 16 distinct chunk slots; in a V
// tile, chunk groups of 64 bytes are XORed with r % 4, so the 8 rows one transposed read
// touches spread over all four 64-byte bank groups.
// D = 64 (128-byte rows, even and odd rows in the two halves of the banks): K chunks are
// XORed with (r / 2) % 8, which again separates 16 consecutive rows; V chunk groups with
// (r / 2) % 2, which halves the conflicts of a transposed read (two 64-byte groups per row).
template <int D>
__device__ __forceinline__ int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }
template <int D>
__device__ __forceinline__ int k_slot(int r, int c) { return r * D + ((c ^ k_swz<D>(r)) << 3); }
template <int D>
__device__ __forceinline__ int v_slot(int r, int c) { return r * D + ((c ^ v_swz<D>(r)) << 3); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}

// value of lane l ^ 32 (v_permlane32_swap exchanges the two wave halves)
__device__ __forceinline__ float other_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float other_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt immediate (gfx9 encoding): vector-memory count <= n, the other counts unconstrained
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;

struct Tile {
  floatx16 s[2];  // S^T of 64 keys: lane holds key 32 kb + 8 (r/4) + 4 hl + r%4 of query lq
};

// kWindow: a causal window is in force (`window` > 0); without it the window terms compile
// away and the register budget of the plain kernel is untouched.  kD: the head dim, 128 or
// 64 (half the Q operand, accumulator, tile and products per step; the same steps).
template <bool kWindow, int kD>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const int32_t* __restrict__ lens, int B,
    int H, int Hkv, int n, int n_kv, int q_start, int n_qtiles, int causal, int window,
    float c_log2) {
  // Q, O, LSE hold n query rows; K, V hold n_kv key rows.  Query row r sits at position
  // q_start + r of the key sequence (the causal mask and the window count positions); the
  // plain call has n_kv = n and q_start = 0.  Lengths (lens) apply to plain calls only.
  constexpr int kTileElems = kBN * kD;
  constexpr int kChunks = kD / 8;        // 16-byte chunks per row
  constexpr int kKSteps = kD / 16;       // k-steps of a score product (Q^T operand registers)
  constexpr int kDBlocks = kD / 32;      // 32-wide output blocks (accumulators)
  constexpr int kSlices = kD / 32;       // 1 KiB slices of a tile each wave fills
  constexpr int kSliceRows = 512 / kD;   // tile rows per 1 KiB slice
  // K tiles in slots 0 and 1, V tiles in slots 2 and 3 (one LDS object: the compiler then
  // keeps the non-aliasing of the four slots declared below)
  __shared__ __attribute__((aligned(1024))) bf16 tiles[4][kTileElems];

  const int HB = H * B;
  int qt, bh;
  if constexpr (kWindow) {  // windows: every full tile has the same work; original order
    qt = n_qtiles - 1 - (int)(blockIdx.x / HB);
    const int j = blockIdx.x % HB;
    bh = (HB % 8 == 0) ? (j % 8) * (HB / 8) + j / 8 : j;
  } else {
    const GridSlot slot = causal_grid_slot((int)blockIdx.x, HB, n_qtiles);
    qt = n_qtiles - 1 - slot.rank;  // the last query tile has the most causal work
    bh = slot.bh;
  }
  const int b = bh / H;
  int L = lens ? lens[b] : n_kv;  // keys (and, in plain calls, queries) past L are padding
  L = L < 0 ? 0 : (L > n_kv ? n_kv : L);
  const size_t base = (size_t)bh * n * kD;
  const size_t kv_base = ((size_t)b * Hkv + (bh % H) / (H / Hkv)) * n_kv * kD;
  const int m0 = qt * kBM;      // first query row of the tile
  const int p0 = q_start + m0;  // its position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int hl = lane >> 5;    // which half of the wave
  const int lq = lane & 31;    // query column within the wave's 32
  const int qi = p0 + w * 32 + lq;  // this lane's query position

  if (p0 >= L) {  // the whole tile is padding: o = 0, lse = -inf
    for (int i = tid; i < kBM * kD / 8; i += kThreads) {
      const int r = m0 + (i * 8) / kD;
      if (r < n) *reinterpret_cast<bf16x8*>(O + base + (size_t)r * kD + (i * 8) % kD) = zero8();
    }
    if (LSE)
      for (int r = m0 + tid; r < min(m0 + kBM, n); r += kThreads) LSE[(size_t)bh * n + r] = -INFINITY;
    return;
  }

  // rows >= L read as zeros through the descriptors' range
  const rsrc_t rq = make_rsrc(Q + base, (uint32_t)(min(L - q_start, n)) * kD * 2);

  // Q^T operand: lane (query lq, half hl) holds dims 16*ks + 8*hl .. +7 for ks < kD/16.
  bf16x8 qop[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks)
    qop[ks] = load_b128(rq, ((qi - q_start) * kD + 16 * ks + 8 * hl) * 2);

  const int kend = causal ? min(L, p0 + kBM) : L;
  const int n_tiles = (kend + kBN - 1) / kBN;                 // tiles [t_first, n_tiles)
  const int t_first = kWindow ? max(0, p0 - window + 1) / kBN : 0;
  const int wave_q_first = p0 + w * 32;
  const int wave_q_last = wave_q_first + 31;
  // tiles a wave takes part in (causal: none strictly above its diagonal)
  const int wave_tiles = causal ? min(n_tiles, wave_q_last / kBN + 1) : n_tiles;

  // Direct global->LDS tile fill: wave w fills 1 KiB slices kSlices*w .. +kSlices-1 of each
  // tile; lane i of slice j lands in row kSliceRows*j + i/kChunks, physical chunk
  // i%kChunks, so it fetches the logical chunk the swizzle puts there.  Each tile is read
  // through a descriptor whose base is the tile's first row and whose range ends at row L,
  // so the per-lane offsets are loop invariants and rows past L still read as zeros.
  int k_src[kSlices], v_src[kSlices];
#pragma unroll
  for (int i = 0; i < kSlices; ++i) {
    const int r = kSliceRows * (kSlices * w + i) + lane / kChunks;
    const int pc = lane % kChunks;
    k_src[i] = (r * kD + 8 * (pc ^ k_swz<kD>(r))) * 2;
    v_src[i] = (r * kD + 8 * (pc ^ v_swz<kD>(r))) * 2;
  }
  const bf16* k_head = K + kv_base;
  const bf16* v_head = V + kv_base;
  auto tile_rsrc = [&](const bf16* head, int t) __attribute__((always_inline)) {
    const int first = t * kBN;
    return make_rsrc(head + (size_t)first * kD, (uint32_t)max(L - first, 0) * kD * 2);
  };
  // this wave's slices of a tile, as a wave-uniform (scalar) LDS byte offset
  const int lds_w = __builtin_amdgcn_readfirstlane(w * kSlices * 1024);
  auto lds_dst = [&](bf16* tile, int i) __attribute__((always_inline)) {
    return (lds_void*)((lds_char*)(lds_void*)tile + lds_w + i * 1024);
  };
  auto issue_k = [&](int t, bf16* Kd) __attribute__((always_inline)) {
    const rsrc_t r = tile_rsrc(k_head, t);
#pragma unroll
    for (int i = 0; i < kSlices; ++i) load_lds16(r, lds_dst(Kd, i), k_src[i]);
  };
  auto issue_v = [&](int t, bf16* Vd) __attribute__((always_inline)) {
    const rsrc_t r = tile_rsrc(v_head, t);
#pragma unroll
    for (int i = 0; i < kSlices; ++i) load_lds16(r, lds_dst(Vd, i), v_src[i]);
  };

  floatx16 acc[kDBlocks];  // O^T, d blocks of 32: lane holds d = 32*db + 8*(r/4) + 4*hl + r%4
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  // Reference maximum (log2 units) the weights are taken against.  It follows the running
  // maximum lazily: it is raised (and l, u rescaled by 2^(old - new)) only when some score
  // of the wave exceeds it by more than kSlack, so weights stay <= 2^kSlack and the
  // rescale — exact in real arithmetic whichever reference is used — is mostly skipped.
  // Whether a tile needs a raise is read off the weights' own row sum: a lane whose sum is
  // at most 2^kSlack has no weight above it, so only a larger (or infinite) sum leads to
  // the tile's exact row maximum, the reference raised to it and a second evaluation of
  // the weights.  No row maximum is taken on the common path.
  float m_ref = -INFINITY;
  float m_use = -1e30f;  // m_ref floored: no -inf - (-inf) on rows with no key yet
  float l_run = 0.f;     // this lane's half of the normaliser
  constexpr float kSumLimit = 256.0f;  // 2^kSlack

  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  // transposed-read addressing for V^T (see header): 16-lane group g, source lane s
  const int g = lane >> 4, s = lane & 15;
  const int tr_row = 4 * (g >> 1) + (s >> 2);              // + 16*grp + 8*read
  const int tr_col = 16 * (g & 1) + 4 * (s & 3);           // + 32*db

  // ---- building blocks ----------------------------------------------------------------
  auto compute_s = [&](Tile& T, const bf16* Kt) __attribute__((always_inline)) {  // S^T = K Q^T: kD/8 MFMA, as many LDS reads
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) T.s[kb][r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&Kt[k_slot<kD>(32 * kb + lq, 2 * ks + hl)]);
        T.s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], T.s[kb], 0, 0, 0);
      }
  };
  auto apply_mask = [&](Tile& T, int k0) __attribute__((always_inline)) {  // key of (kb, r) is k0 + 32 kb + 8 (r/4) + 4 hl + r%4
    if constexpr (kWindow) {
      // with a window (always causal) the key is admitted iff key < L and 0 <= qi - key <
      // window: one unsigned compare plus the length test; o = key - k0 - 4 hl
      const unsigned base = (unsigned)(qi - k0 - 4 * hl);
      const int o_lim = L - k0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool ok = base - (unsigned)o < (unsigned)window && o < o_lim;
          T.s[kb][r] = ok ? T.s[kb][r] : -INFINITY;
        }
    } else {
      // admitted iff key < min(L, qi + 1) (causal) or key < L: one compare per score
      const int lim = (causal ? min(L, qi + 1) : L) - k0 - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
          T.s[kb][r] = o < lim ? T.s[kb][r] : -INFINITY;
        }
    }
  };
  auto need_mask = [&](int t) __attribute__((always_inline)) {  // wave-uniform
    const int k0 = t * kBN;
    return (k0 + kBN > L) || (causal && k0 + kBN - 1 > wave_q_first) ||
           (kWindow && k0 <= wave_q_last - window);
  };
  auto row_max = [&](const Tile& T) __attribute__((always_inline)) {  // scaled (log2 units) max over this tile's 64 keys
    float mx = __builtin_fmaxf(T.s[0][0], T.s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, T.s[0][r]), T.s[0][r + 1]);
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = __builtin_fmaxf(__builtin_fmaxf(mx, T.s[1][r]), T.s[1][r + 1]);
    return other_half_max(mx) * c_log2;
  };
  auto raise_ref = [&](float mx) __attribute__((always_inline)) {  // the lazy rescale of l and u
    if (__any(mx > m_ref + kSlack)) {
      // floor at -1e30: a lane with no admitted key yet gets alpha = 0, never NaN
      const float m_new = __builtin_fmaxf(__builtin_fmaxf(m_ref, mx), -1e30f);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 from the empty state
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    m_use = __builtin_fmaxf(m_ref, -1e30f);
  };
  auto weights = [&](const Tile& T, bf16x8 (&pop)[4]) __attribute__((always_inline)) {  // P^T operand, returns its row sum
    float psum = 0.f;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int kb = grp >> 1, r0 = 8 * (grp & 1);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        floatx2 pp;
        pp[0] = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0 + e], c_log2, -m_use));
        pp[1] = __builtin_amdgcn_exp2f(fmaf(T.s[kb][r0 + e + 1], c_log2, -m_use));
        const bf16x2 pb = __builtin_convertvector(pp, bf16x2);
        psum = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, psum, false);
        pop[grp][e] = pb[0];
        pop[grp][e + 1] = pb[1];
      }
    }
    return psum;
  };
  // The raise check on the weights of tile T (see m_ref): the common case costs one compare.
  // A lane whose row sum exceeds 2^kSlack (or is infinite) sends the wave to the exact row
  // maximum; the reference rises to it (alpha = 1 on lanes it does not move) and the
  // weights are evaluated again, now each at most 1.
  auto checked_weights = [&](const Tile& T, bf16x8 (&pop)[4], float psum) __attribute__((always_inline)) {
    if (__builtin_expect(__any(!(psum <= kSumLimit) && psum == psum), 0)) {
      const float m_new = __builtin_fmaxf(__builtin_fmaxf(m_ref, row_max(T)), -1e30f);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 from the empty state
      m_ref = m_new;
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      psum = weights(T, pop);
    }
    l_run += psum;
  };
  auto pv = [&](const bf16* Vt, const bf16x8 (&pop)[4]) __attribute__((always_inline)) {  // O^T += V^T P^T
#pragma unroll
    for (int grp = 0; grp < 4; ++grp)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const int col = 32 * db + tr_col;
        const int r_lo = 16 * grp + tr_row;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(&Vt[v_slot<kD>(r_lo, col >> 3) + (col & 7)]));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_shortx4*)(&Vt[v_slot<kD>(r_lo + 8, col >> 3) + (col & 7)]));
        const bf16x8 vop = __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo),
                                                   __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3,
                                                   4, 5, 6, 7);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[grp], acc[db], 0, 0, 0);
      }
  };

  // One pipelined step: the weights of tile t (in `cur`) are formed while the matrix cores
  // compute the scores of tile t+1 (into `nxt`); then P(t) V(t) is accumulated.  Loads run
  // two tiles ahead for K (into Kf), one for V (into Vf); the step reads K(t+1) from Kr and
  // V(t) from Vr.  Every wave of the workgroup runs these steps up to the workgroup's last
  // tile, so the step is one straight block and the weights' FMAs and exps interleave with
  // the score products; a wave whose diagonal lies before the last tile scores that tile
  // needlessly but never uses it (step_last skips it).
  const int t_last = n_tiles - 1;
  auto step = [&](int t, Tile& cur, Tile& nxt, bf16* Kf, bf16* Vf, const bf16* Kr,
                  const bf16* Vr) __attribute__((always_inline)) {
    if (t + 2 < n_tiles) issue_k(t + 2, Kf);
    issue_v(t + 1, Vf);
    bf16x8 pop[4];
    // Two waves share each SIMD (one from each of the CU's two workgroups).  The score and
    // weight phase, whose exps and FMAs leave the matrix core idle between its products,
    // issues at raised priority; a wave in its P V phase (back-to-back products) then fills
    // the matrix core in those gaps instead of competing with it for issue.  [4,32,2048,128]
    // 137.4 -> 135.5 us, [1,32,32768,128] 7575 -> 7075 us.
    __builtin_amdgcn_s_setprio(1);
    compute_s(nxt, Kr);
    const float psum = weights(cur, pop);
    // kS score products (one operand read each), ~96 VALU instructions of weights
    constexpr int kS = 2 * kKSteps;
    __builtin_amdgcn_sched_group_barrier(kSchedDSRead, kS / 4, 0);
#pragma unroll
    for (int i = 0; i < kS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedVALU, 96 / kS, 0);
      if (i < kS - kS / 4) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 1, 0);
    }
    checked_weights(cur, pop, psum);
    __builtin_amdgcn_s_setprio(0);
    pv(Vr, pop);
    // kP P.V products (two transposed reads each)
    constexpr int kP = 4 * kDBlocks;
    __builtin_amdgcn_sched_group_barrier(kSchedDSRead, kP / 2, 1);
#pragma unroll
    for (int i = 0; i < kP; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 1);
      if (i < kP - kP / 4) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 1);
    }
    // tile t+1 is used unless it is the last tile and lies past this wave's diagonal
    if ((t + 1 < wave_tiles || t + 1 < t_last) && need_mask(t + 1)) apply_mask(nxt, (t + 1) * kBN);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of the next tiles has landed
    __syncthreads();
  };
  // The last tile: its weights and P V, no loads, no barrier after it (its K tile was read in
  // the step before, whose barrier frees the K buffers for the epilogue).
  auto step_last = [&](int t, Tile& cur, const bf16* Vr) __attribute__((always_inline)) {
    if (t < wave_tiles) {
      bf16x8 pop[4];
      __builtin_amdgcn_s_setprio(1);
      checked_weights(cur, pop, weights(cur, pop));
      __builtin_amdgcn_s_setprio(0);
      pv(Vr, pop);
    }
  };

  // The sweep runs inside one function whose four tile buffers are declared non-aliasing:
  // the compiler then knows that the fills a step issues do not touch the tiles it reads,
  // and leaves the wait for them to the step's closing waitcnt (it would otherwise wait for
  // the fills just issued before the first LDS read after them).  Tile t lives in buffer
  // (t - t0) & 1; its scores in ta when t - t0 is even, else in tb.
  const int t0 = t_first;
  auto sweep = [&](bf16* __restrict__ k0, bf16* __restrict__ k1, bf16* __restrict__ v0,
                   bf16* __restrict__ v1) {
    // ---- prologue: K(t0), V(t0), K(t0+1) in flight; scores and max of tile t0
    issue_k(t0, k0);
    issue_v(t0, v0);
    if (t0 + 1 < n_tiles) issue_k(t0 + 1, k1);
    // Q and K(t0) have landed once at most the later fills (kSlices instructions each) are
    // in flight
    if (t0 + 1 < n_tiles)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kSlices));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kSlices));
    // a bare barrier: __syncthreads() would also wait for the fills still in flight
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Tile ta, tb;
    __builtin_amdgcn_s_setprio(1);
    compute_s(ta, k0);
    if (need_mask(t0)) apply_mask(ta, t0 * kBN);
    raise_ref(row_max(ta));
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0);  // V(t0) and K(t0+1) have landed
    __syncthreads();  // ... for every wave; every wave is done with K(t0) before K(t0+2) overwrites it

    for (int t = t0; t < t_last; t += 2) {
      step(t, ta, tb, k0, v1, k1, v0);
      if (t + 1 < t_last) step(t + 1, tb, ta, k1, v0, k0, v1);
    }
    if (((t_last - t0) & 1) == 0)
      step_last(t_last, ta, v0);
    else
      step_last(t_last, tb, v1);
  };
  // The buffers are passed at an offset the optimiser cannot see (zero at run time): with
  // constant arguments it would substitute the constants into the body before inlining it,
  // and the non-aliasing of the parameters would be lost.
  int hidden_zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
  sweep(tiles[0] + hidden_zero, tiles[1] + hidden_zero, tiles[2] + hidden_zero, tiles[3] + hidden_zero);

  // ---- epilogue: o = u / l, staged through LDS so that each store instruction writes whole
  // rows of O (four of 256 bytes, or eight of 128 at head_dim 64).  Every wave has passed
  // the last step's barrier, so the K buffers are free: wave w takes 32 rows of them, the
  // 16-byte chunks of row r XOR-swizzled by r % (chunks per row).
  const float l_tot = other_half_sum(l_run);
  const bool valid = qi < L;
  const float inv = 1.0f / l_tot;
  bf16* stage = &tiles[0][0] + w * (32 * kD);
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      floatx4 x;
#pragma unroll
      for (int c = 0; c < 4; ++c) x[c] = valid ? acc[db][4 * a + c] * inv : 0.f;
      const int chunk = (4 * db + a) ^ (lq & (kChunks - 1));
      *reinterpret_cast<bf16x4*>(stage + lq * kD + 8 * chunk + 4 * hl) =
          __builtin_convertvector(x, bf16x4);
    }
#pragma unroll
  for (int j = 0; j < kChunks / 2; ++j) {
    const int r = (64 / kChunks) * j + lane / kChunks, c = lane % kChunks;
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(stage + r * kD + 8 * (c ^ (r & (kChunks - 1))));
    const int row = m0 + w * 32 + r;
    // written once and never read here: streamed past the caches, which keep K and V (as
    // whole rows; lane-scattered pieces stored this way would each go to memory alone)
    if (row < n) __builtin_nontemporal_store(y, reinterpret_cast<bf16x8*>(O + base + (size_t)row * kD + 8 * c));
  }
  if (LSE && hl == 0 && qi - q_start < n)
    LSE[(size_t)bh * n + (qi - q_start)] = valid ? (m_ref * ATTN_LN2 + __logf(l_tot)) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_bf16(const bf16* q, const bf16* k, const bf16* v, bf16* o, float* lse,
                           const int32_t* seq_lens, int batch, int heads, int kv_heads, int n,
                           int n_kv, int q_start, int head_dim, int causal, int window,
                           float scale, hipStream_t stream) {
  const int n_qtiles = (n + kBM - 1) / kBM;
  const dim3 grid((unsigned)n_qtiles * batch * heads);
  const float c = scale * ATTN_LOG2E;
  const int w = window > 0 ? window : 0;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, q, k, v, o, lse, seq_lens, batch,
                       heads, kv_heads, n, n_kv, q_start, n_qtiles, causal, w, c);
  };
  if (head_dim == 64) {
    if (w > 0) go(fwd_bf16_kernel<true, 64>);
    else go(fwd_bf16_kernel<false, 64>);
  } else {
    if (w > 0) go(fwd_bf16_kernel<true, 128>);
    else go(fwd_bf16_kernel<false, 128>);
  }
  return hipGetLastError();
}
