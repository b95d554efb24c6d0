// Backward pass of exact attention on gfx950 matrix cores: bf16 inputs, head_dim 128, fp32
// gradients.
//
// pierluigilucio.it "Sviluppo AI ed Algebra Lineare" (section "Ricalcolo nel Backward Pass")
// describes it: the forward pass keeps only the per-row normalisation statistics, and the
// backward pass recomputes the score and probability blocks from Q, K and V instead of
// reading an n x n matrix.  Here the statistic is the log-sum-exp L_i the forward writes,
// so a recomputed weight is P_ij = exp(scale <q_i, k_j> - L_i).  With D_i = <dO_i, O_i>
// (= sum_j P_ij dP_ij):
//     dV_j = sum_i P_ij dO_i            dP_ij = <dO_i, v_j>
//     dS_ij = P_ij (dP_ij - D_i)        dQ_i = scale sum_j dS_ij k_j
//                                       dK_j = scale sum_i dS_ij q_i
// Two kernels: dQ (one wave per 32 queries, sweeping key tiles, as the forward pass does;
// it also forms D_i from the dO row it holds and leaves it for the next kernel) and dK/dV (a pair of waves per 32 keys, sweeping query tiles: one
// wave forms the weights and dV, its partner dP, dS and dK, with the weights handed over
// through LDS).  Both sweeps use the forward's register layouts: the MFMA column is the row
// that owns the accumulator (a query for dQ, a key for dK/dV), weights go from the score
// registers to the B operand as bf16, and the transposed A operands (K^T for dQ; dO^T and
// Q^T for dK/dV) come from row-major LDS tiles through ds_read_b64_tr_b16.  Masked pairs
// get weight 0 by selection, so padding never enters a sum whatever it holds.
//
// Grouped K/V heads: dQ reads the shared K/V slice; one dK/dV workgroup sweeps the query
// tiles of every query head of its group in turn, so the sum over the group stays in
// registers (no atomics, no second pass).  A causal window w narrows both sweeps to the
// pairs i - w < j <= i.
#include "common.h"

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kTile = 64;  // rows per streamed LDS tile
constexpr int kTileElems = kTile * kD;

typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

// LDS tile swizzle (16-byte chunks of 256-byte rows) that serves both access kinds: the
// 16 consecutive rows of one 16-byte operand read land in 16 distinct chunk slots, and the
// 8 rows of one transposed read spread over all four 64-byte bank groups.
__device__ __forceinline__ int sw_slot(int r, int c) {
  return r * kD + ((c ^ (((r & 3) << 2) | ((r >> 2) & 3))) << 3);
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int n) {
  const int L = lens ? lens[b] : n;
  return L < 0 ? 0 : (L > n ? n : L);
}

// Fill a 64-row bf16 tile (rows t*64 .. t*64+63 of the descriptor's range) straight into
// LDS: wave w writes 1 KiB slices 4w..4w+3; lane i of slice j lands in row 4j + i/16, chunk
// slot i%16, and fetches the logical chunk the swizzle puts there.
struct TileFill {
  int src[4];
  __device__ TileFill(int w, int lane) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * (4 * w + i) + (lane >> 4);
      const int pc = lane & 15;
      const int c = pc ^ (((r & 3) << 2) | ((r >> 2) & 3));
      src[i] = (r * kD + 8 * c) * 2;
    }
  }
  __device__ void issue(rsrc_t rs, bf16* dst, int t, int w) const {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      load_lds16(rs, (lds_void*)&dst[(4 * w + i) * 512], t * kTile * kD * 2 + src[i]);
  }
};

// The transposed operand of one 16-row group of a tile: lane (column l % 32, half h) gets
// rows 16 g + 8 (e/4) + 4 h + e%4 (e = 0..7) of column 32 db + l % 32.
__device__ __forceinline__ bf16x8 tr_operand(const bf16* tile, int g, int db, int lane) {
  const int tg = lane >> 4, ts = lane & 15;
  const int col = 32 * db + 16 * (tg & 1) + 4 * (ts & 3);
  const int r_lo = 16 * g + 4 * (tg >> 1) + (ts >> 2);
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(&tile[sw_slot(r_lo, col >> 3) + (col & 7)]));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(&tile[sw_slot(r_lo + 8, col >> 3) + (col & 7)]));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, lo), __builtin_bit_cast(bf16x4, hi), 0, 1, 2, 3, 4, 5, 6, 7);
}

// ------------------------------------------------------------------------ dQ
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const bf16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Dv, const int32_t* __restrict__ lens, float* __restrict__ dQ, int B,
    int H, int Hkv, int n,
    int n_qtiles, int causal, int window, float c_log2, float scale) {
  // K tiles in slots 0 and 1, V tiles in slots 2 and 3 (one LDS object: the compiler then
  // keeps the non-aliasing of the four slots declared below)
  __shared__ __attribute__((aligned(1024))) bf16 tiles[4][kTileElems];
  constexpr int kBM = 128;

  const int HB = H * B;
  const GridSlot slot = causal_grid_slot((int)blockIdx.x, HB, n_qtiles);  // heaviest first
  const int qt = n_qtiles - 1 - slot.rank;
  const int bh = slot.bh;
  const int L = clamp_len(lens, bh / H, n);
  const size_t base = (size_t)bh * n * kD;
  const size_t kv_base = ((size_t)(bh / H) * Hkv + (bh % H) / (H / Hkv)) * n * kD;
  const int m0 = qt * kBM;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hl = lane >> 5, lq = lane & 31;
  const int qi = m0 + 32 * w + lq;

  if (m0 >= L) {
    for (int i = tid; i < kBM * kD / 4; i += kThreads) {
      const int r = m0 + (i * 4) / kD;
      if (r < n) *reinterpret_cast<floatx4*>(dQ + base + (size_t)r * kD + (i * 4) % kD) = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    for (int r = m0 + tid; r < min(m0 + kBM, n); r += kThreads) Dv[(size_t)bh * n + r] = 0.f;
    return;
  }

  const uint32_t valid_bytes = (uint32_t)L * kD * 2;
  const rsrc_t rq = make_rsrc(Q + base, valid_bytes);
  const rsrc_t rk = make_rsrc(K + kv_base, valid_bytes);
  const rsrc_t rv = make_rsrc(V + kv_base, valid_bytes);
  const rsrc_t rg = make_rsrc(dO + base, valid_bytes);

  bf16x8 qop[8], gop[8];  // Q^T and dO^T operands: dims 16 ks + 8 hl .. +7 of query qi
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    qop[ks] = load_b128(rq, (qi * kD + 16 * ks + 8 * hl) * 2);
    gop[ks] = load_b128(rg, (qi * kD + 16 * ks + 8 * hl) * 2);
  }
  const bool row_ok = qi < L;
  const float lse2 = row_ok ? LSE[(size_t)bh * n + qi] * ATTN_LOG2E : 0.f;
  // admitted (this lane's query, key) pairs: lo <= qi - key < hi with lo = 0 when causal
  // (else -n) and hi = window when one is set (else n); a padding query admits none
  const int mask_lo = causal ? 0 : -n;
  const int mask_hi = window ? window : n;
  // D_i = <dO_i, O_i>: this lane holds half of row qi of dO (the operand above); O is read in
  // the same layout and the halves of lanes l and l ^ 32 are added.  Written for the dK/dV
  // kernel (0 on padding rows).
  float Di;
  {
    const rsrc_t ro = make_rsrc(O + base, valid_bytes);
    float x = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 ov = load_b128(ro, (qi * kD + 16 * ks + 8 * hl) * 2);
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        x = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{ov[e], ov[e + 1]}, bf16x2{gop[ks][e], gop[ks][e + 1]}, x, false);
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    Di = row_ok ? __uint_as_float(sw[0]) + __uint_as_float(sw[1]) : 0.f;
    if (hl == 0 && qi < n) Dv[(size_t)bh * n + qi] = Di;
  }

  const int kend = causal ? min(L, m0 + kBM) : L;
  const int n_tiles = (kend + kTile - 1) / kTile;  // tiles [t_first, n_tiles)
  const int t_first = window ? max(0, m0 - window + 1) / kTile : 0;
  const int wave_q_first = m0 + 32 * w, wave_q_last = wave_q_first + 31;
  const int wave_tiles = causal ? min(n_tiles, wave_q_last / kTile + 1) : n_tiles;
  const TileFill fill(w, lane);

  floatx16 acc[4];  // dQ^T: lane holds d = 32 db + 8 (r/4) + 4 hl + r%4 of query qi
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  // One step: tile t+1 is fetched into (Kf, Vf) while tile t is used from (Kt, Vt).
  auto step = [&](int t, bf16* Kf, bf16* Vf, const bf16* Kt, const bf16* Vt)
      __attribute__((always_inline)) {
    if (t + 1 < n_tiles) {
      fill.issue(rk, Kf, t + 1, w);
      fill.issue(rv, Vf, t + 1, w);
    }
    if (t < wave_tiles) {
      const int k0 = t * kTile;
      floatx16 s[2], dp[2];  // S^T and dP^T: lane holds key 32 kb + 8 (r/4) + 4 hl + r%4
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[kb][r] = 0.f;
          dp[kb][r] = 0.f;
        }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Kt[sw_slot(32 * kb + lq, 2 * ks + hl)]);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vt[sw_slot(32 * kb + lq, 2 * ks + hl)]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], s[kb], 0, 0, 0);
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gop[ks], dp[kb], 0, 0, 0);
        }
      const bool need_mask = !row_ok || (k0 + kTile > L) || (causal && k0 + kTile - 1 > wave_q_first) ||
                             (window && k0 <= wave_q_last - window);
      if (need_mask) {  // scores outside the mask become -inf, their weights 0
        // element (kb, r) is key k0 + 4 hl + o with o = 32 kb + 8 (r/4) + r%4; admitted iff
        // lo <= qi - key < hi (one unsigned compare) and key < L
        const unsigned base = (unsigned)(qi - k0 - 4 * hl - mask_lo);
        const unsigned mask_span = row_ok ? (unsigned)(mask_hi - mask_lo) : 0u;
        const int o_lim = L - k0 - 4 * hl;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int o = 32 * kb + 8 * (r >> 2) + (r & 3);
            const bool ok = base - (unsigned)o < mask_span && o < o_lim;
            s[kb][r] = ok ? s[kb][r] : -INFINITY;
          }
      }
      bf16x8 dsop[4];
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int kb = grp >> 1, r0 = 8 * (grp & 1);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          floatx2 d2;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = r0 + e + u;
            const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c_log2, -lse2));  // 0 if masked
            d2[u] = p * (dp[kb][r] - Di);
          }
          const bf16x2 db2 = __builtin_convertvector(d2, bf16x2);
          dsop[grp][e] = db2[0];
          dsop[grp][e + 1] = db2[1];
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Kt, grp, db, lane), dsop[grp], acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile t+1 has landed
    __syncthreads();
  };
  // The sweep runs inside one function whose four tile slots are declared non-aliasing: the
  // compiler then knows that a step's fills do not touch the tile it reads, and leaves the
  // wait for them to the step's closing waitcnt (it would otherwise wait for the fills just
  // issued before the first LDS read).  Tile t lives in slot (t - t_first) & 1.
  auto sweep = [&](bf16* __restrict__ k0, bf16* __restrict__ k1, bf16* __restrict__ v0,
                   bf16* __restrict__ v1) {
    fill.issue(rk, k0, t_first, w);
    fill.issue(rv, v0, t_first, w);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = t_first; t < n_tiles; t += 2) {
      step(t, k1, v1, k0, v0);
      if (t + 1 < n_tiles) step(t + 1, k0, v0, k1, v1);
    }
  };
  // The slots are passed at an offset the optimiser cannot see (zero at run time): with
  // constant arguments it would substitute the constants into the body before inlining it,
  // and the non-aliasing of the parameters would be lost.
  int hidden_zero;
  asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
  sweep(tiles[0] + hidden_zero, tiles[1] + hidden_zero, tiles[2] + hidden_zero, tiles[3] + hidden_zero);

  // dQ rows staged through LDS so that each store writes two whole 512-byte rows: every wave
  // is past the last step's barrier, so the four slots (64 KiB) are free and wave w takes
  // slot w for its 32 rows, the 16-byte chunks of row r XOR-swizzled by r.  The lane's
  // indices are taken afresh from the lane id (mbcnt) rather than kept live through the key
  // loop, which runs at the register limit.
  {
    const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int hl_out = ln >> 5, lq_out = ln & 31;
    const int row0 = __builtin_amdgcn_readfirstlane(qi - lq_out);  // m0 + 32 w
    floatx4* stage = reinterpret_cast<floatx4*>(tiles[(row0 - m0) >> 5]);  // 32 rows x 32 chunks
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        floatx4 x;
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = row_ok ? acc[db][4 * a + c] * scale : 0.f;
        // d = 32 db + 8 a + 4 hl .. +3 is chunk 8 db + 2 a + hl of the row
        stage[32 * lq_out + ((8 * db + 2 * a + hl_out) ^ lq_out)] = x;
      }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int r = 2 * j + hl_out, c = lq_out;
      const int row = row0 + r;
      // written once and never read here: streamed past the caches
      if (row < n) __builtin_nontemporal_store(stage[32 * r + (c ^ r)], reinterpret_cast<floatx4*>(dQ + base + (size_t)row * kD + 4 * c));
    }
  }
}

// ------------------------------------------------------------------------ dK, dV
// Eight waves in four pairs; pair p owns the keys k0 + 32 p .. +31 of the workgroup's 128.
// In each step (one 64-query tile) the V-wave of a pair (waves 0-3) forms S = Q K^T and the
// weights P of its keys and hands P to its partner through LDS, while the K-wave (waves 4-7,
// on the same SIMD) forms dP = dO V^T.  After a barrier the V-wave accumulates dV += dO^T P
// and the K-wave dS = P (dP - D), dK += Q^T dS.  Each wave issues 32 MFMAs per step, and the
// two waves of a SIMD cover each other's latencies.  The K-waves, whose first phase is the
// shorter one, issue the tile loads and subtract D from dP before the barrier.
constexpr int kPairThreads = 512;
__global__ __launch_bounds__(kPairThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    const int32_t* __restrict__ lens, float* __restrict__ dK, float* __restrict__ dV, int B,
    int H, int Hkv, int n, int causal, int window, float c_log2, float scale, float log2e) {
  // one LDS object (the compiler then keeps the non-aliasing of the K-waves' slots below)
  struct Tiles {
    bf16 q[2][kTileElems];
    bf16 g[2][kTileElems];     // dO
    float l[2][kTile];         // log2-unit LSE; +inf on padding
    float d[2][kTile];
    floatx4 p[4][2][4][64];    // weights handed from V-wave to K-wave: [pair][block][group][lane]
  };
  __shared__ __attribute__((aligned(1024))) Tiles lds;
  auto& Qs = lds.q;
  auto& Gs = lds.g;
  auto& Ls = lds.l;
  auto& Ds = lds.d;
  auto& Ps = lds.p;
  constexpr int kBK = 128;

  const int HB = Hkv * B;
  const GridSlot slot = causal_grid_slot((int)blockIdx.x, HB, (n + kBK - 1) / kBK);
  const int kt = slot.rank;  // key block 0 has the most causal work: first
  const int bhk = slot.bh;   // b * Hkv + K/V head
  const int b = bhk / Hkv, G = H / Hkv;
  const int bh0 = b * H + (bhk % Hkv) * G;  // first query head of the group
  const int L = clamp_len(lens, b, n);
  const size_t kv_base = (size_t)bhk * n * kD;
  const int k0 = kt * kBK;
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = w & 3;
  const bool vwave = w < 4;
  const int kj = k0 + 32 * pair + lq;  // this lane's key

  if (k0 >= L) {
    for (int i = tid; i < kBK * kD / 4; i += kPairThreads) {
      const int r = k0 + (i * 4) / kD;
      if (r < n) {
        *reinterpret_cast<floatx4*>(dK + kv_base + (size_t)r * kD + (i * 4) % kD) = floatx4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<floatx4*>(dV + kv_base + (size_t)r * kD + (i * 4) % kD) = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  const uint32_t valid_bytes = (uint32_t)L * kD * 2;
  // the V-wave's operand is this lane's key row of K (for S), the K-wave's its row of V (dP)
  const rsrc_t rop = make_rsrc((vwave ? K : V) + kv_base, valid_bytes);
  bf16x8 op[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) op[ks] = load_b128(rop, (kj * kD + 16 * ks + 8 * hl) * 2);
  const bool key_ok = kj < L;
  // admitted (query q, this lane's key) pairs: lo <= q - kj < hi with lo = 0 when causal
  // (else -n) and hi = window when one is set (else n); a padding key admits none
  const int mask_lo = causal ? 0 : -n;
  const unsigned mask_span = key_ok ? (unsigned)((window ? window : n) - mask_lo) : 0u;
  const int wave_k_first = k0 + 32 * pair, wave_k_last = wave_k_first + 31;

  // query tiles [t0, t1) of each of the G query heads, swept head after head: step `it`
  // is tile t0 + it % nt of head it / nt
  const int t0 = causal ? k0 / kTile : 0;  // first query tile that admits any key here
  const int qend = window ? min(L, k0 + kBK - 1 + window) : L;  // later queries admit none
  const int t1 = (qend + kTile - 1) / kTile;
  const int nt = t1 - t0;
  const int steps = G * nt;
  // Tile fill by the four K-waves (K-wave kw writes the 1 KiB slices 4 kw .. 4 kw + 3 of each
  // tile): the V-waves' first phase is the longer one, and loads issued by all eight waves
  // at once queue behind each other at the start of the step.
  const int kw = w & 3;
  int src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (4 * kw + i) + (lane >> 4);
    const int pc = lane & 15;
    const int c = pc ^ (((r & 3) << 2) | ((r >> 2) & 3));
    src[i] = (r * kD + 8 * c) * 2;
  }
  auto issue = [&](int it, bf16* Qd, bf16* Gd) __attribute__((always_inline)) {  // K-waves only
    const int bh = bh0 + it / nt, t = t0 + it % nt;
    const size_t base = (size_t)bh * n * kD;
    const rsrc_t rq = make_rsrc(Q + base, valid_bytes);
    const rsrc_t rg = make_rsrc(dO + base, valid_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      load_lds16(rq, (lds_void*)&Qd[(4 * kw + i) * 512], t * kTile * kD * 2 + src[i]);
      load_lds16(rg, (lds_void*)&Gd[(4 * kw + i) * 512], t * kTile * kD * 2 + src[i]);
    }
  };
  // the tile's LSE (+inf on padding) and D, one query per lane of wave 0: loaded into
  // registers when the tile's loads are issued and written to LDS (the LSE in log2 units)
  // at the end of the step, so the wave never waits on them mid-step.  log2e arrives as an
  // argument: a literal factor would be folded into the load's branch, and the wave would
  // wait for the load there.
  auto load_ld = [&](int it, float& l, float& d) {
    const int bh = bh0 + it / nt, q = (t0 + it % nt) * kTile + tid;
    l = q < L ? LSE[(size_t)bh * n + q] : INFINITY;
    d = q < L ? Dv[(size_t)bh * n + q] : 0.f;
  };
  auto skip = [&](int t, int qb) {
    const int q0 = t * kTile + 32 * qb;
    return (causal && q0 + 31 < wave_k_first) ||  // every query of the block precedes every key
           (window && q0 - wave_k_last >= window);  // every query is past every key's window
  };
  auto masked = [&](int t, int qb) {
    const int q0 = t * kTile + 32 * qb;
    return !key_ok || (k0 + kBK > L) || (causal && q0 < wave_k_last) ||
           (window && q0 + 31 - wave_k_first >= window);
  };

  floatx16 acc[4];  // dV^T (V-wave) or dK^T (K-wave): lane holds d = 32 db + 8 (r/4) + 4 hl + r%4 of key kj
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  if (!vwave) issue(0, Qs[0], Gs[0]);
  if (tid < kTile) {
    float l, d;
    load_ld(0, l, d);
    Ls[0][tid] = l * log2e;
    Ds[0][tid] = d;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  if (vwave) {
    for (int it = 0; it < steps; ++it) {
      const int buf = it & 1;
      float l_next = 0.f, d_next = 0.f;
      if (it + 1 < steps && tid < kTile) load_ld(it + 1, l_next, d_next);
      const int t = t0 + it % nt;
      const bf16* Qt = Qs[buf];
      const bf16* Gt = Gs[buf];
      // S of both 32-query blocks as two interleaved product chains (a block wholly outside
      // the mask is computed too and masked to zero weights: no branch between the chains
      // and the exps)
      floatx16 s[2];  // S: lane holds query q0 + 8 (r/4) + 4 hl + r%4 of key kj
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qt[sw_slot(32 * qb + lq, 2 * ks + hl)]);
          s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, op[ks], s[qb], 0, 0, 0);
        }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (masked(t, qb)) {  // scores outside the mask become -inf, their weights 0
          // element r is query q = q0 + 4 hl + 8 (r/4) + r%4, admitted iff lo <= q - kj < hi:
          // one unsigned compare of (q - kj - lo) against the span per element
          const unsigned base = (unsigned)(t * kTile + 32 * qb + 4 * hl - kj - mask_lo);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[qb][r] = base + (unsigned)(8 * (r >> 2) + (r & 3)) < mask_span ? s[qb][r] : -INFINITY;
        }
      }
      bf16x8 pop[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const floatx4 l4 = *reinterpret_cast<const floatx4*>(&Ls[buf][32 * qb + 8 * a + 4 * hl]);
          floatx4 p4;
#pragma unroll
          for (int c = 0; c < 4; ++c)  // 0 on padding rows (l = +inf) and masked scores
            p4[c] = __builtin_amdgcn_exp2f(fmaf(s[qb][4 * a + c], c_log2, -l4[c]));
          Ps[pair][qb][a][lane] = p4;
          const bf16x4 pb = __builtin_convertvector(p4, bf16x4);
#pragma unroll
          for (int c = 0; c < 4; ++c) pop[qb][a >> 1][4 * (a & 1) + c] = pb[c];  // register 4a + c
        }
      __syncthreads();  // the weights are in LDS for the K-waves
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (skip(t, qb)) continue;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int db = 0; db < 4; ++db)  // dV^T += dO^T P
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Gt, 2 * qb + g, db, lane), pop[qb][g], acc[db], 0, 0, 0);
      }
      if (it + 1 < steps && tid < kTile) {  // the previous step's readers are past its barrier
        Ls[buf ^ 1][tid] = l_next * log2e;
        Ds[buf ^ 1][tid] = d_next;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    // One K-wave step: tile it+1 is fetched into (Qf, Gf) while tile it is used from (Qt, Gt)
    // with its D values (Dt) and the V-waves' weights (P).
    auto kstep = [&](int it, bf16* Qf, bf16* Gf, const bf16* Qt, const bf16* Gt,
                     const float* Dt, const floatx4* P) __attribute__((always_inline)) {
      if (it + 1 < steps) issue(it + 1, Qf, Gf);
      const int t = t0 + it % nt;
      floatx16 dp[2];  // dP: lane holds query q0 + 8 (r/4) + 4 hl + r%4 of key kj
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)  // both blocks' chains interleaved, as the V-wave's S
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 ga = *reinterpret_cast<const bf16x8*>(&Gt[sw_slot(32 * qb + lq, 2 * ks + hl)]);
          dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, op[ks], dp[qb], 0, 0, 0);
        }
      // dP - D while the V-waves still form the weights (this wave would otherwise wait)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const floatx4 d4 = *reinterpret_cast<const floatx4*>(&Dt[32 * qb + 8 * a + 4 * hl]);
#pragma unroll
          for (int c = 0; c < 4; ++c) dp[qb][4 * a + c] -= d4[c];
        }
      __syncthreads();  // the V-waves' weights are in LDS
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (skip(t, qb)) continue;
        bf16x8 dsop[2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const floatx4 p4 = P[((2 * pair + qb) * 4 + a) * 64 + lane];
          floatx4 ds4;
#pragma unroll
          for (int c = 0; c < 4; ++c) ds4[c] = p4[c] * dp[qb][4 * a + c];  // dS = P (dP - D)
          const bf16x4 db4 = __builtin_convertvector(ds4, bf16x4);
#pragma unroll
          for (int c = 0; c < 4; ++c) dsop[a >> 1][4 * (a & 1) + c] = db4[c];  // register 4a + c
        }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
          for (int db = 0; db < 4; ++db)  // dK^T += Q^T dS
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand(Qt, 2 * qb + g, db, lane), dsop[g], acc[db], 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's share of tile it+1 has landed
      __syncthreads();
    };
    // The K-waves' sweep runs inside one function whose LDS slots are declared
    // non-aliasing: the compiler then knows that a step's fills do not touch what it reads,
    // and leaves the wait for them to the step's closing waitcnt (it would otherwise wait
    // for the fills just issued before the first LDS read).  Tile it lives in slot it & 1.
    auto ksweep = [&](bf16* __restrict__ q0, bf16* __restrict__ q1, bf16* __restrict__ g0,
                      bf16* __restrict__ g1, float* __restrict__ d0, float* __restrict__ d1,
                      floatx4* __restrict__ p) {
      for (int it = 0; it < steps; it += 2) {
        kstep(it, q1, g1, q0, g0, d0, p);
        if (it + 1 < steps) kstep(it + 1, q0, g0, q1, g1, d1, p);
      }
    };
    // The slots are passed at an offset the optimiser cannot see (zero at run time): with
    // constant arguments it would substitute the constants into the body before inlining
    // it, and the non-aliasing of the parameters would be lost.
    int hidden_zero;
    asm volatile("s_mov_b32 %0, 0" : "=s"(hidden_zero));
    ksweep(Qs[0] + hidden_zero, Qs[1] + hidden_zero, Gs[0] + hidden_zero, Gs[1] + hidden_zero,
           Ds[0] + hidden_zero, Ds[1] + hidden_zero, &Ps[0][0][0][0] + hidden_zero);
  }

  // dV (V-waves) then dK (K-waves), staged through LDS so that each store writes two whole
  // 512-byte rows: every wave is past the last step's barrier, so the Q and dO slots (64
  // KiB) are free; the four waves of a group take 16 KiB each (32 rows, the 16-byte chunks
  // of row r XOR-swizzled by r), one group after the other.
  floatx4* stage = reinterpret_cast<floatx4*>(&lds) + pair * (32 * 32);
  const float f = vwave ? 1.f : scale;
  float* out = vwave ? dV : dK;
#pragma unroll
  for (int phase = 0; phase < 2; ++phase) {
    if (phase == 1) __syncthreads();  // the V-waves have read their rows back
    if (vwave == (phase == 0)) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          floatx4 x;
#pragma unroll
          for (int c = 0; c < 4; ++c) x[c] = key_ok ? acc[db][4 * a + c] * f : 0.f;
          stage[32 * lq + ((8 * db + 2 * a + hl) ^ lq)] = x;
        }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int r = 2 * j + hl, c = lq;
        const int row = k0 + 32 * pair + r;
        // written once and never read here: streamed past the caches
        if (row < n) __builtin_nontemporal_store(stage[32 * r + (c ^ r)], reinterpret_cast<floatx4*>(out + kv_base + (size_t)row * kD + 4 * c));
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o,
                           const bf16* dout, const float* lse, const int32_t* seq_lens,
                           float* dq, float* dk, float* dv, int batch, int heads, int kv_heads,
                           int n, int causal, int window, float scale, void* workspace,
                           hipStream_t stream) {
  float* Dv = static_cast<float*>(workspace);  // D_i per query row, written by the dQ kernel
  const float c_log2 = scale * ATTN_LOG2E;
  const int n_qtiles = (n + 127) / 128;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)n_qtiles * batch * heads), dim3(kThreads), 0,
                     stream, q, k, v, dout, o, lse, Dv, seq_lens, dq, batch, heads, kv_heads, n,
                     n_qtiles, causal, window, c_log2, scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_ktiles = (n + 127) / 128;
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)n_ktiles * batch * kv_heads), dim3(kPairThreads),
                     0, stream, q, k, v, dout, lse, Dv, seq_lens, dk, dv, batch, heads, kv_heads,
                     n, causal, window, c_log2, scale, ATTN_LOG2E);
  return hipGetLastError();
}
