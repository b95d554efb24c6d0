// FP8 (E4M3) prefill attention on gfx950 matrix cores, head_dim 128, bf16 output.
//
// The FP8 variant of the aimpact.prandi.net FlashAttention page (FP8 section of
// FlashAttention-3): Q, K, V arrive as E4M3 codes with one fp32 scale per 64-row block
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

typedef int intx8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint4 lds_uint4;

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
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[2][kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t Vs[2][kTileBytes];

  const int HB = H * B;
  const int qt = n_qtiles - 1 - (int)(blockIdx.x / HB);  // heaviest causal tiles first
  const int j = blockIdx.x % HB;
  const int bh = (HB % 8 == 0) ? (j % 8) * (HB / 8) + j / 8 : j;  // one XCD per (b, h) range
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
  const rsrc_t rk = make_rsrc(K8 + (size_t)bhk * n * kD, (uint32_t)L * kD);
  const rsrc_t rv = make_rsrc(VT8 + (size_t)bhk * kD * n_pad, (uint32_t)(kD * n_pad));

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
  auto issue = [&](int t, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      load_lds16(rk, (lds_void*)&Ks[buf][(2 * w + i) * 1024], t * kBN * kD + k_src[i]);
      load_lds16(rv, (lds_void*)&Vs[buf][(2 * w + i) * 1024], t * kBN + v_src[i]);
    }
  };

  floatx16 acc[4];  // O^T: lane holds d = 32 db + 8 (r/4) + 4 hl + r%4 of query qi
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  float m_run = -INFINITY;  // running maximum of this lane's query, log2 units
  float l_run = 0.f;
  const intx8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                      0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
  const floatx16 zero16 = {};

  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) issue(t + 1, buf ^ 1);
    if (t < wave_tiles) {
      const uint8_t* Kt = Ks[buf];
      const uint8_t* Vt = Vs[buf];
      const int k0 = t * kBN;
      // ---- S^T = K Q^T: s[kb][r] is the raw score of key k0 + 32 kb + 16 hl + r
      floatx16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16;
        const int R = 32 * kb + lq;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c0 = 4 * ks + 2 * hl;
          const intx8 a = read32(Kt, k_off(R, c0), k_off(R, c0 + 1));
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qop[ks], s[kb], 0, 0, 0, 0, 0, 0);
        }
      }
      // ---- mask, tile maximum, exact running maximum
      const float c = c_q * ks_row[t];  // scale * s_Q * s_K * log2(e)
      const bool need_mask = (k0 + kBN > L) || (causal && k0 + kBN - 1 > wave_q_first);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r] * c;
          if (need_mask) {
            const int key = k0 + 32 * kb + 16 * hl + r;
            x = (key < L && (!causal || key <= qi)) ? x : -INFINITY;
          }
          s[kb][r] = x;
          mx = __builtin_fmaxf(mx, x);
        }
      mx = other_half_max(mx);
      const float m_new = __builtin_fmaxf(m_run, mx);
      if (__any(m_new > m_run)) {
        // floor at -1e30: a lane with no admitted key yet keeps alpha = 1 and weights 0
        const float alpha = __builtin_amdgcn_exp2f(__builtin_fmaxf(m_run, -1e30f) - __builtin_fmaxf(m_new, -1e30f));
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
      }
      m_run = m_new;
      const float m_use = __builtin_fmaxf(m_new, -1e30f);
      // ---- weights rounded to E4M3: byte e = 16 kb + r of the B operand
      intx8 pop;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = wd >> 2, r0 = 4 * (wd & 3);
        const float p0 = __builtin_amdgcn_exp2f(s[kb][r0] - m_use);
        const float p1 = __builtin_amdgcn_exp2f(s[kb][r0 + 1] - m_use);
        const float p2 = __builtin_amdgcn_exp2f(s[kb][r0 + 2] - m_use);
        const float p3 = __builtin_amdgcn_exp2f(s[kb][r0 + 3] - m_use);
        int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        pop[wd] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
      }
      // ---- l += row sum of the rounded weights; O^T += s_V (V^T P^T)
      const floatx16 lsum = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pop, zero16, 0, 0, 0, 0, 0, 0);
      const float sv = vs_row[t];
      floatx16 tmp[4];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int D = 32 * db + lq;
        const intx8 a = read32(Vt, v_off(D, hl), v_off(D, 2 + hl));
        tmp[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pop, zero16, 0, 0, 0, 0, 0, 0);
      }
      l_run += lsum[0];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = fmaf(sv, tmp[db][r], acc[db][r]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- epilogue: o = u / l (l is the whole row's sum: every lane of the MFMA column has it)
  if (qi < n) {
    bf16* orow = O + o_base + (size_t)qi * kD;
    const bool valid = qi < L;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        floatx4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = valid ? acc[db][4 * a + e] * inv : 0.f;
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * a + 4 * hl) = __builtin_convertvector(x, bf16x4);
      }
    if (LSE && hl == 0)
      LSE[(size_t)bh * n + qi] = valid ? (m_run * ATTN_LN2 + __logf(l_run)) : -INFINITY;
  }
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
