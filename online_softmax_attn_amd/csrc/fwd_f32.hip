// fp32 prefill attention with fp64 scores (gfx950).
//
// The stress workload multiplies Q and K by 40, so scaled scores reach the thousands.  An
// fp32 dot product of 64 such terms carries an absolute error of ~1e-3 in the score, which
// moves the output by far more than the 1e-5 the fp32 path must hold.  The product of two
// fp32 numbers is exact in fp64, so the scores are accumulated in fp64, and the running
// (m, l, u) summary of el-ai.com "Attenzione: softmax online, riscalamento e memoria"
// (section 2) is kept in fp64 as well: for each admitted key, m' = max(m, s); l and u are
// both multiplied by exp(m - m') before the key's exp(s - m') and exp(s - m') v are added.
// The empty state m = -inf is safe: the first admitted key always has s > -inf, and
// exp(-inf) = 0 clears l and u.
//
// Work decomposition: one workgroup of 256 threads owns QPB consecutive queries of one
// (batch, head); each query is served by TPQ = head_dim / 32 threads that each hold 32 of
// its dimensions (query slice, accumulator slice) and combine partial dot products with
// lane shuffles.  K and V stream through LDS in tiles of 32 keys.  This path exists for
// exactness, not speed: its workloads are small.  Grouped K/V heads only change which K/V
// slice is read; a causal window only narrows each query's admitted key range.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTileKeys = 32;
constexpr int kSlice = 32;  // dimensions per thread

template <int D>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(const float* __restrict__ Q,
                                                           const float* __restrict__ K,
                                                           const float* __restrict__ V,
                                                           float* __restrict__ O,
                                                           float* __restrict__ LSE,
                                                           const int32_t* __restrict__ lens,
                                                           int H, int Hkv, int n, int causal,
                                                           int window, double scale) {
  constexpr int TPQ = D / kSlice;        // threads per query
  constexpr int QPB = kThreads / TPQ;    // queries per workgroup
  __shared__ float Ks[kTileKeys * D];
  __shared__ float Vs[kTileKeys * D];

  const int bh = blockIdx.y;
  const int b = bh / H;
  const int q0 = blockIdx.x * QPB;
  int L = lens ? lens[b] : n;
  L = L < 0 ? 0 : (L > n ? n : L);
  const size_t base = (size_t)bh * n * D;
  const size_t kv_base = ((size_t)b * Hkv + (bh % H) / (H / Hkv)) * n * D;

  const int tid = threadIdx.x;
  const int qi = q0 + tid / TPQ;
  const int part = tid % TPQ;
  const bool row_valid = qi < L;

  double qv[kSlice];
  double u[kSlice];
#pragma unroll
  for (int c = 0; c < kSlice; ++c) {
    qv[c] = row_valid ? (double)Q[base + (size_t)qi * D + part * kSlice + c] : 0.0;
    u[c] = 0.0;
  }
  double m = -INFINITY, l = 0.0;

  // keys any row of this workgroup can admit
  int kend = L;
  if (causal) kend = min(kend, q0 + QPB);
  const int kbeg = window ? max(0, q0 - window + 1) : 0;
  const int kmax = row_valid ? (causal ? min(qi, L - 1) : L - 1) : -1;  // last admitted key
  const int kmin = window ? qi - window + 1 : 0;                       // first admitted key

  for (int k0 = kbeg; k0 < kend; k0 += kTileKeys) {
    // cooperative fp32 tile load; keys past L are zero-filled and never admitted
    for (int i = tid; i < kTileKeys * D / 4; i += kThreads) {
      const int row = (i * 4) / D, col = (i * 4) % D;
      const int key = k0 + row;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (key < L) {
        kk = *reinterpret_cast<const float4*>(K + kv_base + (size_t)key * D + col);
        vv = *reinterpret_cast<const float4*>(V + kv_base + (size_t)key * D + col);
      }
      *reinterpret_cast<float4*>(Ks + row * D + col) = kk;
      *reinterpret_cast<float4*>(Vs + row * D + col) = vv;
    }
    __syncthreads();
    const int jn = min(kTileKeys, kend - k0);
    for (int j = 0; j < jn; ++j) {
      double s = 0.0;
#pragma unroll
      for (int c = 0; c < kSlice; ++c) s = fma(qv[c], (double)Ks[j * D + part * kSlice + c], s);
#pragma unroll
      for (int off = 1; off < TPQ; off <<= 1) s += __shfl_xor(s, off);
      s *= scale;
      if (k0 + j <= kmax && k0 + j >= kmin) {
        const float* vrow = Vs + j * D + part * kSlice;
        if (s > m) {
          const double a = exp(m - s);  // rescales l and u together; 0 on the first key
          l = l * a + 1.0;
#pragma unroll
          for (int c = 0; c < kSlice; ++c) u[c] = fma(u[c], a, (double)vrow[c]);
          m = s;
        } else {
          const double p = exp(s - m);
          l += p;
#pragma unroll
          for (int c = 0; c < kSlice; ++c) u[c] = fma(p, (double)vrow[c], u[c]);
        }
      }
    }
    __syncthreads();
  }

  if (qi < n) {
    float* orow = O + base + (size_t)qi * D + part * kSlice;
    if (row_valid) {
      const double inv = 1.0 / l;
#pragma unroll
      for (int c = 0; c < kSlice; ++c) orow[c] = (float)(u[c] * inv);
      if (LSE && part == 0) LSE[(size_t)bh * n + qi] = (float)(m + log(l));
    } else {
#pragma unroll
      for (int c = 0; c < kSlice; ++c) orow[c] = 0.f;
      if (LSE && part == 0) LSE[(size_t)bh * n + qi] = -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const int32_t* seq_lens, int batch, int heads, int kv_heads, int n,
                          int head_dim, int causal, int window, float scale, hipStream_t stream) {
  const dim3 block(kThreads);
  if (head_dim == 64) {
    const dim3 grid((n + 127) / 128, batch * heads);
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, q, k, v, o, lse, seq_lens,
                       heads, kv_heads, n, causal, window, (double)scale);
  } else {
    const dim3 grid((n + 63) / 64, batch * heads);
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, q, k, v, o, lse, seq_lens,
                       heads, kv_heads, n, causal, window, (double)scale);
  }
  return hipGetLastError();
}
