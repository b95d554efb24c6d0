// Merge of attention results computed over disjoint key sets.
//
// el-ai.com "Attenzione: softmax online, riscalamento e memoria", section 4: the summaries
// (m, l, u) of two disjoint blocks of keys combine by bringing both to the larger maximum
// and adding.  A finished part is an output o_s normalised over its own keys plus that set's
// log-sum-exp lse_s, i.e. the summary (lse_s, 1, o_s); folding all parts against
// m* = max_s lse_s gives
//     l = sum_s exp(lse_s - m*),   o = sum_s exp(lse_s - m*) o_s / l,   lse = m* + ln l.
// Parts with lse_s = -inf admit no key of the row and are skipped, so whatever their output
// holds never enters the sum.
//
// The parts are folded in one pass with a running maximum (section 2's recurrence applied to
// whole parts): a part above the maximum raises it and rescales what is already summed.
// Layout: 8 consecutive elements of a row per lane (16 bytes of bf16, 32 of fp32), d / 8
// lanes per row; each lane walks the parts with four loads in flight.  The kernel streams
// parts x rows x d elements once and is bound by HBM.
#include "common.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // parts whose loads are in flight together

__device__ __forceinline__ void load8(const bf16* p, float (&x)[8]) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
  const floatx4 a = *reinterpret_cast<const floatx4*>(p);
  const floatx4 b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[e + 4] = b[e];
  }
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];  // round to nearest even
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *reinterpret_cast<floatx4*>(p) = floatx4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<floatx4*>(p + 4) = floatx4{x[4], x[5], x[6], x[7]};
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const T* __restrict__ parts,
                                                         const float* __restrict__ lse_parts,
                                                         T* __restrict__ out,
                                                         float* __restrict__ lse_out,
                                                         int n_parts, long long rows) {
  constexpr int kLanes = D / 8;  // lanes per row
  constexpr int kRows = kThreads / kLanes;
  const long long row = (long long)blockIdx.x * kRows + threadIdx.x / kLanes;
  const int col = 8 * (threadIdx.x % kLanes);
  if (row >= rows) return;  // no barriers below

  // one pass over the parts with the running maximum of section 2: a part above it raises
  // it and rescales what is already summed; four parts' loads are in flight together
  float m = -INFINITY, l = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_parts; s0 += kUnroll) {
    float x[kUnroll][8], ls[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = s0 + u;
      ls[u] = s < n_parts ? lse_parts[(long long)s * rows + row] : -INFINITY;
      if (s < n_parts) load8(parts + ((long long)s * rows + row) * D + col, x[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!(ls[u] > -INFINITY)) continue;  // the part admits no key of this row
      const float m_new = __builtin_fmaxf(m, ls[u]);
      const float f = __builtin_amdgcn_exp2f((m - m_new) * ATTN_LOG2E);  // 0 from the empty state
      const float w = __builtin_amdgcn_exp2f((ls[u] - m_new) * ATTN_LOG2E);
      l = fmaf(l, f, w);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[u][e], acc[e] * f);
      m = m_new;
    }
  }
  if (m > -INFINITY) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
  }
  store8(out + row * D + col, acc);
  if (lse_out && col == 0) lse_out[row] = m > -INFINITY ? m + __logf(l) : -INFINITY;
}

template <typename T, int D>
hipError_t launch(const void* parts, const float* lse_parts, void* out, float* lse_out,
                  int n_parts, long long rows, hipStream_t stream) {
  constexpr int kRows = kThreads / (D / 8);
  const dim3 grid((unsigned)((rows + kRows - 1) / kRows));
  hipLaunchKernelGGL((merge_kernel<T, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const T*>(parts), lse_parts, static_cast<T*>(out), lse_out,
                     n_parts, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(bool bf16_data, const void* parts, const float* lse_parts, void* out,
                        float* lse_out, int n_parts, long long rows, int head_dim,
                        hipStream_t stream) {
  if (bf16_data)
    return head_dim == 128 ? launch<bf16, 128>(parts, lse_parts, out, lse_out, n_parts, rows, stream)
                           : launch<bf16, 64>(parts, lse_parts, out, lse_out, n_parts, rows, stream);
  return head_dim == 128 ? launch<float, 128>(parts, lse_parts, out, lse_out, n_parts, rows, stream)
                         : launch<float, 64>(parts, lse_parts, out, lse_out, n_parts, rows, stream);
}
