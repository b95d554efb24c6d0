// Measurement kernels (include/attn_probe.h): the sustained rates of the units the attention
// kernels use, on the device they run on.  Each kernel does one kind of work only and
// leaves a checksum of it, so that nothing can be optimised away and the caller can verify
// that the work was done.
#include "attn_probe.h"

#include "common.h"

namespace {

constexpr int kThreads = ATTN_PROBE_THREADS;
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Two accumulation chains per wave on blocks of ones times blocks of twos (A and B in
// distinct registers): a chain's next product issues one product after its last one.
// Measured against other forms of the same loop: four chains, or one register feeding both
// operands, lose 9-12% of the rate.
template <bool kFp8>
__global__ __launch_bounds__(kThreads, 2) void probe_mfma_kernel(int iters, float* __restrict__ out) {
  floatx16 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  if constexpr (kFp8) {
    const intx8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
    const intx8 twos = {0x40404040, 0x40404040, 0x40404040, 0x40404040,
                        0x40404040, 0x40404040, 0x40404040, 0x40404040};  // E4M3 2.0
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, twos, acc[c], 0, 0, 0, 0, 0, 0);
  } else {
    bf16x8 ones, twos;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ones[e] = (bf16)1.0f;
      twos[e] = (bf16)2.0f;
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, twos, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = s;
}

// Eight independent chains x <- 2^(-x) per lane: one v_exp_f32 per step (the negation is an
// input modifier of the instruction).
__global__ __launch_bounds__(kThreads) void probe_exp_kernel(int iters, float* __restrict__ out) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.5f + 0.01f * j;
  for (int i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

__device__ __forceinline__ uint32_t word_sum(u32x4 a) { return a.x + a.y + a.z + a.w; }

// Streaming read: lane i of the grid reads 16-byte chunks i, i + S, i + 2S, ... (S = the
// grid's thread count), four in flight, marked non-temporal (read once).
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* __restrict__ src,
                                                              size_t n16, uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t s = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    s += word_sum(a) + word_sum(b) + word_sum(c) + word_sum(d);
  }
  for (; i < n16; i += stride) s += word_sum(__builtin_nontemporal_load(src + i));
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Paged read: each wave takes pages p, p + W, ... of `order` (W = the grid's wave count),
// two pages in flight, each page four 1 KiB loads (lane l reads bytes 16 l .. 16 l + 15 of
// each KiB).
__global__ __launch_bounds__(kThreads) void probe_read_pages_kernel(
    const u32x4* __restrict__ pool, int pool_pages, const int32_t* __restrict__ order,
    int n_pages, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int n_waves = gridDim.x * (kThreads / 64);
  auto page = [&](int p) {
    const int g = min(max(order[p], 0), pool_pages - 1);
    return pool + (size_t)g * 256;  // 4096 bytes = 256 chunks of 16
  };
  uint32_t s = 0;
  int p = wave;
  for (; p + n_waves < n_pages; p += 2 * n_waves) {
    const u32x4* a = page(p);
    const u32x4* b = page(p + n_waves);
    u32x4 x[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = __builtin_nontemporal_load(a + 64 * k + lane);
      x[4 + k] = __builtin_nontemporal_load(b + 64 * k + lane);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) s += word_sum(x[k]);
  }
  if (p < n_pages) {
    const u32x4* a = page(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) s += word_sum(__builtin_nontemporal_load(a + 64 * k + lane));
  }
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

attn_status launched() { return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH; }

constexpr int kMaxBlocks = 1 << 24;  // keeps every output index within 32 bits
bool bad_blocks(int blocks) { return blocks <= 0 || blocks > kMaxBlocks; }

}  // namespace

extern "C" {

attn_status attn_probe_mfma(int fp8, int blocks, int iters, float* out, void* stream) {
  if (!out || bad_blocks(blocks) || iters <= 0 || iters > 16384 || (fp8 != 0 && fp8 != 1))
    return ATTN_ERR_INVALID;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (fp8)
    hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, iters, out);
  return launched();
}

attn_status attn_probe_exp(int blocks, int iters, float* out, void* stream) {
  if (!out || bad_blocks(blocks) || iters <= 0) return ATTN_ERR_INVALID;
  hipLaunchKernelGGL(probe_exp_kernel, dim3(blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, out);
  return launched();
}

attn_status attn_probe_read(const void* src, size_t bytes, int blocks, uint32_t* out,
                            void* stream) {
  if (!src || !out || bytes == 0 || bytes % 4096 != 0 || bad_blocks(blocks)) return ATTN_ERR_INVALID;
  hipLaunchKernelGGL(probe_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, out);
  return launched();
}

attn_status attn_probe_read_pages(const void* pool, int pool_pages, const int32_t* order,
                                  int n_pages, int blocks, uint32_t* out, void* stream) {
  if (!pool || !order || !out || pool_pages <= 0 || n_pages <= 0 || bad_blocks(blocks))
    return ATTN_ERR_INVALID;
  hipLaunchKernelGGL(probe_read_pages_kernel, dim3(blocks), dim3(kThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(pool),
                     pool_pages, order, n_pages, out);
  return launched();
}

}  // extern "C"
