// Block quantisation of bf16 [B, H, n, 128] tensors to FP8 E4M3 on gfx950.
//
// pierluigilucio.it "Sviluppo AI ed Algebra Lineare", FP8 part on FlashAttention-3, section
// "Quantizzazione a Blocchi e Scaling Algebrico": a block X of rows gets the scale s = max|X| / 448 (448 = the largest E4M3
// magnitude) and the codes clip(round(X / s), -448, 448).  Blocks are 64 rows of one
// (batch, head); rows at or past the sequence length count as 0 and are written as code 0;
// a block with max|X| = 0 has s = 0 and codes 0.  X / s is a correctly rounded fp32
// division and the rounding to E4M3 is v_cvt_pk_fp8_f32 (nearest, ties to even, OCP E4M3
// codes), so every code is a function of the bf16 input alone.
//
// Output layouts: row-major [B, H, n, 128] bytes (Q and K), or transposed per (batch, head)
// [128][n_pad] with n_pad = 64 * ceil(n / 64) (V: the layout the P.V product reads, one
// row of keys per dimension); the padding columns are written as 0.
#include "common.h"

namespace {

constexpr int kD = 128;
constexpr int kRows = 64;
constexpr int kThreads = 256;  // each thread: one row, 32 dims

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__global__ __launch_bounds__(kThreads) void quantize_fp8_kernel(
    const bf16* __restrict__ X, uint8_t* __restrict__ X8, float* __restrict__ scales,
    const int32_t* __restrict__ lens, int H, int n, int n_blocks, int transpose) {
  __shared__ float wave_max[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kRows][kD + 16];  // +16: stagger rows

  const int blk = blockIdx.x;               // block within the (batch, head)
  const long long bh = blockIdx.y;
  const int b = (int)(bh / H);
  int L = lens ? lens[b] : n;
  L = L < 0 ? 0 : (L > n ? n : L);
  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;    // row within the block, 32-dim quarter
  const int row = blk * kRows + r;
  const bool live = row < L;

  float x[32];
  if (live) {
    const uint4* src = reinterpret_cast<const uint4*>(X + (bh * n + row) * kD + 32 * part);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 w = src[i];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * i + 2 * e] = bf16_to_f32((uint16_t)(ws[e] & 0xffff));
        x[8 * i + 2 * e + 1] = bf16_to_f32((uint16_t)(ws[e] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.f;
  }

  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) mx = __builtin_fmaxf(mx, __builtin_fabsf(x[i]));
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = __builtin_fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) wave_max[tid >> 6] = mx;
  __syncthreads();
  mx = __builtin_fmaxf(__builtin_fmaxf(wave_max[0], wave_max[1]), __builtin_fmaxf(wave_max[2], wave_max[3]));
  const float s = __fdiv_rn(mx, 448.0f);
  if (tid == 0) scales[bh * n_blocks + blk] = s;

  uint32_t codes[8];  // 32 codes, 4 per word, in dimension order
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q = s > 0.f ? __fdiv_rn(x[4 * i + e], s) : 0.f;
      y[e] = __builtin_fminf(__builtin_fmaxf(q, -448.0f), 448.0f);
    }
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
    codes[i] = (uint32_t)w;
  }

  if (!transpose) {
    if (row < n) {
      uint4* dst = reinterpret_cast<uint4*>(X8 + (bh * n + row) * kD + 32 * part);
      dst[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
      dst[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
    }
    return;
  }
  // transposed: stage the 64 x 128 block in LDS, then write 128 rows of 64 keys
  uint4* trow = reinterpret_cast<uint4*>(&tile[r][32 * part]);
  trow[0] = make_uint4(codes[0], codes[1], codes[2], codes[3]);
  trow[1] = make_uint4(codes[4], codes[5], codes[6], codes[7]);
  __syncthreads();
  const long long n_pad = (long long)n_blocks * kRows;
  const int dim = tid >> 1, half = tid & 1;  // 32 keys of one dimension
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= (uint32_t)tile[32 * half + 4 * i + e][dim] << (8 * e);
    out[i] = w;
  }
  uint4* dst = reinterpret_cast<uint4*>(X8 + (bh * kD + dim) * n_pad + (long long)blk * kRows + 32 * half);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

}  // namespace

hipError_t launch_quantize_fp8(const bf16* x, uint8_t* x8, float* scales, const int32_t* seq_lens,
                               int batch, int heads, int n, int transpose, hipStream_t stream) {
  const int n_blocks = (n + kRows - 1) / kRows;
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(n_blocks, batch * heads), dim3(kThreads), 0, stream,
                     x, x8, scales, seq_lens, heads, n, n_blocks, transpose);
  return hipGetLastError();
}
