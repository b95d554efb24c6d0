// Stand-ins for the kernel launchers (common.h) in the host-only build of the C ABI layer:
// each records that it was reached and with which derived arguments, and enqueues nothing.
// The layer's contract is that a launcher is reached only with validated arguments.
#include "common.h"
#include "stubs.h"

HostCheckLog g_log;

static hipError_t reached(const char* name) {
  g_log.calls += 1;
  g_log.last = name;
  return g_log.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

hipError_t launch_fwd_f32(const float*, const float*, const float*, float*, float*, const int32_t*,
                          int, int, int, int, int, int, int, float, hipStream_t) {
  return reached("fwd_f32");
}
hipError_t launch_fwd_bf16(const bf16*, const bf16*, const bf16*, bf16*, float*, const int32_t*,
                           int, int, int, int n, int n_kv, int q_start, int head_dim, int, int,
                           float, hipStream_t) {
  g_log.n = n;
  g_log.n_kv = n_kv;
  g_log.q_start = q_start;
  g_log.head_dim = head_dim;
  return reached("fwd_bf16");
}
hipError_t launch_bwd_bf16(const bf16*, const bf16*, const bf16*, const bf16*, const bf16*,
                           const float*, const int32_t*, float*, float*, float*, int, int, int,
                           int, int, int, float, void*, hipStream_t) {
  return reached("bwd_bf16");
}
hipError_t launch_decode_paged(const bf16*, const bf16*, const bf16*, const int32_t*,
                               const int32_t*, bf16*, float*, int, int, int, int, int, int, int,
                               float, int split, void*, hipStream_t) {
  g_log.split = split;
  return reached("decode_paged");
}
hipError_t launch_decode_gqa(const bf16*, const bf16*, const bf16*, const int32_t*,
                             const int32_t*, int, int, int, int, int, int, int, float, int, int,
                             void*, size_t, hipStream_t) {
  return reached("decode_gqa");
}
hipError_t launch_quantize_fp8(const bf16*, uint8_t*, float*, const int32_t*, int, int, int, int,
                               hipStream_t) {
  return reached("quantize_fp8");
}
hipError_t launch_fwd_fp8(const uint8_t*, const uint8_t*, const uint8_t*, const float*,
                          const float*, const float*, bf16*, float*, const int32_t*, int, int,
                          int, int, int, float, hipStream_t) {
  return reached("fwd_fp8");
}
hipError_t launch_merge(bool, const void*, const float*, void*, float*, int, long long, int,
                        hipStream_t) {
  return reached("merge");
}
