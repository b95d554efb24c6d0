// Host-side check of the C ABI layer (online_softmax_attn_amd/csrc/api.hip) built with the
// address and undefined-behaviour sanitizers and with stand-in launchers (stubs.cpp): every
// entry point is called with invalid, unsupported, extreme and valid host arguments; a
// rejected call must return its status without reaching a launcher, an accepted one must
// reach exactly one launcher with the derived arguments, and no call may overflow or touch
// memory it does not own.  Device pointers are a fixed non-null value that nothing
// dereferences.  Exit status 0 when every case holds.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "attn.h"
#include "stubs.h"

namespace {

int g_cases = 0, g_failures = 0;

void expect(bool ok, int line, const char* what) {
  ++g_cases;
  if (!ok) {
    ++g_failures;
    std::printf("FAIL line %d: %s\n", line, what);
  }
}
#define EXPECT(cond) expect((cond), __LINE__, #cond)

void* const P = reinterpret_cast<void*>(uintptr_t{0x10000});
float* const PF = reinterpret_cast<float*>(uintptr_t{0x10000});
const int32_t* const PI = reinterpret_cast<const int32_t*>(uintptr_t{0x10000});
const float kNaN = std::nanf("");
const float kInf = INFINITY;

// a call that must be rejected with `want` without reaching a launcher
#define REJECT(call, want)                            \
  do {                                                \
    const int before = g_log.calls;                   \
    const attn_status got = (call);                   \
    EXPECT(got == (want));                            \
    EXPECT(g_log.calls == before);                    \
  } while (0)

// a call that must succeed by reaching the launcher `name` once
#define ACCEPT(call, name)                            \
  do {                                                \
    const int before = g_log.calls;                   \
    const attn_status got = (call);                   \
    EXPECT(got == ATTN_OK);                           \
    EXPECT(g_log.calls == before + 1);                \
    EXPECT(std::strcmp(g_log.last, (name)) == 0);     \
  } while (0)

struct Fwd {
  int dtype = ATTN_BF16;
  void *q = P, *k = P, *v = P, *o = P;
  int B = 1, H = 1, Hkv = 1, n = 16, d = 128, causal = 0, window = 0;
  float scale = 0.1f;
};
attn_status fwd(Fwd a) {
  return attn_fwd((attn_dtype)a.dtype, a.q, a.k, a.v, a.o, nullptr, nullptr, a.B, a.H, a.Hkv,
                  a.n, a.d, a.causal, a.window, a.scale, nullptr);
}

void check_fwd() {
  Fwd a;
  ACCEPT(fwd(a), "fwd_bf16");
  EXPECT(g_log.n == 16 && g_log.n_kv == 16 && g_log.q_start == 0 && g_log.head_dim == 128);
  Fwd f32;
  f32.dtype = ATTN_F32;
  f32.d = 64;
  ACCEPT(fwd(f32), "fwd_f32");
  Fwd w;
  w.H = 4, w.Hkv = 2, w.causal = 1, w.window = 8;
  ACCEPT(fwd(w), "fwd_bf16");
  for (int i = 0; i < 4; ++i) {
    Fwd x;
    (i == 0 ? x.q : i == 1 ? x.k : i == 2 ? x.v : x.o) = nullptr;
    REJECT(fwd(x), ATTN_ERR_INVALID);
  }
  const int bad_sizes[][4] = {{0, 1, 16, 128}, {1, -1, 16, 128}, {1, 1, 0, 128}, {1, 1, 16, 0},
                              {INT_MIN, 1, 16, 128}, {1, 1, INT_MIN, 128}};
  for (const auto& s : bad_sizes) {
    Fwd x;
    x.B = s[0], x.H = s[1], x.n = s[2], x.d = s[3];
    REJECT(fwd(x), ATTN_ERR_INVALID);
  }
  for (float sc : {0.f, -1.f, kNaN, kInf, -kInf}) {
    Fwd x;
    x.scale = sc;
    REJECT(fwd(x), ATTN_ERR_INVALID);
  }
  const int bad_heads[][2] = {{1, 0}, {4, 3}, {4, 8}, {4, -2}, {INT_MIN, -1}};
  for (const auto& h : bad_heads) {
    Fwd x;
    x.H = h[0], x.Hkv = h[1];
    REJECT(fwd(x), ATTN_ERR_INVALID);
  }
  Fwd wn;
  wn.window = -1, wn.causal = 1;
  REJECT(fwd(wn), ATTN_ERR_INVALID);
  Fwd wc;
  wc.window = 8;
  REJECT(fwd(wc), ATTN_ERR_INVALID);
  Fwd d96;
  d96.d = 96;
  REJECT(fwd(d96), ATTN_ERR_UNSUPPORTED);
  Fwd dt;
  dt.dtype = 7;
  REJECT(fwd(dt), ATTN_ERR_UNSUPPORTED);
  Fwd b64;
  b64.d = 64;
  ACCEPT(fwd(b64), "fwd_bf16");
  EXPECT(g_log.head_dim == 64);
  Fwd b32;
  b32.d = 32;
  REJECT(fwd(b32), ATTN_ERR_UNSUPPORTED);
  // extremes: every size product must be formed without overflow
  Fwd e1;
  e1.n = INT_MAX;
  REJECT(fwd(e1), ATTN_ERR_UNSUPPORTED);
  Fwd e2;
  e2.B = INT_MAX, e2.H = INT_MAX, e2.Hkv = INT_MAX, e2.n = 1 << 22;
  REJECT(fwd(e2), ATTN_ERR_UNSUPPORTED);
  Fwd e3;
  e3.dtype = ATTN_F32, e3.n = INT_MAX, e3.d = INT_MAX;
  REJECT(fwd(e3), ATTN_ERR_UNSUPPORTED);
  Fwd e4;
  e4.dtype = ATTN_F32, e4.d = 64, e4.B = 256, e4.H = 256, e4.Hkv = 256;
  REJECT(fwd(e4), ATTN_ERR_UNSUPPORTED);
  // a launch the runtime refuses
  g_log.fail_launch = true;
  const int before = g_log.calls;
  EXPECT(fwd(Fwd{}) == ATTN_ERR_LAUNCH);
  EXPECT(g_log.calls == before + 1);
  g_log.fail_launch = false;
}

attn_status chunk(int q_len, int kv_len, int q_start, int dtype = ATTN_BF16) {
  return attn_fwd_chunk((attn_dtype)dtype, P, P, P, P, nullptr, 1, 2, 2, q_len, kv_len, q_start,
                        128, 1, 0, 0.1f, nullptr);
}

void check_chunk() {
  ACCEPT(chunk(16, 64, 48), "fwd_bf16");
  EXPECT(g_log.n == 16 && g_log.n_kv == 64 && g_log.q_start == 48);
  REJECT(chunk(16, 64, 49), ATTN_ERR_INVALID);
  REJECT(chunk(16, 64, -1), ATTN_ERR_INVALID);
  REJECT(chunk(INT_MAX, INT_MAX, INT_MAX), ATTN_ERR_INVALID);
  REJECT(chunk(0, 64, 0), ATTN_ERR_INVALID);
  REJECT(chunk(16, 64, 0, ATTN_F32), ATTN_ERR_UNSUPPORTED);
  REJECT(chunk(1, INT_MAX, 0), ATTN_ERR_UNSUPPORTED);
}

attn_status bwd(int B, int H, int n, void* ws, size_t wsb, int dtype = ATTN_BF16, int d = 128) {
  return attn_bwd((attn_dtype)dtype, P, P, P, P, P, PF, nullptr, PF, PF, PF, B, H, H, n, d, 1, 0,
                  0.1f, ws, wsb, nullptr);
}

void check_bwd() {
  const size_t need = attn_bwd_workspace_bytes(2, 4, 100);
  EXPECT(need == 2u * 4u * 100u * 4u);
  ACCEPT(bwd(2, 4, 100, P, need), "bwd_bf16");
  REJECT(bwd(2, 4, 100, nullptr, need), ATTN_ERR_WORKSPACE);
  REJECT(bwd(2, 4, 100, P, need - 1), ATTN_ERR_WORKSPACE);
  REJECT(bwd(2, 4, 100, P, need, ATTN_F32), ATTN_ERR_UNSUPPORTED);
  REJECT(bwd(2, 4, 100, P, need, ATTN_BF16, 64), ATTN_ERR_UNSUPPORTED);
  REJECT(bwd(0, 4, 100, P, need), ATTN_ERR_INVALID);
  REJECT(bwd(INT_MAX, INT_MAX, 1 << 20, P, SIZE_MAX), ATTN_ERR_UNSUPPORTED);
  REJECT(bwd(1, 1, INT_MAX, P, SIZE_MAX), ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX) == 0);
  EXPECT(attn_bwd_workspace_bytes(0, 1, 1) == 0);
  EXPECT(attn_bwd_workspace_bytes(1, 1, -5) == 0);
}

struct Dec {
  int dtype = ATTN_BF16, B = 2, H = 4, Hkv = 4, d = 128, bs = 16, nb = 10, mb = 8, msl = 128;
  int window = 0, split = 0;
  float scale = 0.1f;
  void* ws = P;
  size_t wsb = size_t{1} << 30;
};
attn_status dec(Dec a) {
  return attn_decode_paged((attn_dtype)a.dtype, P, P, P, PI, PI, P, nullptr, a.B, a.H, a.Hkv,
                           a.d, a.bs, a.nb, a.mb, a.msl, a.window, a.scale, a.split, a.ws, a.wsb,
                           nullptr);
}

void check_decode() {
  Dec a;
  ACCEPT(dec(a), "decode_paged");
  EXPECT(g_log.split == 64);  // too few waves for longer splits
  Dec s32;
  s32.split = 32;
  ACCEPT(dec(s32), "decode_paged");
  EXPECT(g_log.split == 32);
  Dec g8;
  g8.H = 64, g8.Hkv = 8, g8.msl = 8192, g8.mb = 512, g8.B = 32;
  ACCEPT(dec(g8), "decode_paged");
  const size_t need = attn_decode_workspace_bytes(32, 64, 8, 128, 8192, 0, 0);
  EXPECT(need > 0);
  Dec small = g8;
  small.wsb = need - 1;
  REJECT(dec(small), ATTN_ERR_WORKSPACE);
  Dec nows;
  nows.ws = nullptr;
  REJECT(dec(nows), ATTN_ERR_WORKSPACE);
  for (int sp : {20, -16, 2048}) {
    Dec x;
    x.split = sp;
    REJECT(dec(x), ATTN_ERR_INVALID);
  }
  Dec bs32;
  bs32.bs = 32;
  REJECT(dec(bs32), ATTN_ERR_UNSUPPORTED);
  Dec shortt;
  shortt.mb = 7;  // 7 * 16 < 128
  REJECT(dec(shortt), ATTN_ERR_INVALID);
  Dec f32;
  f32.dtype = ATTN_F32;
  REJECT(dec(f32), ATTN_ERR_UNSUPPORTED);
  Dec big;
  big.B = 65536;
  REJECT(dec(big), ATTN_ERR_UNSUPPORTED);
  // extremes: partial sizes past size_t are refused, not wrapped
  Dec huge;
  huge.B = 65535, huge.H = 65535, huge.Hkv = 65535, huge.msl = INT_MAX,
  huge.mb = INT_MAX / 16 + 1, huge.split = 64, huge.wsb = SIZE_MAX;
  REJECT(dec(huge), ATTN_ERR_UNSUPPORTED);
  EXPECT(attn_decode_workspace_bytes(65535, 65535, 65535, 128, INT_MAX, 0, 64) == 0);
  EXPECT(attn_decode_workspace_bytes(65536, 1, 1, 128, 128, 0, 0) == 0);
  EXPECT(attn_decode_workspace_bytes(2, 4, 3, 128, 128, 0, 0) == 0);
  EXPECT(attn_decode_workspace_bytes(2, 4, 4, 128, INT_MAX, INT_MAX, 0) > 0);
}

void check_fp8_and_merge() {
  ACCEPT(attn_quantize_fp8(P, P, PF, nullptr, 2, 4, 100, 128, 0, nullptr), "quantize_fp8");
  REJECT(attn_quantize_fp8(P, P, PF, nullptr, 256, 256, 100, 128, 0, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_quantize_fp8(P, P, PF, nullptr, 2, 4, 100, 64, 0, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_quantize_fp8(nullptr, P, PF, nullptr, 2, 4, 100, 128, 0, nullptr), ATTN_ERR_INVALID);
  ACCEPT(attn_fwd_fp8(P, P, P, PF, PF, PF, P, nullptr, nullptr, 2, 4, 4, 100, 128, 1, 0.1f, nullptr),
         "fwd_fp8");
  REJECT(attn_fwd_fp8(P, P, P, PF, PF, PF, P, nullptr, nullptr, 2, 4, 4, INT_MAX, 128, 1, 0.1f, nullptr),
         ATTN_ERR_UNSUPPORTED);
  REJECT(attn_fwd_fp8(P, P, P, PF, PF, PF, P, nullptr, nullptr, INT_MAX, INT_MAX, 1, 1 << 20, 128, 1,
                      0.1f, nullptr),
         ATTN_ERR_UNSUPPORTED);
  REJECT(attn_fwd_fp8(P, P, P, nullptr, PF, PF, P, nullptr, nullptr, 2, 4, 4, 100, 128, 1, 0.1f, nullptr),
         ATTN_ERR_INVALID);
  ACCEPT(attn_merge(ATTN_BF16, P, PF, P, nullptr, 4, 1000, 128, nullptr), "merge");
  REJECT(attn_merge(ATTN_BF16, P, PF, P, nullptr, 4, INT64_MAX, 128, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_merge(ATTN_BF16, P, PF, P, nullptr, 1025, 1000, 128, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_merge(ATTN_F32, P, PF, P, nullptr, 4, 1000, 96, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_merge((attn_dtype)7, P, PF, P, nullptr, 4, 1000, 128, nullptr), ATTN_ERR_UNSUPPORTED);
  REJECT(attn_merge(ATTN_BF16, P, PF, P, nullptr, 0, 1000, 128, nullptr), ATTN_ERR_INVALID);
  REJECT(attn_merge(ATTN_BF16, P, PF, P, nullptr, 4, INT64_MIN, 128, nullptr), ATTN_ERR_INVALID);
}

void check_misc() {
  EXPECT(attn_abi_version() == ATTN_ABI_VERSION);
  EXPECT(std::strcmp(attn_status_str(ATTN_OK), "ATTN_OK") == 0);
  EXPECT(std::strcmp(attn_status_str(ATTN_ERR_LAUNCH), "ATTN_ERR_LAUNCH") == 0);
  EXPECT(std::strcmp(attn_status_str((attn_status)99), "ATTN_ERR_UNKNOWN") == 0);
  EXPECT(std::strcmp(attn_status_str((attn_status)-1), "ATTN_ERR_UNKNOWN") == 0);
}

}  // namespace

int main() {
  check_fwd();
  check_chunk();
  check_bwd();
  check_decode();
  check_fp8_and_merge();
  check_misc();
  std::printf("host check: %d cases, %d failures\n", g_cases, g_failures);
  return g_failures == 0 ? 0 : 1;
}
