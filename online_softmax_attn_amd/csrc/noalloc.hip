// attn_decode_paged_noalloc: the paged decode without a caller workspace, for callers that
// cannot allocate device memory (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The split partials go to `scratch`, a fixed device array the
// library holds on every GPU it runs on until the process ends.  Nothing is allocated or
// freed here.  Calls on one GPU share that GPU's array: calls that overlap in time on one GPU
// race on it and must be serialised by the caller.
#include <mutex>

#include "attn.h"
#include "common.h"

// One copy per GPU.  In host code this name is only a stand-in for the symbol: its device
// address is looked up per device below and only that address is ever used.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_lookup[kMaxDevices];

// Device address of `scratch` on `dev`, looked up once per device with that device current.
void* scratch_address(int dev) {
  std::call_once(g_once[dev], [dev] {
    int prev = -1;
    g_lookup[dev] = hipGetDevice(&prev);
    if (g_lookup[dev] != hipSuccess) return;
    if (prev != dev && (g_lookup[dev] = hipSetDevice(dev)) != hipSuccess) return;
    void* p = nullptr;
    g_lookup[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
    if (prev != dev) {
      const hipError_t e = hipSetDevice(prev);
      if (g_lookup[dev] == hipSuccess) g_lookup[dev] = e;
    }
  });
  return g_lookup[dev] == hipSuccess ? g_scratch[dev] : nullptr;
}

}  // namespace

extern "C" attn_status attn_decode_paged_noalloc(
    attn_dtype dtype, const void* q, const void* k_cache, const void* v_cache,
    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, int batch,
    int heads, int kv_heads, int head_dim, int block_size, int num_blocks,
    int max_blocks_per_seq, int max_seq_len, int window, float scale, int kv_split,
    void* stream) {
  // every argument check of attn_decode_paged, before any runtime call
  int split = 0;
  size_t need = 0;
  const attn_status st = decode_paged_check(dtype, q, k_cache, v_cache, block_table, seq_lens,
                                            o, batch, heads, kv_heads, head_dim, block_size,
                                            num_blocks, max_blocks_per_seq, max_seq_len, window,
                                            scale, kv_split, &split, &need);
  if (st != ATTN_OK) return st;
  if (need > ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
  // the kernels run on the stream's device; the null stream means the current device
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = -1;
  if ((s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev)) != hipSuccess) return ATTN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  void* ws = scratch_address(dev);
  if (!ws) return ATTN_ERR_LAUNCH;
  const hipError_t e = launch_decode_paged(
      static_cast<const bf16*>(q), static_cast<const bf16*>(k_cache),
      static_cast<const bf16*>(v_cache), block_table, seq_lens, static_cast<bf16*>(o), lse,
      batch, heads, kv_heads, num_blocks, max_blocks_per_seq, max_seq_len, window, scale, split,
      ws, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
