// paged_attn_decode for callers that cannot allocate device memory: the same
// path with its workspace (plan and partials) in a fixed device array of this
// library, one per GPU, instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"
#include "pagedattn.h"

namespace {

// The fixed workspace. In host code its name is only a handle for
// hipGetSymbolAddress; kernels get the per-device address looked up below.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of `scratch` on device `dev`: looked up once per device with that
// device current (each device holds its own copy at its own address).
int scratch_on(int dev, void **ptr) {
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return PA_ERR_LAUNCH;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return PA_ERR_LAUNCH;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress((void **)&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) return PA_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" int paged_attn_decode_noalloc(
    const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_query_tokens,
    int32_t num_q_heads, int32_t head_dim, const void *k_cache, const void *v_cache,
    const float *k_scale, const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
    int32_t num_kv_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *context_lens, const int32_t *query_start, int32_t max_context_len,
    int32_t sliding_window, float scale, int32_t split_tokens, void *out, hipStream_t stream) {
  size_t need = 0;
  const int st = pa::decode_workspace_need(
      q, q_dtype, num_seqs, num_query_tokens, num_q_heads, head_dim, k_cache, v_cache, k_scale,
      v_scale, cache_dtype, num_blocks, num_kv_heads, block_tables, max_blocks_per_seq,
      context_lens, query_start, max_context_len, sliding_window, split_tokens, out, &need);
  if (st != PA_OK || need == 0) return st;
  if (need > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_SCRATCH;
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return PA_ERR_LAUNCH;
  void *ws = nullptr;
  const int sst = scratch_on(dev, &ws);
  if (sst != PA_OK) return sst;
  return paged_attn_decode(q, q_dtype, num_seqs, num_query_tokens, num_q_heads, head_dim,
                           k_cache, v_cache, k_scale, v_scale, cache_dtype, num_blocks,
                           num_kv_heads, block_tables, max_blocks_per_seq, context_lens,
                           query_start, max_context_len, sliding_window, scale, split_tokens,
                           out, ws, PA_NOALLOC_SCRATCH_BYTES, stream);
}
