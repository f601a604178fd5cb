// C ABI of libpagedattn: argument checks, launch planning and dispatch.
// The operations and their conventions are documented in include/pagedattn.h.
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "pa_internal.h"
#include "pagedattn.h"

namespace {

bool misaligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) != 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// Caches of 8-bit codes with per-(token, KV head) scales.
bool quantised(int32_t cache_dtype) { return cache_dtype == PA_I8 || cache_dtype == PA_FP8; }

int check_split_tokens(int32_t split_tokens) {
  if (split_tokens <= 0 || split_tokens % PA_BLOCK_SIZE != 0 || split_tokens > PA_MAX_SPLIT_TOKENS)
    return PA_ERR_SPLIT;
  return PA_OK;
}

bool bad_query_shape(int32_t num_query_tokens, int32_t sliding_window) {
  return num_query_tokens < 1 || num_query_tokens > PA_MAX_QUERY_TOKENS || sliding_window < 0;
}

// Query counts: Q per sequence, or (packed) the total N of all sequences.
bool bad_queries(bool packed, int32_t num_query_tokens, int32_t sliding_window) {
  if (!packed) return bad_query_shape(num_query_tokens, sliding_window);
  return num_query_tokens < 0 || num_query_tokens > PA_MAX_PACKED_QUERY_TOKENS ||
         sliding_window < 0;
}

// Largest query count of one sequence: Q, or at most min(N, PA_MAX_QUERY_TOKENS).
int32_t query_bound(bool packed, int32_t num_query_tokens) {
  return packed ? std::max(1, std::min(num_query_tokens, PA_MAX_QUERY_TOKENS)) : num_query_tokens;
}

// Query count the default split size is chosen for: Q, or with packed
// queries the mean count per sequence.
int32_t query_for_default(bool packed, int32_t num_query_tokens, int32_t num_seqs) {
  if (!packed) return num_query_tokens;
  const int64_t mean = ((int64_t)num_query_tokens + std::max(num_seqs, 1) - 1) /
                       std::max(num_seqs, 1);
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(mean, PA_MAX_QUERY_TOKENS));
}

// Entries the plan lists at most: one per split of each sequence, or with
// packed queries one per (split, block of 64 query rows) of each sequence
// (sum over s of ceil(Q_s*g/64) <= num_seqs + ceil(N*g/64)).
int64_t plan_capacity(int32_t num_seqs, int32_t max_splits, bool packed, int32_t num_query_tokens,
                      int32_t g) {
  const int64_t per_split =
      packed ? (int64_t)num_seqs + ((int64_t)num_query_tokens * g + pa::kPackedRows - 1) /
                                       pa::kPackedRows
             : num_seqs;
  return per_split * std::max(max_splits, 1);
}

int launch_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

// The length bound the kernels clamp every context length to.
int32_t clamped_bound(int32_t max_context_len, int32_t max_blocks_per_seq) {
  return (int32_t)std::min<int64_t>(max_context_len, (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE);
}

constexpr int32_t kMinDefaultSplit = 64;  // smallest split the default picks
constexpr int64_t kMinWorkItems = 1024;   // (split, KV head) items the default aims for
constexpr int64_t kGrowWorkItems = 2048;  // items a decode step keeps when its splits grow
constexpr int64_t kGrowMaxBytes = 1 << 20;  // K/V bytes per (split, KV head) growth stops at
constexpr int32_t kGrowStep = 64;           // tokens a decode step's split grows by

}  // namespace

namespace pa {

int compute_units(hipStream_t stream) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> known[kMaxDevices];  // a device property, looked up once
  int dev = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) {
    (void)hipGetLastError();
    if (hipGetDevice(&dev) != hipSuccess) (void)hipGetLastError();
  }
  if (dev >= 0 && dev < kMaxDevices) {
    const int v = known[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                     hipSuccess) {
    (void)hipGetLastError();
    n = 0;
  }
  n = std::max(n, 1);
  if (dev >= 0 && dev < kMaxDevices) known[dev].store(n, std::memory_order_relaxed);
  return n;
}

int trace_level() {
  static const int level = [] {
    const char *e = getenv("PAGEDATTN_TRACE");
    return e ? atoi(e) : 0;
  }();
  return level;
}

void trace(const char *fmt, ...) {
  if (trace_level() <= 0) return;
  char line[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(line, sizeof line, fmt, ap);
  va_end(ap);
  fprintf(stderr, "[pagedattn] %s\n", line);
}

const char *dtype_name(int dtype) {
  switch (dtype) {
    case PA_F32: return "f32";
    case PA_BF16: return "bf16";
    case PA_I8: return "int8";
    case PA_FP8: return "fp8";
    default: return "?";
  }
}

// Trace level 2: wait for the plan just launched on `stream` and print its
// list (header, group entries, the first entries). Reads through fixed stack
// buffers: nothing is allocated.
void trace_plan(const int32_t *sched, int64_t capacity, hipStream_t stream) {
  if (trace_level() < 2) return;
  int32_t head[kSchedHeader];
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(head, sched, sizeof head, hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    trace("plan: could not be read back");
    return;
  }
  const int64_t n = std::min<int64_t>(head[0], capacity);
  constexpr int kChunk = 1024;
  int32_t buf[2 * kChunk];
  int64_t groups = 0;
  char first[256] = "";
  int used = 0;
  for (int64_t i0 = 0; i0 < n; i0 += kChunk) {
    const int64_t cnt = std::min<int64_t>(kChunk, n - i0);
    if (hipMemcpy(buf, sched + kSchedHeader + 2 * i0, (size_t)cnt * 2 * sizeof(int32_t),
                  hipMemcpyDeviceToHost) != hipSuccess) {
      (void)hipGetLastError();
      trace("plan: could not be read back");
      return;
    }
    for (int64_t i = 0; i < cnt; ++i) {
      if (buf[2 * i + 1] < 0 && head[6] > 1) ++groups;
      if (i0 + i < 6 && used < (int)sizeof first - 48)
        used += snprintf(first + used, sizeof first - used, " (s %u, j %u, %d)",
                         (uint32_t)buf[2 * i] >> 16, (uint32_t)buf[2 * i] & 0xffffu,
                         buf[2 * i + 1]);
    }
  }
  trace("plan: %lld entries (%lld group entries of up to %d sequences), split %d tokens, %d "
        "sequences, length bound %d, %d query tokens, window %d; first:%s",
        (long long)n, (long long)groups, head[6], head[1], head[2], head[3], head[4], head[5],
        first);
}

int resident_per_cu(const void *kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) {
    (void)hipGetLastError();
    n = 1;
  }
  return std::max(n, 1);
}

}  // namespace pa

extern "C" {

const char *pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case PA_ERR_SHAPE: return "unsupported sizes (head_dim 64/128, Hq/Hkv in {1,2,4,8,16}, 1..4096 query tokens per sequence, window >= 0, counts >= 0)";
    case PA_ERR_SPLIT: return "split_tokens must be a positive multiple of 16 up to 4096, and max_splits must cover the longest split range";
    case PA_ERR_WORKSPACE: return "workspace smaller than pa_workspace_bytes()";
    case PA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case PA_ERR_LAUNCH: return "kernel launch failed (or the device's fixed scratch could not be set up)";
    case PA_ERR_SCRATCH: return "the call needs more than the library's fixed scratch (PA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t pa_num_splits(int32_t context_len, int32_t split_tokens) {
  if (split_tokens <= 0) return 0;
  if (context_len <= 0) return 1;
  const int64_t n = ((int64_t)context_len + split_tokens - 1) / split_tokens;
  return (int32_t)(n < 1 ? 1 : n);
}

int32_t pa_max_splits(int32_t max_context_len, int32_t num_query_tokens, int32_t sliding_window,
                      int32_t split_tokens) {
  if (split_tokens <= 0 || bad_query_shape(num_query_tokens, sliding_window)) return 0;
  return pa_num_splits(pa::max_span(std::max(max_context_len, 0), num_query_tokens, sliding_window),
                       split_tokens);
}

int32_t pa_default_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t cache_dtype, int32_t max_context_len,
                                int32_t num_query_tokens, int32_t sliding_window) {
  int elt;
  switch (cache_dtype) {
    case PA_F32: elt = 4; break;
    case PA_BF16: elt = 2; break;
    case PA_I8:
    case PA_FP8: elt = 1; break;
    default: return 0;
  }
  if (head_dim != 64 && head_dim != 128) return 0;
  if (bad_query_shape(num_query_tokens, sliding_window)) return 0;
  if (num_kv_heads <= 0 || num_q_heads < num_kv_heads) return 0;
  // 256 KiB of K and V codes per (split, KV head) and 8 query rows: 512
  // tokens of a 16-bit 128-dim cache for up to 15 rows (one query token,
  // g <= 8), 1024 for 16 rows (g = 16, or 4 query tokens at g = 4; an item's
  // fixed cost, its q rows and merged partials, grows with its rows), 1024
  // tokens of an INT8 cache for up to 15 rows.
  const int64_t rows = (int64_t)num_query_tokens * (num_q_heads / num_kv_heads);
  const int64_t kv_bytes_per_token = 2LL * head_dim * elt;
  int32_t t = (int32_t)std::min<int64_t>(
      PA_MAX_SPLIT_TOKENS, (256 << 10) * std::max<int64_t>(1, rows / 8) / kv_bytes_per_token);
  t = t / PA_BLOCK_SIZE * PA_BLOCK_SIZE;
  // Work items: (split, KV head, set of up to 64 query rows); a decode step
  // has one row set per KV head, a prefill chunk many.
  const int64_t per_split = (int64_t)std::max(num_seqs, 0) * num_kv_heads * ((rows + 63) / 64);
  auto items = [&](int32_t tt) {
    return per_split * pa_max_splits(max_context_len, num_query_tokens, sliding_window, tt);
  };
  // Halve while the batch has too few work items to fill the device (a
  // workgroup per item, 256 compute units); with many query rows, double
  // while it keeps enough (longer splits write fewer partials).
  while (t > kMinDefaultSplit && items(t) < kMinWorkItems) t /= 2;
  if (rows > 64)
    while (t < PA_MAX_SPLIT_TOKENS && items(2 * t) >= kMinWorkItems) t *= 2;
  // A decode step with at most 8 rows per KV head, or at most 16 rows of
  // several query tokens (4 draft + target tokens at g = 4): longer splits
  // (fewer items and partials, each a longer stream), kGrowStep tokens at a time,
  // while at least kGrowWorkItems items remain and a split's K/V stays within
  // kGrowMaxBytes per KV head. Items are counted at the longest context, so a
  // batch of many short sequences stays where the bytes put it; the byte cap
  // keeps a few very long sequences (whose item count the longest context
  // overstates) at enough items. One query token with 16 rows (g = 16) keeps
  // its size: it is the shape of shared-prefix batches, whose group entries
  // (one per shared full split) get longer with it.
  if (rows <= 8 || (rows <= 16 && num_query_tokens >= 2))
    while (t + kGrowStep <= PA_MAX_SPLIT_TOKENS && items(t + kGrowStep) >= kGrowWorkItems &&
           (t + kGrowStep) * kv_bytes_per_token <= kGrowMaxBytes)
      t += kGrowStep;
  return t;
}

size_t pa_sched_bytes(int32_t num_seqs, int32_t max_splits) {
  if (num_seqs < 0 || max_splits < 0) return 0;
  return align256((pa::kSchedHeader + 2 * (size_t)plan_capacity(num_seqs, max_splits, false, 0, 1)) *
                  sizeof(int32_t));
}

size_t pa_sched_bytes_packed(int32_t num_seqs, int32_t max_splits, int32_t total_query_tokens,
                             int32_t q_heads_per_kv) {
  if (num_seqs < 0 || max_splits < 0 || total_query_tokens < 0 || q_heads_per_kv <= 0) return 0;
  return align256((pa::kSchedHeader +
                   2 * (size_t)plan_capacity(num_seqs, max_splits, true, total_query_tokens,
                                             q_heads_per_kv)) *
                  sizeof(int32_t));
}

size_t pa_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                          int32_t head_dim, int32_t max_splits) {
  if (num_seqs < 0 || num_query_tokens < 0 || num_q_heads < 0 || head_dim < 0 || max_splits < 0)
    return 0;
  const size_t rows = (size_t)num_seqs * num_query_tokens * num_q_heads * max_splits;
  return pa_sched_bytes(num_seqs, max_splits) + 2 * align256(rows * sizeof(float)) +
         align256(rows * head_dim * sizeof(float));
}

size_t pa_workspace_bytes_packed(int32_t num_seqs, int32_t total_query_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_splits) {
  if (num_seqs < 0 || total_query_tokens < 0 || num_q_heads < 0 || num_kv_heads <= 0 ||
      head_dim < 0 || max_splits < 0)
    return 0;
  const size_t rows = (size_t)total_query_tokens * num_q_heads * max_splits;
  return pa_sched_bytes_packed(num_seqs, max_splits, total_query_tokens,
                               std::max(1, num_q_heads / num_kv_heads)) +
         2 * align256(rows * sizeof(float)) + align256(rows * head_dim * sizeof(float));
}

}  // extern "C"

namespace {

// Argument checks of the KV write; fills `out` on success.
int check_write(const void *k, const void *v, int32_t in_dtype, const int64_t *slot_mapping,
                int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, void *k_cache,
                void *v_cache, float *k_scale, float *v_scale, int64_t num_blocks,
                int32_t cache_dtype, pa::WriteParams *out) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_SHAPE;
  if (in_dtype != PA_F32 && in_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (cache_dtype != PA_I8 && cache_dtype != PA_FP8 && cache_dtype != in_dtype)
    return PA_ERR_DTYPE;
  if (num_blocks > INT64_MAX / (PA_BLOCK_SIZE * (int64_t)num_kv_heads * head_dim * 4))
    return PA_ERR_SHAPE;
  if (num_tokens > 0) {
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_NULL;
    if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL;
    if (misaligned16(k) || misaligned16(v) || misaligned16(k_cache) || misaligned16(v_cache))
      return PA_ERR_ALIGN;
  }
  *out = pa::WriteParams{k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale, num_tokens,
                         num_blocks, num_kv_heads, head_dim, in_dtype, cache_dtype};
  return PA_OK;
}

// Argument checks of the plan; fills `out` on success.
int check_plan(const int32_t *context_lens, const int32_t *query_start,
               const int32_t *block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
               int32_t max_context_len, int32_t num_query_tokens, int32_t q_heads_per_kv,
               int32_t sliding_window, int32_t split_tokens, int32_t group_members,
               int32_t *sched, pa::PlanParams *out) {
  const bool packed = query_start != nullptr;
  if (num_seqs < 0 || num_seqs > PA_MAX_SEQS || max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (bad_queries(packed, num_query_tokens, sliding_window)) return PA_ERR_SHAPE;
  if (packed && !supported_group(q_heads_per_kv)) return PA_ERR_SHAPE;
  if (group_members < 1 || group_members > PA_MAX_GROUP_MEMBERS) return PA_ERR_SHAPE;
  if (group_members > 1 && (sliding_window > 0 || packed)) return PA_ERR_SHAPE;
  if (check_split_tokens(split_tokens) != PA_OK) return PA_ERR_SPLIT;
  if (num_seqs > 0 && (!context_lens || !sched)) return PA_ERR_NULL;
  if (num_seqs > 0 && group_members > 1 && !block_tables) return PA_ERR_NULL;
  const int32_t lmax = clamped_bound(max_context_len, max_blocks_per_seq);
  const int32_t ns = pa_max_splits(lmax, query_bound(packed, num_query_tokens), sliding_window,
                                   split_tokens);
  if (ns > PA_MAX_SPLITS) return PA_ERR_SPLIT;
  const int64_t cap = plan_capacity(num_seqs, ns, packed, num_query_tokens,
                                    packed ? q_heads_per_kv : 1);
  if (cap > INT_MAX / 2) return PA_ERR_SHAPE;
  *out = pa::PlanParams{context_lens, sched, num_seqs, lmax, split_tokens, num_query_tokens,
                        sliding_window, block_tables, max_blocks_per_seq, group_members,
                        query_start, packed ? q_heads_per_kv : 0, (int32_t)cap};
  return PA_OK;
}

}  // namespace

extern "C" {

int paged_kv_write(const void *k, const void *v, int32_t in_dtype, const int64_t *slot_mapping,
                   int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, void *k_cache,
                   void *v_cache, float *k_scale, float *v_scale, int64_t num_blocks,
                   int32_t cache_dtype, hipStream_t stream) {
  pa::WriteParams w;
  const int st = check_write(k, v, in_dtype, slot_mapping, num_tokens, num_kv_heads, head_dim,
                             k_cache, v_cache, k_scale, v_scale, num_blocks, cache_dtype, &w);
  if (st != PA_OK || num_tokens == 0) return st;
  pa::trace("paged_kv_write: %lld tokens x %d KV heads x %d dims, %s into a %s cache of %lld "
            "blocks", (long long)num_tokens, num_kv_heads, head_dim, pa::dtype_name(in_dtype),
            pa::dtype_name(cache_dtype), (long long)num_blocks);
  return launch_status(pa::launch_kv_write(w, stream));
}

int paged_attn_plan(const int32_t *context_lens, const int32_t *query_start,
                    const int32_t *block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t max_context_len, int32_t num_query_tokens, int32_t q_heads_per_kv,
                    int32_t sliding_window, int32_t split_tokens, int32_t group_members,
                    int32_t *sched, hipStream_t stream) {
  pa::PlanParams pl;
  const int st = check_plan(context_lens, query_start, block_tables, num_seqs,
                            max_blocks_per_seq, max_context_len, num_query_tokens,
                            q_heads_per_kv, sliding_window, split_tokens, group_members, sched,
                            &pl);
  if (st != PA_OK || num_seqs == 0) return st;
  pa::trace("paged_attn_plan: %d sequences, length bound %d, %d query tokens%s (g %d), "
            "window %d, split %d tokens, group members %d, capacity %lld entries", num_seqs,
            max_context_len, num_query_tokens, query_start ? " packed" : " each",
            query_start ? q_heads_per_kv : 0, sliding_window, split_tokens, group_members,
            (long long)pl.capacity);
  const int ls = launch_status(pa::launch_plan(pl, stream));
  if (ls == PA_OK) pa::trace_plan(sched, pl.capacity, stream);
  return ls;
}

int paged_decode_prepare(const void *k, const void *v, int32_t in_dtype,
                         const int64_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, void *k_cache, void *v_cache, float *k_scale,
                         float *v_scale, int64_t num_blocks, int32_t cache_dtype,
                         const int32_t *context_lens, const int32_t *query_start,
                         const int32_t *block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t num_query_tokens, int32_t q_heads_per_kv,
                         int32_t sliding_window, int32_t split_tokens, int32_t group_members,
                         int32_t *sched, hipStream_t stream) {
  pa::WriteParams w;
  pa::PlanParams pl;
  int st = check_write(k, v, in_dtype, slot_mapping, num_tokens, num_kv_heads, head_dim, k_cache,
                       v_cache, k_scale, v_scale, num_blocks, cache_dtype, &w);
  if (st != PA_OK) return st;
  st = check_plan(context_lens, query_start, block_tables, num_seqs, max_blocks_per_seq,
                  max_context_len, num_query_tokens, q_heads_per_kv, sliding_window,
                  split_tokens, group_members, sched, &pl);
  if (st != PA_OK) return st;
  if (num_seqs == 0) return num_tokens == 0 ? PA_OK : launch_status(pa::launch_kv_write(w, stream));
  pa::trace("paged_decode_prepare: %lld new tokens (%s into %s), %d sequences, length bound %d, "
            "%d query tokens%s (g %d), window %d, split %d tokens, group members %d",
            (long long)num_tokens, pa::dtype_name(in_dtype), pa::dtype_name(cache_dtype),
            num_seqs, max_context_len, num_query_tokens, query_start ? " packed" : " each",
            query_start ? q_heads_per_kv : 0, sliding_window, split_tokens, group_members);
  const int ls = launch_status(pa::launch_prepare(w, pl, stream));
  if (ls == PA_OK) pa::trace_plan(sched, pl.capacity, stream);
  return ls;
}

int paged_attn_decode_partial(const void *q, int32_t q_dtype, int32_t num_seqs,
                              int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                              const void *k_cache, const void *v_cache, const float *k_scale,
                              const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
                              int32_t num_kv_heads, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              const int32_t *query_start, int32_t max_context_len,
                              int32_t sliding_window, float scale, int32_t split_tokens,
                              int32_t max_splits, float *part_m, float *part_l,
                              float *part_acc, const int32_t *sched, hipStream_t stream) {
  const bool packed = query_start != nullptr;
  if (num_seqs < 0 || num_seqs > PA_MAX_SEQS || num_q_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if (bad_queries(packed, num_query_tokens, sliding_window)) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0 || !supported_group(num_q_heads / num_kv_heads))
    return PA_ERR_SHAPE;
  if (num_blocks <= 0 || num_blocks > INT_MAX) return PA_ERR_SHAPE;
  const bool dt_ok = (q_dtype == PA_BF16 && cache_dtype == PA_BF16) ||
                     (q_dtype == PA_F32 && cache_dtype == PA_F32) ||
                     ((q_dtype == PA_BF16 || q_dtype == PA_F32) && quantised(cache_dtype));
  if (!dt_ok) return PA_ERR_DTYPE;
  const int32_t qmax = query_bound(packed, num_query_tokens);
  if (split_tokens == 0)
    split_tokens = pa_default_split_tokens(
        num_seqs, num_q_heads, num_kv_heads, head_dim, cache_dtype, max_context_len,
        query_for_default(packed, num_query_tokens, num_seqs), sliding_window);
  if (check_split_tokens(split_tokens) != PA_OK) return PA_ERR_SPLIT;
  // Splits of the longest range any sequence can have under the clamped bound.
  const int32_t grid_splits = pa_max_splits(clamped_bound(max_context_len, max_blocks_per_seq),
                                            qmax, sliding_window, split_tokens);
  if (max_splits < grid_splits || grid_splits > PA_MAX_SPLITS) return PA_ERR_SPLIT;
  // Entries the plan can list: the grid has one workgroup per possible item.
  const int64_t max_entries = plan_capacity(num_seqs, grid_splits, packed, num_query_tokens,
                                            num_q_heads / num_kv_heads);
  // Workgroups per entry: Hkv, times (uniform Q) the sets of at least 32 rows
  // of a KV head's Q*g rows.
  const int64_t per_entry =
      (int64_t)num_kv_heads *
      (packed ? 1 : ((int64_t)qmax * (num_q_heads / num_kv_heads) + 31) / 32);
  if (max_entries * per_entry > INT_MAX) return PA_ERR_SHAPE;
  if (num_seqs == 0 || (packed && num_query_tokens == 0)) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !part_m || !part_l ||
      !part_acc || !sched)
    return PA_ERR_NULL;
  if ((int64_t)num_query_tokens * num_q_heads * (packed ? 1 : num_seqs) * max_splits >
      INT64_MAX / (head_dim * 4))
    return PA_ERR_SHAPE;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache) || misaligned16(part_acc))
    return PA_ERR_ALIGN;

  pa::DecodeParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.part_m = part_m;
  p.part_l = part_l;
  p.part_acc = part_acc;
  p.num_blocks = num_blocks;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.split_tokens = split_tokens;
  p.max_splits = max_splits;
  p.num_query_tokens = num_query_tokens;
  p.window = sliding_window;
  p.group = num_q_heads / num_kv_heads;
  p.group_shift = __builtin_ctz((unsigned)p.group);
  p.fd_split = pa::FastDiv::make((uint32_t)split_tokens);
  p.fd_kv_heads = pa::FastDiv::make((uint32_t)num_kv_heads);
  p.query_start = query_start;
  p.sched = sched;
  p.scale_log2 = scale * 1.4426950408889634f;
  pa::trace("paged_attn_decode_partial: q %s, cache %s, %d sequences x %d query tokens%s, %d/%d "
            "heads, D %d, window %d, split %d tokens, %d partial slots per row (%d needed), %lld "
            "possible entries x %lld items each", pa::dtype_name(q_dtype),
            pa::dtype_name(cache_dtype), num_seqs, num_query_tokens,
            packed ? " (packed total)" : "", num_q_heads, num_kv_heads, head_dim,
            sliding_window, split_tokens, max_splits, grid_splits, (long long)max_entries,
            (long long)per_entry);

  hipError_t e;
  if (q_dtype == PA_BF16 && cache_dtype == PA_BF16)
    e = pa::decode_bf16_bf16(p, max_entries, stream);
  else if (q_dtype == PA_F32 && cache_dtype == PA_F32)
    e = pa::decode_f32_f32(p, max_entries, stream);
  else if (q_dtype == PA_BF16 && cache_dtype == PA_I8)
    e = pa::decode_bf16_i8(p, max_entries, stream);
  else if (cache_dtype == PA_I8)
    e = pa::decode_f32_i8(p, max_entries, stream);
  else if (q_dtype == PA_BF16)
    e = pa::decode_bf16_fp8(p, max_entries, stream);
  else
    e = pa::decode_f32_fp8(p, max_entries, stream);
  return launch_status(e);
}

int paged_attn_reduce(const float *part_m, const float *part_l, const float *part_acc,
                      const int32_t *context_lens, const int32_t *query_start, int32_t num_seqs,
                      int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                      int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t sliding_window, int32_t split_tokens, int32_t max_splits,
                      void *out, int32_t out_dtype, hipStream_t stream) {
  const bool packed = query_start != nullptr;
  if (num_seqs < 0 || num_seqs > PA_MAX_SEQS || num_q_heads <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return PA_ERR_SHAPE;
  if (bad_queries(packed, num_query_tokens, sliding_window)) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_SHAPE;
  if ((int64_t)num_query_tokens * num_q_heads > INT_MAX) return PA_ERR_SHAPE;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_DTYPE;
  if (check_split_tokens(split_tokens) != PA_OK || max_splits <= 0) return PA_ERR_SPLIT;
  if (num_seqs == 0 || (packed && num_query_tokens == 0)) return PA_OK;
  if (!part_m || !part_l || !part_acc || !context_lens || !out) return PA_ERR_NULL;
  pa::ReduceParams p{part_m, part_l, part_acc, context_lens, out, num_seqs, num_q_heads,
                     head_dim, split_tokens, max_splits, out_dtype, num_query_tokens,
                     sliding_window, query_start,
                     clamped_bound(max_context_len, max_blocks_per_seq)};
  pa::trace("paged_attn_reduce: %d sequences x %d query tokens%s x %d heads, D %d, %d partial "
            "slots per row, out %s", num_seqs, num_query_tokens, packed ? " (packed total)" : "",
            num_q_heads, head_dim, max_splits, pa::dtype_name(out_dtype));
  return launch_status(pa::launch_reduce(p, stream));
}

}  // extern "C"

namespace pa {

int decode_workspace_need(const void *q, int32_t q_dtype, int32_t num_seqs,
                          int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                          const void *k_cache, const void *v_cache, const float *k_scale,
                          const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
                          int32_t num_kv_heads, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                          const int32_t *query_start, int32_t max_context_len,
                          int32_t sliding_window, int32_t split_tokens, const void *out,
                          size_t *need) {
  *need = 0;
  const bool packed = query_start != nullptr;
  if (max_context_len < 0 || num_seqs < 0 || num_seqs > PA_MAX_SEQS || num_q_heads <= 0 ||
      num_kv_heads <= 0 || max_blocks_per_seq <= 0 || num_q_heads % num_kv_heads != 0 ||
      !supported_group(num_q_heads / num_kv_heads) || num_blocks <= 0 || num_blocks > INT_MAX)
    return PA_ERR_SHAPE;
  if (bad_queries(packed, num_query_tokens, sliding_window)) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_SHAPE;
  const bool dt_ok = (q_dtype == PA_BF16 && cache_dtype == PA_BF16) ||
                     (q_dtype == PA_F32 && cache_dtype == PA_F32) ||
                     ((q_dtype == PA_BF16 || q_dtype == PA_F32) && quantised(cache_dtype));
  if (!dt_ok) return PA_ERR_DTYPE;
  const int32_t qmax = query_bound(packed, num_query_tokens);
  if (split_tokens == 0)
    split_tokens = pa_default_split_tokens(
        num_seqs, num_q_heads, num_kv_heads, head_dim, cache_dtype, max_context_len,
        query_for_default(packed, num_query_tokens, num_seqs), sliding_window);
  if (check_split_tokens(split_tokens) != PA_OK) return PA_ERR_SPLIT;
  const int32_t ns = pa_max_splits(clamped_bound(max_context_len, max_blocks_per_seq), qmax,
                                   sliding_window, split_tokens);
  if (ns > PA_MAX_SPLITS) return PA_ERR_SPLIT;
  if (num_seqs == 0 || (packed && num_query_tokens == 0)) return PA_OK;
  if (!q || !out || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (quantised(cache_dtype) && (!k_scale || !v_scale)) return PA_ERR_NULL;
  if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache)) return PA_ERR_ALIGN;
  *need = packed ? pa_workspace_bytes_packed(num_seqs, num_query_tokens, num_q_heads,
                                             num_kv_heads, head_dim, ns)
                 : pa_workspace_bytes(num_seqs, num_query_tokens, num_q_heads, head_dim, ns);
  return PA_OK;
}

}  // namespace pa

extern "C" {

int paged_attn_decode(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_query_tokens,
                      int32_t num_q_heads, int32_t head_dim, const void *k_cache,
                      const void *v_cache, const float *k_scale, const float *v_scale,
                      int32_t cache_dtype, int64_t num_blocks, int32_t num_kv_heads,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, const int32_t *query_start,
                      int32_t max_context_len, int32_t sliding_window, float scale,
                      int32_t split_tokens, void *out, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  size_t need;
  int st = pa::decode_workspace_need(q, q_dtype, num_seqs, num_query_tokens, num_q_heads,
                                     head_dim, k_cache, v_cache, k_scale, v_scale, cache_dtype,
                                     num_blocks, num_kv_heads, block_tables, max_blocks_per_seq,
                                     context_lens, query_start, max_context_len, sliding_window,
                                     split_tokens, out, &need);
  if (st != PA_OK || need == 0) return st;
  if (!workspace) return PA_ERR_NULL;
  if (((uintptr_t)workspace & 255u) != 0) return PA_ERR_ALIGN;
  if (workspace_bytes < need) return PA_ERR_WORKSPACE;
  const bool packed = query_start != nullptr;
  if (split_tokens == 0)
    split_tokens = pa_default_split_tokens(
        num_seqs, num_q_heads, num_kv_heads, head_dim, cache_dtype, max_context_len,
        query_for_default(packed, num_query_tokens, num_seqs), sliding_window);
  const int32_t ns = pa_max_splits(clamped_bound(max_context_len, max_blocks_per_seq),
                                   query_bound(packed, num_query_tokens), sliding_window,
                                   split_tokens);
  const int32_t g = num_q_heads / num_kv_heads;
  const size_t rows = (size_t)(packed ? 1 : num_seqs) * num_query_tokens * num_q_heads * ns;
  char *base = (char *)workspace;
  int32_t *sched = (int32_t *)base;
  base += packed ? pa_sched_bytes_packed(num_seqs, ns, num_query_tokens, g)
                 : pa_sched_bytes(num_seqs, ns);
  float *m = (float *)base;
  float *l = (float *)(base + align256(rows * sizeof(float)));
  float *acc = (float *)(base + 2 * align256(rows * sizeof(float)));
  st = paged_attn_plan(context_lens, query_start, block_tables, num_seqs, max_blocks_per_seq,
                       max_context_len, num_query_tokens, g, sliding_window, split_tokens, 1,
                       sched, stream);
  if (st != PA_OK) return st;
  st = paged_attn_decode_partial(q, q_dtype, num_seqs, num_query_tokens, num_q_heads, head_dim,
                                 k_cache, v_cache, k_scale, v_scale, cache_dtype, num_blocks,
                                 num_kv_heads, block_tables, max_blocks_per_seq, context_lens,
                                 query_start, max_context_len, sliding_window, scale,
                                 split_tokens, ns, m, l, acc, sched, stream);
  if (st != PA_OK) return st;
  return paged_attn_reduce(m, l, acc, context_lens, query_start, num_seqs, num_query_tokens,
                           num_q_heads, head_dim, max_blocks_per_seq, max_context_len,
                           sliding_window, split_tokens, ns, out, q_dtype, stream);
}

int pa_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t sink_words,
                      hipStream_t stream) {
  if (!src || !sink) return PA_ERR_NULL;
  if (misaligned16(src)) return PA_ERR_ALIGN;
  if (sink_words < 256 || bytes % 16 != 0) return PA_ERR_SHAPE;
  const int blocks = sink_words / 256;
  return launch_status(pa::launch_read_probe(src, bytes, sink, blocks, stream));
}

}  // extern "C"
