// Host-side launch interfaces between the C ABI layer and the kernel units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_kernel.h"

namespace pa {

struct ReduceParams {
  const float *part_m;
  const float *part_l;
  const float *part_acc;
  const int32_t *context_lens;
  void *out;
  int32_t num_seqs, num_q_heads, head_dim, split_tokens, max_splits, out_dtype;
  int32_t num_query_tokens, window;  // per sequence, or the packed total with query_start
  const int32_t *query_start;        // [num_seqs + 1] packed query offsets, or nullptr
  int32_t len_bound;  // context lengths are clamped to [0, len_bound], as in the split kernel
};

struct WriteParams {
  const void *k;
  const void *v;
  const int64_t *slot_mapping;
  void *k_cache;
  void *v_cache;
  float *k_scale;
  float *v_scale;
  int64_t num_tokens;
  int64_t num_blocks;
  int32_t num_kv_heads, head_dim, in_dtype, cache_dtype;
};

constexpr int kPlanThreads = 256;  // threads of the plan workgroup (and write workgroups)

struct PlanParams {
  const int32_t *context_lens;
  int32_t *sched;
  int32_t num_seqs, max_len, split_tokens;
  int32_t num_query_tokens;     // per sequence, or the packed total with query_start
  int32_t window;
  const int32_t *block_tables;  // read only with group_members > 1
  int32_t max_blocks_per_seq;
  int32_t group_members;        // 1: no grouping; 2..4: sequences per group entry
  const int32_t *query_start;   // [num_seqs + 1] packed query offsets, or nullptr
  int32_t group;                // g = Hq / Hkv (used with query_start)
  int32_t capacity;             // entries the scheduling scratch holds
};

hipError_t launch_plan(const PlanParams &p, hipStream_t stream);
// KV write and plan in one launch: the last workgroup plans, the others write.
hipError_t launch_prepare(const WriteParams &w, const PlanParams &p, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams &p, hipStream_t stream);
hipError_t launch_kv_write(const WriteParams &p, hipStream_t stream);
hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream);

// paged_attn_decode's argument checks (every one made before it enqueues
// anything) and the workspace it needs: *need = 0 when the call has nothing to
// do. split_tokens 0 means the default.
int decode_workspace_need(const void *q, int32_t q_dtype, int32_t num_seqs,
                          int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                          const void *k_cache, const void *v_cache, const float *k_scale,
                          const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
                          int32_t num_kv_heads, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                          const int32_t *query_start, int32_t max_context_len,
                          int32_t sliding_window, int32_t split_tokens, const void *out,
                          size_t *need);

// One per (q dtype, cache dtype) pair; p.group = Hq / Hkv in {1, 2, 4, 8, 16}.
hipError_t decode_bf16_bf16(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_f32(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_bf16_i8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_i8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_bf16_fp8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_fp8(const DecodeParams &p, int64_t max_entries, hipStream_t s);

}  // namespace pa
