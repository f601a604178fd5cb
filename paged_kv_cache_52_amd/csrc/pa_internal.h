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

// One per (q dtype, cache dtype) pair; p.group = Hq / Hkv in {1, 2, 4, 8, 16}.
hipError_t decode_bf16_bf16(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_f32(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_bf16_i8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_i8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_bf16_fp8(const DecodeParams &p, int64_t max_entries, hipStream_t s);
hipError_t decode_f32_fp8(const DecodeParams &p, int64_t max_entries, hipStream_t s);

}  // namespace pa
