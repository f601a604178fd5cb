// Plan of a decode step, as device code shared by the plan kernel and the
// fused write-and-plan kernel.
//
// One workgroup of kPlanThreads threads turns context_lens into the list of
// splits the split kernel works through [EchoLLMServing notes, section 2:
// split count derived from the context length, max(1, ceil(L/T)); with a
// sliding window, of the span the window reaches]. It writes
// into the scheduling scratch:
//   sched[0]  = number of splits of the batch
//   sched[1..6] = split_tokens, num_seqs, clamped max length, query tokens,
//                 window, group_members (0 when grouping is off), checked by
//                 the split kernel; sched[7] = 0
//   sched[8+2i], sched[9+2i] = (s << 16) | j, L_s   split i, in this order:
//     1. all splits but the last of each sequence (full T-token splits),
//        sequence by sequence; with grouping on (group_members M > 1), the
//        full split j of up to M consecutive sequences of an aligned run of M
//        whose split j starts on the same physical block is one entry
//        ((s0 << 16) | j, -count), listed at its first sequence;
//     2. the last split of each sequence, longest first (counting sort on its
//        16-token tile count), so the shortest work runs at the very end.
// A sequence of length 0 contributes one empty split. Lengths are clamped
// exactly as the split kernel clamps them. A group entry is only a hint for
// cache sharing: the split kernel reads each member's own block table.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kMaxTileBuckets = PA_MAX_SPLIT_TOKENS / kBlock;  // tile counts 1..256

__device__ __forceinline__ int clamp_len(const PlanParams &p, int s) {
  return max(0, min(p.context_lens[s], p.max_len));
}

__device__ __forceinline__ int seq_splits(const PlanParams &p, int L) {
  return splits_of(L, p.num_query_tokens, p.window, p.split_tokens);
}

// Tiles of the last split (1 for an empty split range, which sorts last).
__device__ __forceinline__ int last_tiles(const PlanParams &p, int L) {
  const int span = L - split_base(L, p.num_query_tokens, p.window);
  if (span <= 0) return 1;
  const int rest = span - (seq_splits(p, L) - 1) * p.split_tokens;
  return (rest + kBlock - 1) / kBlock;
}

// Join flags of the full split j of sequence s: bit c (c < M) is set when
// sequence s + c takes part in the group of sequence s + c - 1 for split j,
// that is when both splits are full and start on the same physical block.
// Lengths and table words of sequences s - 1 .. s + M - 1 are read together
// (two rounds of loads, whatever M).
__device__ __forceinline__ int join_bits(const PlanParams &p, int s, int j) {
  constexpr int kMax = PA_MAX_GROUP_MEMBERS;
  const int M = p.group_members;
  const int jb = j * (p.split_tokens / kBlock);  // first block of split j (no window: base 0)
  bool full[kMax + 1];
  int blk[kMax + 1];
#pragma unroll
  for (int c = 0; c <= kMax; ++c) {
    const int t = s - 1 + c;
    full[c] = c <= M && t >= 0 && t < p.num_seqs && j < seq_splits(p, clamp_len(p, t)) - 1;
  }
#pragma unroll
  for (int c = 0; c <= kMax; ++c)  // j < splits - 1 keeps jb inside the table row
    blk[c] = full[c] ? p.block_tables[(int64_t)(s - 1 + c) * p.max_blocks_per_seq + jb] : -1;
  int bits = 0;
#pragma unroll
  for (int c = 0; c < kMax; ++c)
    if (c < M && full[c] && full[c + 1] && blk[c] == blk[c + 1]) bits |= 1 << c;
  return bits;
}

// Last i with first[i] <= e, over a chunk's ascending entry offsets.
// Sequences with no full split share their offset with the next one; the
// search lands on the last of them, which is the one that owns entry e.
__device__ __forceinline__ int owner_of(const int (&first)[kPlanThreads], int e) {
  int lo = 0, hi = kPlanThreads - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (first[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

static __device__ void plan_workgroup(const PlanParams &p) {
  __shared__ int wave_sum[kPlanThreads / kWave];
  __shared__ int bucket[kMaxTileBuckets + 1];  // count, then start offset, of each tile count
  __shared__ int carry;
  __shared__ int chunk_first[kPlanThreads];  // first entry of each sequence of the chunk
  __shared__ int chunk_len[kPlanThreads];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;

  for (int i = tid; i <= kMaxTileBuckets; i += kPlanThreads) bucket[i] = 0;
  if (tid == 0) carry = 0;
  __syncthreads();

  // Pass 1: the full splits. Per chunk of kPlanThreads sequences, a
  // workgroup-wide exclusive scan of their counts gives each sequence's first
  // entry; all threads then write the chunk's entries together (each finds its
  // sequence by binary search over the chunk's offsets). The last splits are
  // histogrammed by tile count on the way.
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int s = base + tid;
    const bool valid = s < p.num_seqs;
    const int L = valid ? clamp_len(p, s) : 0;
    const int f = valid ? seq_splits(p, L) - 1 : 0;
    int incl = f;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wave_sum[wave] = incl;
    if (valid) atomicAdd(&bucket[last_tiles(p, L)], 1);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      if (w < wave) before += wave_sum[w];
      total += wave_sum[w];
    }
    chunk_first[tid] = before + incl - f;  // offset inside the chunk
    chunk_len[tid] = L;
    __syncthreads();
    const int base_entry = carry;
    if (p.group_members <= 1) {
      for (int e = tid; e < total; e += kPlanThreads) {
        const int lo = owner_of(chunk_first, e);
        const int q = e - chunk_first[lo];
        p.sched[kSchedHeader + 2 * (base_entry + e)] = ((base + lo) << 16) | q;
        p.sched[kSchedHeader + 2 * (base_entry + e) + 1] = chunk_len[lo];
      }
      __syncthreads();
      if (tid == 0) carry += total;
      __syncthreads();
    } else {
      // Grouping: an entry (s, j) whose sequence joins its predecessor inside
      // the aligned run of M is dropped (its group's first sequence lists it);
      // the others count how many following sequences of the run join. The
      // kept entries are compacted with a workgroup scan per stride.
      const int M = p.group_members;
      for (int e0 = 0; e0 < total; e0 += kPlanThreads) {
        const int e = e0 + tid;
        int keep = 0, cnt = 1, word0 = 0, L_e = 0;
        if (e < total) {
          const int lo = owner_of(chunk_first, e);
          const int s_e = base + lo, j = e - chunk_first[lo];
          word0 = (s_e << 16) | j;
          L_e = chunk_len[lo];
          const int pos = s_e % M;
          const int bits = join_bits(p, s_e, j);
          keep = !(pos > 0 && (bits & 1));
          if (keep)
            while (pos + cnt < M && ((bits >> cnt) & 1)) ++cnt;
        }
        int incl_k = keep;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl_k, o);
          if (lane >= o) incl_k += y;
        }
        __syncthreads();  // wave_sum is free again
        if (lane == kWave - 1) wave_sum[wave] = incl_k;
        __syncthreads();
        int before_k = 0, total_k = 0;
#pragma unroll
        for (int w = 0; w < kPlanThreads / kWave; ++w) {
          if (w < wave) before_k += wave_sum[w];
          total_k += wave_sum[w];
        }
        if (keep) {
          const int at = carry + before_k + incl_k - 1;
          p.sched[kSchedHeader + 2 * at] = word0;
          p.sched[kSchedHeader + 2 * at + 1] = cnt > 1 ? -cnt : L_e;
        }
        __syncthreads();
        if (tid == 0) carry += total_k;
        __syncthreads();
      }
    }
  }
  const int n_full = carry;

  // Start offset of each tile-count bucket, longest first: a reverse
  // exclusive scan over buckets kMaxTileBuckets .. 1 (one bucket per thread).
  {
    const int b = kMaxTileBuckets - tid;  // tid 0 -> 256, ..., tid 255 -> 1
    const int c = bucket[b];
    int incl = c;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == kWave - 1) wave_sum[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w)
      if (w < wave) before += wave_sum[w];
    bucket[b] = n_full + before + incl - c;
  }
  __syncthreads();

  // Pass 2: place each sequence's last split in its bucket (the order inside
  // a bucket does not affect any result).
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int s = base + tid;
    if (s < p.num_seqs) {
      const int L = clamp_len(p, s);
      const int pos = atomicAdd(&bucket[last_tiles(p, L)], 1);
      p.sched[kSchedHeader + 2 * pos] = (s << 16) | (seq_splits(p, L) - 1);
      p.sched[kSchedHeader + 2 * pos + 1] = L;
    }
  }
  if (tid == 0) {
    p.sched[0] = n_full + p.num_seqs;
    p.sched[1] = p.split_tokens;
    p.sched[2] = p.num_seqs;
    p.sched[3] = p.max_len;
    p.sched[4] = p.num_query_tokens;
    p.sched[5] = p.window;
    p.sched[6] = p.group_members > 1 ? p.group_members : 0;
    p.sched[7] = 0;
  }
}

}  // namespace pa
