// Plan of a decode step, as device code shared by the plan kernel and the
// fused write-and-plan kernel.
//
// One workgroup of kPlanThreads threads turns context_lens into the list of
// splits the split kernel works through [EchoLLMServing notes, section 2:
// split count derived from the context length, max(1, ceil(L/T)); with a
// sliding window, of the span the window reaches]. It writes
// into the scheduling scratch:
//   sched[0]  = number of entries of the list
//   sched[1..7] = split_tokens, num_seqs, clamped max length, query tokens
//                 (per sequence, or the packed total), window, group_members
//                 (0 when grouping is off), and g = Hq/Hkv with packed
//                 queries (0 otherwise); the split kernel checks them
//   sched[8+2i], sched[9+2i] = entry i: (s << 16) | j, then L_s (or, with
//     packed queries, the index of the block of kPackedRows query rows of the
//     sequence the entry covers), in this order:
//     1. all splits but the last of each sequence (full T-token splits),
//        sequence by sequence (with packed queries, every row block of a split
//        in turn); with grouping on (group_members M > 1), the full split j
//        of up to M consecutive sequences of an aligned run of M whose split j
//        starts on the same physical block is one entry ((s0 << 16) | j,
//        -count), listed at its first sequence;
//     2. the last split of each sequence (all its row blocks), longest first
//        (counting sort on its 16-token tile count), so the shortest work
//        runs at the very end.
// A sequence of length 0 contributes one empty split; with packed queries a
// sequence without query tokens contributes nothing. Lengths are clamped
// exactly as the split kernel clamps them, and no entry is written past the
// capacity the caller sized the scratch for. A group entry is only a hint for
// cache sharing: the split kernel reads each member's own block table.
#pragma once

#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kMaxTileBuckets = PA_MAX_SPLIT_TOKENS / kBlock;  // tile counts 1..256
// Grouped plans of one chunk take a faster path when no sequence has more
// full splits than this (one bit of a mask each).
constexpr int kJoinSplits = 16;
static_assert(kJoinSplits <= 32, "one 32-bit mask per sequence");

__device__ __forceinline__ int clamp_len(const PlanParams &p, int s) {
  return max(0, min(p.context_lens[s], p.max_len));
}

__device__ __forceinline__ int seq_splits(const PlanParams &p, int L, int Q) {
  return splits_of(L, Q, p.window, p.split_tokens);
}

// Tiles of the last split (1 for an empty split range, which sorts last).
__device__ __forceinline__ int last_tiles(const PlanParams &p, int L, int Q) {
  const int span = L - split_base(L, Q, p.window);
  if (span <= 0) return 1;
  const int rest = span - (seq_splits(p, L, Q) - 1) * p.split_tokens;
  return (rest + kBlock - 1) / kBlock;
}

// What the plan needs of sequence s: clamped length, query tokens, splits and
// entries per split (1, or with packed queries its blocks of kPackedRows
// query rows; 0 for a sequence without query tokens).
struct SeqPlan {
  int L, Q, splits, per_split;
};

__device__ __forceinline__ SeqPlan seq_plan(const PlanParams &p, int s) {
  SeqPlan r;
  r.L = clamp_len(p, s);
  if (p.query_start == nullptr) {
    r.Q = p.num_query_tokens;
    r.per_split = 1;
  } else {
    r.Q = query_span(p.query_start, s, 0, p.num_query_tokens).count;
    r.per_split = (r.Q * p.group + kPackedRows - 1) / kPackedRows;
  }
  r.splits = seq_splits(p, r.L, r.Q);
  return r;
}

// First word of an entry: sequence s (< 65536) in the high 16 bits, split j
// (< 65536) in the low 16, packed as unsigned (the word is negative for
// s >= 32768; readers shift it as unsigned).
__device__ __forceinline__ int entry_word(int s, int j) {
  return (int)(((uint32_t)s << 16) | (uint32_t)j);
}

__device__ __forceinline__ void put_entry(const PlanParams &p, int idx, int w0, int w1) {
  if (idx < p.capacity) {
    p.sched[kSchedHeader + 2 * idx] = w0;
    p.sched[kSchedHeader + 2 * idx + 1] = w1;
  }
}

// Join flags of the full split j of sequence s: bit c (c < M) is set when
// sequence s + c takes part in the group of sequence s + c - 1 for split j,
// that is when both splits are full and start on the same physical block.
// Split counts of sequences s - 1 .. s + M - 1 come from the chunk's counts in
// LDS (sequences base .. base + kPlanThreads - 1) or, past the chunk, from
// their lengths in global memory; their table words at block jb are loaded in
// the same round (a word of a sequence whose split j is not full is read but
// not used).
__device__ __forceinline__ int join_bits(const PlanParams &p, int s, int j, int base,
                                         const int (&chunk_splits)[kPlanThreads]) {
  constexpr int kMax = PA_MAX_GROUP_MEMBERS;
  const int M = p.group_members;
  const int jb = j * (p.split_tokens / kBlock);  // first block of split j (no window: base 0)
  int nsp[kMax + 1], blk[kMax + 1];
#pragma unroll
  for (int c = 0; c <= kMax; ++c) {
    const int t = s - 1 + c;
    const bool seq = c <= M && t >= 0 && t < p.num_seqs;
    nsp[c] = 0;
    blk[c] = -1;
    if (seq) {
      nsp[c] = t >= base && t < base + kPlanThreads
                   ? chunk_splits[t - base]
                   : seq_splits(p, clamp_len(p, t), p.num_query_tokens);
      if (jb < p.max_blocks_per_seq)
        blk[c] = p.block_tables[(int64_t)t * p.max_blocks_per_seq + jb];
    }
  }
  bool full[kMax + 1];
#pragma unroll
  for (int c = 0; c <= kMax; ++c) full[c] = j < nsp[c] - 1;
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
  __shared__ int chunk_per[kPlanThreads];    // entries per split of each sequence
  __shared__ int chunk_splits[kPlanThreads]; // splits of each sequence
  __shared__ uint32_t join_mask[kPlanThreads];  // grouping, one chunk: see below
  __shared__ int many_full;  // some sequence has more than kJoinSplits full splits
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  const bool packed = p.query_start != nullptr;

  for (int i = tid; i <= kMaxTileBuckets; i += kPlanThreads) bucket[i] = 0;
  if (tid == 0) {
    carry = 0;
    many_full = 0;
  }
  __syncthreads();

  // Pass 1: the full splits. Per chunk of kPlanThreads sequences, a
  // workgroup-wide exclusive scan of their entry counts gives each sequence's
  // first entry; all threads then write the chunk's entries together (each
  // finds its sequence by binary search over the chunk's offsets). The last
  // splits are histogrammed by tile count on the way.
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int s = base + tid;
    const bool valid = s < p.num_seqs;
    SeqPlan sp{0, 0, 1, 0};
    if (valid) sp = seq_plan(p, s);
    const int f = (sp.splits - 1) * sp.per_split;
    if (f > kJoinSplits) many_full = 1;
    int incl = f;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wave_sum[wave] = incl;
    if (sp.per_split > 0) atomicAdd(&bucket[last_tiles(p, sp.L, sp.Q)], sp.per_split);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      if (w < wave) before += wave_sum[w];
      total += wave_sum[w];
    }
    chunk_first[tid] = before + incl - f;  // offset inside the chunk
    chunk_len[tid] = sp.L;
    chunk_per[tid] = max(sp.per_split, 1);
    chunk_splits[tid] = sp.splits;
    __syncthreads();
    const int base_entry = carry;
    if (p.group_members <= 1) {
      for (int e = tid; e < total; e += kPlanThreads) {
        const int lo = owner_of(chunk_first, e);
        const int q = e - chunk_first[lo], per = chunk_per[lo];
        const int j = q / per, rb = q % per;  // row blocks of a split are adjacent
        put_entry(p, base_entry + e, entry_word(base + lo, j), packed ? rb : chunk_len[lo]);
      }
      __syncthreads();
      if (tid == 0) carry += total;
      __syncthreads();
    } else if (p.num_seqs <= kPlanThreads && !many_full) {
      // Grouping with the whole batch in one chunk and at most kJoinSplits
      // full splits per sequence: the entries and their order are those of
      // the general loop below, found with one round of table reads. Thread s
      // reads the first table word of each of its full splits and of its
      // predecessor's same split (all at once), and keeps the splits on which
      // the two share a block as a bit mask in LDS. Split j of s is listed
      // unless s joins its predecessor inside the aligned run of M; a listed
      // split counts the following sequences of the run that join one after
      // another. One workgroup scan places every sequence's listed splits.
      const int M = p.group_members;
      const int step = p.split_tokens / kBlock;  // blocks per split (no window: base 0)
      const int fp = tid > 0 ? chunk_splits[tid - 1] - 1 : 0;  // predecessor's full splits
      int own[kJoinSplits], prev[kJoinSplits];
#pragma unroll
      for (int j = 0; j < kJoinSplits; ++j) {
        own[j] = 0;
        prev[j] = -1;
        if (j < f) {
          own[j] = p.block_tables[(int64_t)s * p.max_blocks_per_seq + j * step];
          if (j < fp) prev[j] = p.block_tables[(int64_t)(s - 1) * p.max_blocks_per_seq + j * step];
        }
      }
      uint32_t joined = 0u;
#pragma unroll
      for (int j = 0; j < kJoinSplits; ++j)
        if (j < f && j < fp && own[j] == prev[j]) joined |= 1u << j;
      join_mask[tid] = joined;
      __syncthreads();
      const int pos = s % M;
      const uint32_t full = f > 0 ? (~0u >> (32 - f)) : 0u;
      const uint32_t listed = pos > 0 ? full & ~joined : full;
      uint32_t follow[PA_MAX_GROUP_MEMBERS];  // follow[c]: splits that s + c joins (c >= 1)
#pragma unroll
      for (int c = 1; c < PA_MAX_GROUP_MEMBERS; ++c)
        follow[c] = pos + c < M && s + c < p.num_seqs ? join_mask[tid + c] : 0u;
      const int nk = __builtin_popcount(listed);
      int incl_k = nk;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl_k, o);
        if (lane >= o) incl_k += y;
      }
      if (lane == kWave - 1) wave_sum[wave] = incl_k;
      __syncthreads();
      int before_k = 0, total_k = 0;
#pragma unroll
      for (int w = 0; w < kPlanThreads / kWave; ++w) {
        if (w < wave) before_k += wave_sum[w];
        total_k += wave_sum[w];
      }
      int idx = carry + before_k + incl_k - nk;
      for (uint32_t m = listed; m != 0u; m &= m - 1u) {
        const int j = __builtin_ctz(m);
        int cnt = 1;
#pragma unroll
        for (int c = 1; c < PA_MAX_GROUP_MEMBERS; ++c)
          if (cnt == c && ((follow[c] >> j) & 1u)) ++cnt;
        put_entry(p, idx++, entry_word(s, j), cnt > 1 ? -cnt : sp.L);
      }
      __syncthreads();
      if (tid == 0) carry += total_k;
      __syncthreads();
    } else {
      // Grouping (one entry per split, no packed queries): an entry (s, j)
      // whose sequence joins its predecessor inside the aligned run of M is
      // dropped (its group's first sequence lists it); the others count how
      // many following sequences of the run join. The kept entries are
      // compacted with a workgroup scan per stride.
      const int M = p.group_members;
      for (int e0 = 0; e0 < total; e0 += kPlanThreads) {
        const int e = e0 + tid;
        int keep = 0, cnt = 1, word0 = 0, L_e = 0;
        if (e < total) {
          const int lo = owner_of(chunk_first, e);
          const int s_e = base + lo, j = e - chunk_first[lo];
          word0 = entry_word(s_e, j);
          L_e = chunk_len[lo];
          const int pos = s_e % M;
          const int bits = join_bits(p, s_e, j, base, chunk_splits);
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
        if (keep) put_entry(p, carry + before_k + incl_k - 1, word0, cnt > 1 ? -cnt : L_e);
        __syncthreads();
        if (tid == 0) carry += total_k;
        __syncthreads();
      }
    }
  }
  const int n_full = carry;

  // Start offset of each tile-count bucket, longest first: a reverse
  // exclusive scan over buckets kMaxTileBuckets .. 1 (one bucket per thread).
  int n_last = 0;
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
    for (int w = 0; w < kPlanThreads / kWave; ++w) {
      if (w < wave) before += wave_sum[w];
      n_last += wave_sum[w];
    }
    bucket[b] = n_full + before + incl - c;
  }
  __syncthreads();

  // Pass 2: place each sequence's last split (each of its row blocks, kept
  // together) in its bucket (the order inside a bucket does not affect any
  // result).
  for (int base = 0; base < p.num_seqs; base += kPlanThreads) {
    const int s = base + tid;
    if (s < p.num_seqs) {
      const SeqPlan sp = seq_plan(p, s);
      if (sp.per_split > 0) {
        const int pos = atomicAdd(&bucket[last_tiles(p, sp.L, sp.Q)], sp.per_split);
        for (int rb = 0; rb < sp.per_split; ++rb)
          put_entry(p, pos + rb, entry_word(s, sp.splits - 1), packed ? rb : sp.L);
      }
    }
  }
  if (tid == 0) {
    p.sched[0] = min(n_full + n_last, p.capacity);
    p.sched[1] = p.split_tokens;
    p.sched[2] = p.num_seqs;
    p.sched[3] = p.max_len;
    p.sched[4] = p.num_query_tokens;
    p.sched[5] = p.window;
    p.sched[6] = p.group_members > 1 ? p.group_members : 0;
    p.sched[7] = packed ? p.group : 0;
  }
}

}  // namespace pa
