// Device helpers shared by the libpagedattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

constexpr int kBlock = PA_BLOCK_SIZE;  // tokens per KV block
constexpr int kWave = 64;              // CDNA wavefront width

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running-max start value: finite, so exp2(m_old - m_new) never sees inf - inf.
constexpr float kNegBig = -3.0e38f;

template <int DT> struct DtypeBytes;
template <> struct DtypeBytes<PA_F32> { static constexpr int value = 4; };
template <> struct DtypeBytes<PA_BF16> { static constexpr int value = 2; };
template <> struct DtypeBytes<PA_I8> { static constexpr int value = 1; };
template <> struct DtypeBytes<PA_FP8> { static constexpr int value = 1; };

// Caches stored as 8-bit codes with a per-(token, KV head) fp32 scale.
template <int CT>
struct Quantised {
  static constexpr bool value = CT == PA_I8 || CT == PA_FP8;
};

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Lane permutation inside a 16-lane DPP row; every lane's source is active.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Values of lane l and lane l ^ K (K = 16 or 32) as (the one whose bit K is
// clear, the one whose bit K is set), the same pair in both lanes: gfx950's
// v_permlane16_swap / v_permlane32_swap of x with itself, one VALU op instead
// of an LDS permute.
struct LanePair {
  float lo, hi;
};
template <int K>
__device__ __forceinline__ LanePair lane_pair(float x) {
  static_assert(K == 16 || K == 32, "row pairs of 16 or halves of 32 lanes");
  const uint32_t u = __float_as_uint(x);
#if __HIP_DEVICE_COMPILE__
  if constexpr (K == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
  }
#else
  return {__uint_as_float(u), __uint_as_float(u)};
#endif
}
template <int K>
__device__ __forceinline__ float xor_sum(float x) {
  const LanePair p = lane_pair<K>(x);
  return p.lo + p.hi;
}
template <int K>
__device__ __forceinline__ float xor_max(float x) {
  const LanePair p = lane_pair<K>(x);
  return fmaxf(p.lo, p.hi);
}

// Maximum of two or three floats as one v_max / v_max3. fmaxf must quiet a
// signalling NaN operand, so the compiler puts a canonicalising max in front
// of every operand it cannot prove canonical (matrix-core results, lane
// swaps); these skip that and return the largest non-NaN operand, as fmaxf
// does for every input but a signalling NaN.
__device__ __forceinline__ float max_raw(float a, float b) {
#if __HIP_DEVICE_COMPILE__
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
#else
  return fmaxf(a, b);
#endif
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
#if __HIP_DEVICE_COMPILE__
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return fmaxf(fmaxf(a, b), c);
#endif
}
template <int K>
__device__ __forceinline__ float xor_max_raw(float x) {
  const LanePair p = lane_pair<K>(x);
  return max_raw(p.lo, p.hi);
}

// Sum over each aligned group of N consecutive lanes; every lane of the group
// receives the same (bitwise) result because each step adds commutative pairs.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kRowMirror>(x);
  if constexpr (N >= 32) x = xor_sum<16>(x);
  if constexpr (N >= 64) x = xor_sum<32>(x);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<kQuadXor1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<kQuadXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kRowMirror>(x));
  if constexpr (N >= 32) x = xor_max<16>(x);
  if constexpr (N >= 64) x = xor_max<32>(x);
  return x;
}

// Sum / max over the lanes that share lane % N (strides N, 2N, ... < 64).
template <int N>
__device__ __forceinline__ float stride_sum(float x) {
#pragma unroll
  for (int k = N; k < kWave; k <<= 1) x += __shfl_xor(x, k);
  return x;
}

template <int N>
__device__ __forceinline__ float stride_max(float x) {
#pragma unroll
  for (int k = N; k < kWave; k <<= 1) x = fmaxf(x, __shfl_xor(x, k));
  return x;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Raw buffer descriptor over [base, base + bytes) (gfx9 word 3: 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// Cache policy bits for K/V tile loads. K/V tiles are read exactly once per
// launch, so they are loaded non-temporal (nt): measured ~10% faster on MI355X
// than the default policy for the decode batch.
constexpr int kStreamPolicy = 2;

// 2^x on the transcendental unit (v_exp_f32); exact 0 for -inf, 1 for 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Division by a divisor fixed for a launch, as a multiply and a shift instead
// of the long integer-division sequence (Granlund and Montgomery, "Division
// by invariant integers using multiplication", PLDI 1994, theorem 4.2 with
// N = 31): for 1 <= d < 2^31, l = ceil(log2 d) and m = ceil(2^(31+l) / d),
// which fits 32 bits, floor(n / d) = floor(n * m / 2^(31+l)) for every
// 0 <= n < 2^31. Built on the host, read by the kernels as launch arguments.
struct FastDiv {
  uint32_t d, m, s;  // divisor, multiplier, shift 31 + l
  static FastDiv make(uint32_t d) {
    uint32_t l = 0;
    while (l < 31 && (1u << l) < d) ++l;
    const uint64_t num = 1ull << (31 + l);
    return FastDiv{d, (uint32_t)((num + d - 1) / d), 31 + l};
  }
  __host__ __device__ __forceinline__ int div(int n) const {  // 0 <= n < 2^31
    return (int)(((uint64_t)(uint32_t)n * m) >> s);
  }
  __host__ __device__ __forceinline__ int mod(int n) const { return n - div(n) * (int)d; }
};

// ---------------------------------------------------------------------------
// Split geometry of one sequence, shared by the host checks, the plan, the
// split kernel and the reduce. A sequence of length L carries Q query tokens
// (its last Q positions; query token i sits at L - Q + i and attends the
// positions up to its own) and, with a sliding window of W > 0 tokens, each
// query token attends only its W most recent positions [ATOM 4.2 for the Q
// new tokens of an MTP step; EchoLLMServing notes, section 4, for the
// window]. The splits cover [split_base, L).
// ---------------------------------------------------------------------------

// Start of the block holding the earliest token any query token attends.
__host__ __device__ inline int split_base(int L, int Q, int W) {
  if (W <= 0) return 0;
  const int first = L - Q - W + 1;
  return first > 0 ? first / kBlock * kBlock : 0;
}

// max(1, ceil((L - split_base) / T)).
__host__ __device__ inline int splits_of(int L, int Q, int W, int T) {
  const int n = (L - split_base(L, Q, W) + T - 1) / T;
  return n > 1 ? n : 1;
}

// splits_of with T as a FastDiv (L < 2^28, as the split-count bound ensures).
__device__ __forceinline__ int splits_of(int L, int Q, int W, const FastDiv &T) {
  const int n = T.div(L - split_base(L, Q, W) + (int)T.d - 1);
  return n > 1 ? n : 1;
}

// Largest L - split_base(L) over 0 <= L <= lmax: the longest split range.
__host__ __device__ inline int max_span(int lmax, int Q, int W) {
  if (W <= 0) return lmax;
  const int cap = Q + W + kBlock - 2;  // (Q + W - 1) + up to 15 leading tokens of a block
  return lmax < cap ? lmax : cap;
}

// ---------------------------------------------------------------------------
// Query tokens of a sequence. Every sequence has Q query tokens (rows s*Q ..
// s*Q + Q - 1 of q), or, with per-sequence offsets qs ([num_seqs + 1]), the
// packed rows [qs[s], qs[s+1]) of the n query tokens of the batch [EchoLLMServing
// notes, section 3, chunked prefill: one call for a batch that mixes prefill
// chunks and decodes]. The span is clamped into [0, n) and to at most
// PA_MAX_QUERY_TOKENS tokens, so that no row index leaves the packed arrays
// whatever the offsets hold.
// ---------------------------------------------------------------------------
struct QuerySpan {
  int first;  // row (token index) of query token 0
  int count;  // query tokens of the sequence
};

__device__ __forceinline__ QuerySpan query_span(const int32_t *qs, int s, int Q, int n) {
  if (qs == nullptr) return QuerySpan{s * Q, Q};
  const int a = min(max(qs[s], 0), n);
  const int b = min(max(qs[s + 1], a), min(n, a + PA_MAX_QUERY_TOKENS));
  return QuerySpan{a, b - a};
}

// Sequence owning packed query token t: the last s with qs[s] <= t (binary
// search over nondecreasing offsets; empty sequences share their offset with
// the next one, and the search lands on the last of them).
__device__ __forceinline__ int seq_of_token(const int32_t *qs, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qs[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// seq_of_token for a whole wave that asks about one token t (t the same in
// every lane): a 64-ary search. Each round, lane j probes the pivot lo + j *
// step of the remaining range [lo, hi) (one load per lane, all in flight at
// once), and the highest lane whose pivot is <= t narrows the range to its
// step: ceil(log64(num_seqs)) dependent loads instead of log2(num_seqs). Same
// result as seq_of_token: the largest s in [0, num_seqs) with qs[s] <= t, else
// 0; for offsets that are not nondecreasing, some s in [0, num_seqs).
__device__ __forceinline__ int seq_of_token_wave(const int32_t *qs, int num_seqs, int t) {
  int lo = 0, hi = num_seqs;
  const int lane = __lane_id();
  while (hi - lo > 1) {  // uniform: lo and hi come from the ballot
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const unsigned long long le = __ballot(idx < hi && qs[idx] <= t);
    const int j = le ? 63 - __clzll(le) : 0;
    lo += j * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

// Query rows (query token x query head of a KV head's group) per work item
// with packed queries: the plan lists one item per (split, block of this many
// rows) of a sequence.
constexpr int kPackedRows = 64;

}  // namespace pa
