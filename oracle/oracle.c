/*
 * Reference oracle for paged-KV decode attention. TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously correct CPU definition that the HIP
 * library is checked against. It shares no code, header, table or helper with
 * the GPU path and is never linked into it. Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it.
 *
 * Sources (the pages this follows):
 *   [Primer 8.1]  "LLM Primer VI, chapter 8: next-generation KV memory
 *                 management", section 8.1 "PagedAttention is virtual memory for
 *                 KV": KV is cut into fixed blocks of (usually) 16 tokens held in
 *                 one flat physical pool; a per-sequence block table maps logical
 *                 positions to physical block ids; the attention kernel takes the
 *                 table as an extra input and gathers K and V through it.
 *   [ATOM 5.1]    "AMD ATOM Inference Engine" article, section 5.1 (BlockManager):
 *                 16-token blocks by default, one block_table per Sequence.
 *   [Echo 2]      "EchoLLMServing inference framework notes", section 2,
 *                 "PagedAttention (V1 -> V2)" and "FlashDecoding": online softmax
 *                 over blocks of the context; split-K over the context where
 *                 each split leaves temporaries (m, l, acc) and a second reduce
 *                 kernel merges them.
 *   [Echo 3]      same notes, section 3, "KV Cache INT8 quantisation": INT8
 *                 cache with per-token scales, dequantised right after loading.
 *   [Echo 3, chunked prefill]  same notes, section 3, "Chunked Prefill"
 *                 scheduling: prompts run in chunks beside decode steps; a
 *                 mixed batch runs either as two kernels or as one unified
 *                 kernel that treats a decode as a prefill of length 1.
 *   [ATOM 3]      same article, quick start: every example runs with
 *                 --kv_cache_dtype fp8 (an FP8 KV cache).
 *   [ATOM 4.2]    "AMD ATOM Inference Engine" article, section 4.2 (decode
 *                 scheduling): with MTP speculative decoding every decode step
 *                 of a sequence carries mtp_k + 1 new tokens (the target token
 *                 and the draft tokens), each with its own KV slot.
 *   [Echo 4]      EchoLLMServing notes, section 4 (design trade-offs): sliding
 *                 window attention as an algorithm-level way to bound decode
 *                 cost; the ATOM article's model table lists it for GPT-OSS
 *                 and MiMo.
 *
 * Readings where the pages are silent (each one is listed with its reason in
 * the design notes of the repository):
 *   - cache layout [num_blocks][num_kv_heads][16][head_dim]; physical slot of
 *     token t of sequence s is block_tables[s][t/16]*16 + t%16; a negative
 *     slot in slot_mapping means "skip";
 *   - grouped-query heads: query head h reads KV head h / (Hq/Hkv);
 *   - logits are scale * q.k with a natural-exponent softmax over all tokens
 *     t < context_len (the token written this step included);
 *   - context_len 0 gives a zero output and empty partials (m=-inf, l=0, acc=0);
 *   - Q = num_query_tokens >= 1 query tokens per sequence (Q = mtp_k + 1): they
 *     are the last Q tokens of the context, query token i at position
 *     p = L - Q + i, and it attends the tokens t <= p (causal among the new
 *     tokens); with a sliding window of W > 0 tokens only p - W < t <= p
 *     (the W most recent positions, its own included); W = 0 means no window.
 *     A query with p < 0 attends nothing and gives a zero output;
 *   - per-sequence query counts [Echo 3, chunked prefill: a batch mixing
 *     prefill chunks and decodes in one call]: with query_start, sequence s
 *     has Q_s = query_start[s+1] - query_start[s] query tokens (0 allowed),
 *     stored as rows query_start[s] .. query_start[s+1]-1 of a packed q of
 *     [query_start[num_seqs]][num_q_heads][head_dim]; each follows the rule
 *     above with Q = Q_s (a decode sequence is the case Q_s = 1);
 *   - splits cover [base, L) with base = the start of the block holding the
 *     earliest attended token (0 without a window); split j holds tokens
 *     [base + j*T, min(base + (j+1)*T, L)), T = split_tokens, and there are
 *     max(1, ceil((L - base)/T)) splits (max(1, ceil(L/T)) without a window);
 *   - partials: m = max logit of the split, l = sum exp(z - m), acc =
 *     sum exp(z - m) * v, NOT divided by l;
 *   - INT8 quantiser per (token, KV head): a = max |x| in fp32, sc = a/127 (IEEE
 *     fp32 divide), q = clamp(round-half-even(x/sc), -127, 127), a = 0 -> q = 0;
 *     its input is the bf16/fp32 source widened exactly to fp32;
 *   - FP8 cache [ATOM 3]: OCP FP8 E4M3 (bias 7, no infinities, 0x7F/0xFF NaN,
 *     largest finite 448) with the same per-(token, KV head) fp32 scale,
 *     sc = a/448, code = e4m3(x/sc) rounded to nearest (ties to even),
 *     a = 0 -> codes 0; dequantised as e4m3 value * sc.
 *
 * Floating point: every attention quantity is computed in double. Build with
 * -ffp-contract=off and without -ffast-math (the INT8 quantiser relies on IEEE
 * fp32 division and the default round-to-nearest-even mode).
 */
#define _GNU_SOURCE /* syscall() for the NUMA placement helper at the end */
#include <errno.h>
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <sys/syscall.h>
#include <unistd.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_I8 = 2, OR_FP8 = 3 };
enum { OR_BLOCK = 16 };

/* bf16 is the top half of an IEEE binary32: widening is a 16-bit shift. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Value of an OCP FP8 E4M3 code: sign, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent 0 holds the subnormals m * 2^-9; S.1111.111 is NaN
 * (the format has no infinities). */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* The E4M3 code nearest to x (ties to the even mantissa); finite values past
 * the largest code, 448, saturate to +-448; NaN gives 0x7F. */
uint8_t oracle_e4m3_encode(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return 0x7F;
  float a = fabsf(x);
  if (a >= 448.0f) return sign | 0x7E;
  if (a < 0.015625f) { /* below 2^-6: subnormal codes m * 2^-9 (m = 8 is 2^-6) */
    float q = rintf(a * 512.0f);
    return sign | (uint8_t)q;
  }
  int e;
  frexpf(a, &e); /* a = f * 2^e with f in [0.5, 1) */
  e -= 1;        /* a = 1.xxx * 2^e, e in [-6, 8] */
  float q = rintf(ldexpf(a, 3 - e)); /* 8 .. 16: 1.xxx in eighths */
  if (q == 16.0f) {
    q = 8.0f;
    e += 1;
  }
  return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* Element idx of an array of `dtype` values, widened exactly to double. */
static double load_elem(const void *base, int dtype, int64_t idx) {
  if (dtype == OR_F32) return (double)((const float *)base)[idx];
  if (dtype == OR_BF16) return (double)bf16_bits_to_float(((const uint16_t *)base)[idx]);
  if (dtype == OR_FP8) return oracle_e4m3_decode(((const uint8_t *)base)[idx]);
  return (double)((const int8_t *)base)[idx];
}

/* Element idx of an fp32 or bf16 array, widened exactly to float. */
static float load_elem_f32(const void *base, int dtype, int64_t idx) {
  if (dtype == OR_F32) return ((const float *)base)[idx];
  return bf16_bits_to_float(((const uint16_t *)base)[idx]);
}

static size_t dtype_size(int dtype) { return dtype == OR_F32 ? 4 : dtype == OR_BF16 ? 2 : 1; }

/* Flat index of element d of (block b, kv head h, offset o) in the pool. */
static int64_t cache_index(int64_t b, int h, int o, int d, int num_kv_heads, int head_dim) {
  return ((b * num_kv_heads + h) * OR_BLOCK + o) * (int64_t)head_dim + d;
}

/* Flat index of the per-token scale of (block b, kv head h, offset o). */
static int64_t scale_index(int64_t b, int h, int o, int num_kv_heads) {
  return (b * num_kv_heads + h) * OR_BLOCK + o;
}

/* FP8 quantiser of one row [ATOM 3]: the INT8 recipe with 448 (the largest
 * E4M3 value) in place of 127 and E4M3 rounding in place of integer rounding. */
static void quantise_row_fp8(const void *src, int src_dtype, int64_t row_off, int head_dim,
                             uint8_t *dst, float *scale_out) {
  float a = 0.0f;
  for (int d = 0; d < head_dim; ++d) {
    float ax = fabsf(load_elem_f32(src, src_dtype, row_off + d));
    if (ax > a) a = ax;
  }
  float sc = a / 448.0f;
  for (int d = 0; d < head_dim; ++d)
    dst[d] = a == 0.0f ? 0 : oracle_e4m3_encode(load_elem_f32(src, src_dtype, row_off + d) / sc);
  *scale_out = sc;
}

/* INT8 quantiser of one row of head_dim values [Echo 3]. */
static void quantise_row(const void *src, int src_dtype, int64_t row_off, int head_dim,
                         int8_t *dst, float *scale_out) {
  float a = 0.0f;
  for (int d = 0; d < head_dim; ++d) {
    float ax = fabsf(load_elem_f32(src, src_dtype, row_off + d));
    if (ax > a) a = ax;
  }
  float sc = a / 127.0f;
  for (int d = 0; d < head_dim; ++d) {
    if (a == 0.0f) {
      dst[d] = 0;
      continue;
    }
    float x = load_elem_f32(src, src_dtype, row_off + d);
    float r = rintf(x / sc); /* default rounding mode: ties to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    dst[d] = (int8_t)r;
  }
  *scale_out = sc;
}

/*
 * KV write ("reshape and cache"): each new token's K and V rows go to the
 * physical slot slot_mapping[t] of the pool [ATOM 5.1, Primer 8.1].
 *   k, v        [num_tokens][num_kv_heads][head_dim] of in_dtype (0 fp32, 1 bf16)
 *   k_cache,... [num_blocks][num_kv_heads][16][head_dim] of cache_dtype
 *   k_scale,... [num_blocks][num_kv_heads][16] fp32, used when cache_dtype is INT8
 * INT8 and FP8 caches are quantised per (token, KV head); other caches need
 * in_dtype == cache_dtype and receive an exact copy.
 * Returns 0, or -1 on an unsupported combination or a slot outside the pool.
 */
int oracle_kv_write(const void *k, const void *v, int in_dtype, const int64_t *slot_mapping,
                    int64_t num_tokens, int num_kv_heads, int head_dim, void *k_cache,
                    void *v_cache, float *k_scale, float *v_scale, int64_t num_blocks,
                    int cache_dtype) {
  if (in_dtype != OR_F32 && in_dtype != OR_BF16) return -1;
  if (cache_dtype != OR_I8 && cache_dtype != OR_FP8 && cache_dtype != in_dtype) return -1;
  for (int64_t t = 0; t < num_tokens; ++t) {
    int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    int64_t b = slot / OR_BLOCK;
    int o = (int)(slot % OR_BLOCK);
    if (b >= num_blocks) return -1;
    for (int h = 0; h < num_kv_heads; ++h) {
      int64_t src_off = (t * num_kv_heads + h) * (int64_t)head_dim;
      int64_t dst_off = cache_index(b, h, o, 0, num_kv_heads, head_dim);
      if (cache_dtype == OR_I8) {
        int64_t si = scale_index(b, h, o, num_kv_heads);
        quantise_row(k, in_dtype, src_off, head_dim, (int8_t *)k_cache + dst_off, &k_scale[si]);
        quantise_row(v, in_dtype, src_off, head_dim, (int8_t *)v_cache + dst_off, &v_scale[si]);
      } else if (cache_dtype == OR_FP8) {
        int64_t si = scale_index(b, h, o, num_kv_heads);
        quantise_row_fp8(k, in_dtype, src_off, head_dim, (uint8_t *)k_cache + dst_off,
                         &k_scale[si]);
        quantise_row_fp8(v, in_dtype, src_off, head_dim, (uint8_t *)v_cache + dst_off,
                         &v_scale[si]);
      } else {
        size_t es = dtype_size(cache_dtype);
        memcpy((char *)k_cache + dst_off * es, (const char *)k + src_off * es, es * head_dim);
        memcpy((char *)v_cache + dst_off * es, (const char *)v + src_off * es, es * head_dim);
      }
    }
  }
  return 0;
}

/* Everything the decode definition reads. */
typedef struct {
  const void *q; /* [num_seqs][num_query_tokens][num_q_heads][head_dim] of q_dtype, or
                    [query_start[num_seqs]][num_q_heads][head_dim] with query_start */
  int q_dtype, num_q_heads, num_query_tokens;
  const int32_t *query_start; /* NULL: num_query_tokens per sequence */
  const void *k, *v;      /* pool, [num_blocks][num_kv_heads][16][head_dim] */
  const float *k_scale, *v_scale; /* [num_blocks][num_kv_heads][16], INT8 / FP8 only */
  int cache_dtype, num_kv_heads, head_dim;
  const int32_t *block_tables; /* [num_seqs][max_blocks_per_seq] */
  int max_blocks_per_seq;
  double scale;
  int window; /* sliding window in tokens, 0 = none */
} decode_args;

/* Tokens [*t0, *t1) that query token i of a sequence of length L attends
 * [ATOM 4.2, Echo 4]: its position is p = L - Q + i; t <= p, and with a
 * window W > 0 also t > p - W. */
static void query_range(int L, int Q, int W, int i, int *t0, int *t1) {
  int p = L - Q + i;
  if (p < 0) {
    *t0 = *t1 = 0;
    return;
  }
  *t1 = p + 1;
  *t0 = (W > 0 && p - W + 1 > 0) ? p - W + 1 : 0;
}

/* Dequantised element d of the K (which=0) or V (which=1) row of logical
 * token t of sequence s in KV head kv, reached through the block table. */
static double kv_elem(const decode_args *a, int which, int s, int kv, int t, int d) {
  int64_t b = a->block_tables[(int64_t)s * a->max_blocks_per_seq + t / OR_BLOCK];
  int o = t % OR_BLOCK;
  const void *base = which ? a->v : a->k;
  double x = load_elem(base, a->cache_dtype, cache_index(b, kv, o, d, a->num_kv_heads, a->head_dim));
  if (a->cache_dtype == OR_I8 || a->cache_dtype == OR_FP8) {
    const float *sc = which ? a->v_scale : a->k_scale;
    x *= (double)sc[scale_index(b, kv, o, a->num_kv_heads)];
  }
  return x;
}

/* Number of query tokens of sequence s; *first = the q row (token index) of
 * its query token 0. */
static int seq_queries(const decode_args *a, int s, int64_t *first) {
  if (a->query_start) {
    *first = a->query_start[s];
    return a->query_start[s + 1] - a->query_start[s];
  }
  *first = (int64_t)s * a->num_query_tokens;
  return a->num_query_tokens;
}

/* Logit z_t = scale * q[s][i][h] . k_t (query token i of sequence s). */
static double logit(const decode_args *a, int s, int i, int h, int t) {
  int kv = h / (a->num_q_heads / a->num_kv_heads);
  int64_t first;
  seq_queries(a, s, &first);
  int64_t row = (first + i) * a->num_q_heads + h;
  double dot = 0.0;
  for (int d = 0; d < a->head_dim; ++d) {
    double qd = load_elem(a->q, a->q_dtype, row * a->head_dim + d);
    dot += qd * kv_elem(a, 0, s, kv, t, d);
  }
  return a->scale * dot;
}

/* Softmax-weighted sums over tokens [t0, t1) of sequence s, query token i,
 * head h, taken relative to the maximum logit of that range:
 *   *m = max z_t,  *l = sum exp(z_t - m),  acc[d] = sum exp(z_t - m) v_t[d].
 * An empty range gives m = -inf, l = 0, acc = 0. */
static void weighted_sums(const decode_args *a, int s, int i, int h, int t0, int t1, double *m,
                          double *l, double *acc) {
  int kv = h / (a->num_q_heads / a->num_kv_heads);
  for (int d = 0; d < a->head_dim; ++d) acc[d] = 0.0;
  *l = 0.0;
  *m = -INFINITY;
  if (t1 <= t0) return;
  double *z = (double *)malloc(sizeof(double) * (size_t)(t1 - t0));
  double mx = -INFINITY;
  for (int t = t0; t < t1; ++t) {
    z[t - t0] = logit(a, s, i, h, t);
    if (z[t - t0] > mx) mx = z[t - t0];
  }
  double sum = 0.0;
  for (int t = t0; t < t1; ++t) {
    double w = exp(z[t - t0] - mx);
    sum += w;
    for (int d = 0; d < a->head_dim; ++d) acc[d] += w * kv_elem(a, 1, s, kv, t, d);
  }
  free(z);
  *m = mx;
  *l = sum;
}

/*
 * Decode attention by definition [Primer 8.1, Echo 2]: for each requested
 * (sequence, query token, query head) row,
 *   out = sum_t softmax_t(scale * q.k_t) v_t   over the tokens t the query
 * token attends (query_range), with K and V gathered token by token through
 * the block table and the whole range taken at once (no splitting). Rows are
 * given as index lists so that a caller can check a sample of a large batch;
 * out is [n_rows][head_dim]. query_start may be NULL (num_query_tokens per
 * sequence).
 */
void oracle_decode(const void *q, int q_dtype, int num_q_heads, int num_query_tokens,
                   int window, const int32_t *query_start, const void *k_cache,
                   const void *v_cache, const float *k_scale,
                   const float *v_scale, int cache_dtype, int num_kv_heads, int head_dim,
                   const int32_t *block_tables, int max_blocks_per_seq,
                   const int32_t *context_lens, double scale, const int32_t *row_seq,
                   const int32_t *row_tok, const int32_t *row_head, int64_t n_rows,
                   double *out) {
  decode_args a = {q, q_dtype, num_q_heads, num_query_tokens, query_start, k_cache, v_cache,
                   k_scale, v_scale, cache_dtype, num_kv_heads, head_dim, block_tables,
                   max_blocks_per_seq, scale, window};
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    int s = row_seq[r], i = row_tok[r], h = row_head[r];
    int64_t first;
    int Q = seq_queries(&a, s, &first);
    int t0, t1;
    query_range(context_lens[s], Q, window, i, &t0, &t1);
    double m, l;
    double *o = out + r * head_dim;
    weighted_sums(&a, s, i, h, t0, t1, &m, &l, o);
    for (int d = 0; d < head_dim; ++d) o[d] = l > 0.0 ? o[d] / l : 0.0;
  }
}

/* Number of splits of a context of length L: max(1, ceil(L / split_tokens)). */
int oracle_num_splits(int context_len, int split_tokens) {
  int n = (context_len + split_tokens - 1) / split_tokens;
  return n < 1 ? 1 : n;
}

/* First token of the split range of a sequence of length L with Q query
 * tokens and window W: the start of the block that holds the earliest token
 * any of its query tokens attends (0 without a window). */
int oracle_split_base(int context_len, int num_query_tokens, int window) {
  if (window <= 0) return 0;
  int first = context_len - num_query_tokens - window + 1;
  if (first < 0) first = 0;
  return first / OR_BLOCK * OR_BLOCK;
}

/*
 * Split-K partials [Echo 2, FlashDecoding]: split j of sequence s covers
 * tokens [base + j*T, min(base + (j+1)*T, L)), base = oracle_split_base, and
 * yields, for every (query token i, head h), (m_j, l_j, acc_j) as defined
 * for weighted_sums over the tokens of the split that query token attends.
 * Splits j >= max(1, ceil((L - base)/T)) are empty.
 * Layout: m, l [num_seqs][num_query_tokens][num_q_heads][max_splits];
 *         acc  [num_seqs][num_query_tokens][num_q_heads][max_splits][head_dim];
 * with query_start the leading [num_seqs][num_query_tokens] is the packed
 * [query_start[num_seqs]] of q.
 */
void oracle_decode_split(const void *q, int q_dtype, int num_seqs, int num_q_heads,
                         int num_query_tokens, int window, const int32_t *query_start,
                         const void *k_cache,
                         const void *v_cache, const float *k_scale, const float *v_scale,
                         int cache_dtype, int num_kv_heads, int head_dim,
                         const int32_t *block_tables, int max_blocks_per_seq,
                         const int32_t *context_lens, double scale, int split_tokens,
                         int max_splits, double *m, double *l, double *acc) {
  decode_args a = {q, q_dtype, num_q_heads, num_query_tokens, query_start, k_cache, v_cache,
                   k_scale, v_scale, cache_dtype, num_kv_heads, head_dim, block_tables,
                   max_blocks_per_seq, scale, window};
  /* The sequence and query token of every q row (token index). */
  int64_t n_tok = query_start ? query_start[num_seqs] : (int64_t)num_seqs * num_query_tokens;
  int *tok_seq = (int *)malloc(sizeof(int) * (size_t)(n_tok > 0 ? n_tok : 1));
  int *tok_idx = (int *)malloc(sizeof(int) * (size_t)(n_tok > 0 ? n_tok : 1));
  for (int s = 0; s < num_seqs; ++s) {
    int64_t first;
    int Q = seq_queries(&a, s, &first);
    for (int i = 0; i < Q; ++i) {
      tok_seq[first + i] = s;
      tok_idx[first + i] = i;
    }
  }
  int64_t jobs = n_tok * num_q_heads * max_splits;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < jobs; ++r) {
    int j = (int)(r % max_splits);
    int64_t row = r / max_splits; /* (token, h) */
    int64_t tok = row / num_q_heads;
    int s = tok_seq[tok], i = tok_idx[tok];
    int h = (int)(row % num_q_heads);
    int64_t first;
    int Q = seq_queries(&a, s, &first);
    int L = context_lens[s];
    int base = oracle_split_base(L, Q, window);
    int t0 = base + j * split_tokens;
    int t1 = t0 + split_tokens < L ? t0 + split_tokens : L;
    if (j >= oracle_num_splits(L - base, split_tokens)) t1 = t0; /* empty split */
    int q0, q1; /* the query token's own range */
    query_range(L, Q, window, i, &q0, &q1);
    if (q0 > t0) t0 = q0;
    if (q1 < t1) t1 = q1;
    weighted_sums(&a, s, i, h, t0, t1, &m[r], &l[r], acc + r * head_dim);
  }
  free(tok_seq);
  free(tok_idx);
}

/*
 * Reduce of split partials [Echo 2, FlashDecoding]: with M = max_j m_j over
 * non-empty splits and w_j = exp(m_j - M),
 *   out = sum_j w_j acc_j / sum_j w_j l_j.
 * Empty splits (l_j == 0) are skipped; no non-empty split gives out = 0.
 * Layouts as for oracle_decode_split; out is [num_rows][head_dim] where a row is
 * one (sequence, query token, head) triple.
 */
void oracle_merge(const double *m, const double *l, const double *acc, int64_t num_rows,
                  int max_splits, int head_dim, double *out) {
  for (int64_t r = 0; r < num_rows; ++r) {
    const double *mr = m + r * max_splits, *lr = l + r * max_splits;
    double M = -INFINITY;
    for (int j = 0; j < max_splits; ++j)
      if (lr[j] > 0.0 && mr[j] > M) M = mr[j];
    double den = 0.0;
    double *o = out + r * head_dim;
    for (int d = 0; d < head_dim; ++d) o[d] = 0.0;
    for (int j = 0; j < max_splits; ++j) {
      if (!(lr[j] > 0.0)) continue;
      double w = exp(mr[j] - M);
      den += w * lr[j];
      const double *aj = acc + (r * max_splits + j) * head_dim;
      for (int d = 0; d < head_dim; ++d) o[d] += w * aj[d];
    }
    for (int d = 0; d < head_dim; ++d) o[d] = den > 0.0 ? o[d] / den : 0.0;
  }
}

/* Threads the OpenMP loops above use (reported with the CPU baseline). */
int oracle_num_threads(void) { return omp_get_max_threads(); }

/* Thread binding of the OpenMP loops, as omp_get_proc_bind() reports it
 * (0 false, 1 true, 2 primary, 3 close, 4 spread); reported with the CPU
 * baseline. */
int oracle_proc_bind(void) { return (int)omp_get_proc_bind(); }

/* Spread the pages of [addr, addr + bytes) round robin over NUMA nodes
 * 0 .. nodes - 1 (the memory policy `numactl --interleave` gives a whole
 * process), moving pages that are already placed, so that the CPU baseline's
 * threads read a large pool from every node's memory rather than from the
 * node that first touched it. Returns 0, or the errno of the mbind call. */
int oracle_interleave(void *addr, size_t bytes, int nodes) {
  enum { MPOL_INTERLEAVE_ = 3, MPOL_MF_MOVE_ = 1 << 1 };
  unsigned long mask[16] = {0};
  if (nodes < 1 || nodes > (int)(8 * sizeof mask)) return EINVAL;
  for (int n = 0; n < nodes; ++n) mask[n / (8 * sizeof(unsigned long))] |= 1UL << (n % (8 * sizeof(unsigned long)));
  const uintptr_t page = (uintptr_t)sysconf(_SC_PAGESIZE);
  const uintptr_t a0 = (uintptr_t)addr & ~(page - 1);
  const uintptr_t a1 = ((uintptr_t)addr + bytes + page - 1) & ~(page - 1);
  if (syscall(SYS_mbind, (void *)a0, (unsigned long)(a1 - a0), MPOL_INTERLEAVE_, mask,
              (unsigned long)(8 * sizeof mask), MPOL_MF_MOVE_) != 0)
    return errno;
  return 0;
}
