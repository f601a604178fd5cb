/*
 * libpagedattn: decode-phase attention over a paged KV cache, for AMD
 * Instinct MI355X (gfx950).
 *
 * What it computes (the pages it follows):
 *   - "LLM Primer VI, chapter 8", section 8.1 (PagedAttention is virtual memory
 *     for KV): the KV cache is one flat pool of fixed 16-token blocks; each
 *     sequence owns a block table that maps its logical positions to physical
 *     block ids; attention takes the table as an extra input and gathers K and
 *     V through it.
 *   - "AMD ATOM Inference Engine" article, section 5.1 (BlockManager): blocks of
 *     16 tokens; new tokens are written into the KV cache before attention runs.
 *   - "EchoLLMServing inference framework notes", section 2 (PagedAttention
 *     V1 -> V2, FlashDecoding): online softmax over blocks of the context,
 *     split-K over the context with per-split temporaries (m, l, acc) merged by
 *     a second reduce kernel, and a split count that follows the context length
 *     (split_num = context_len / chunk, chunk 256 or 512 from profiling);
 *     section 3 (KV Cache INT8): INT8 cache with per-token scales, dequantised
 *     inside the attention kernel right after loading, and chunked prefill
 *     (prompts run in chunks beside decode steps; a mixed batch runs as two
 *     kernels or as one unified kernel that treats a decode as a prefill of
 *     length 1); section 4: sliding window attention as a way to bound decode
 *     cost.
 *   - "AMD ATOM Inference Engine" article, quick start (section 3): an FP8 KV
 *     cache (--kv_cache_dtype fp8); section 4.2 (decode scheduling):
 *     with MTP speculative decoding each decode step of a sequence carries
 *     mtp_k + 1 new tokens, each with its own KV slot.
 *
 * Conventions shared by every entry point:
 *   - Pool layout: k_cache, v_cache are [num_blocks][num_kv_heads][16][head_dim]
 *     of the cache dtype, so one (block, KV head) tile is 16*head_dim contiguous
 *     elements. INT8 and FP8 pools carry k_scale, v_scale
 *     [num_blocks][num_kv_heads][16] fp32, one scale per (token, KV head); an
 *     element's value is code * scale (FP8: the E4M3 value of the code).
 *   - Token t of sequence s lives in block block_tables[s][t / 16], row t % 16.
 *     A slot is block * 16 + row.
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - Query tokens: each sequence carries Q = num_query_tokens (1 to 4096) query
 *     tokens, its last Q positions: query token i sits at p = L - Q + i
 *     (L = context_lens[s], the new tokens already written) and attends the
 *     tokens t <= p (causal among the new tokens). With a sliding window of
 *     W = sliding_window > 0 tokens it attends only p - W < t <= p (its W most
 *     recent positions, its own included); W = 0 means no window. A query
 *     token with p < 0, or a sequence with L == 0, gives a zero output.
 *     q and out are [num_seqs][Q][num_q_heads][head_dim] (for Q = 1 the same
 *     memory as [num_seqs][num_q_heads][head_dim]). Q = 1 is a decode step,
 *     Q = mtp_k + 1 an MTP verification step, a larger Q a chunk of prefill
 *     over the cache. With packed queries (a query_start array, see
 *     paged_attn_plan) every sequence has its own count Q_s (0 to 4096), the
 *     same rule applies with Q = Q_s, and q, out and the partials' rows are
 *     packed as [N][num_q_heads] with N = sum Q_s, sequence s owning rows
 *     query_start[s] .. query_start[s+1] - 1: one call for a batch that mixes
 *     decodes and prefill chunks.
 *   - Logits are scale * q.k; softmax uses the natural exponent over the
 *     tokens a query token attends.
 *   - Splits cover [base, L), base = 16 * floor(max(0, L - Q - W + 1) / 16)
 *     with a window (the block holding the earliest attended token), else 0.
 *     Split j covers [base + j*T, min(base + (j+1)*T, L)), T = split_tokens (a
 *     positive multiple of 16, at most 4096); a sequence has
 *     max(1, ceil((L - base) / T)) splits (max(1, ceil(L / T)) without a
 *     window). Blocks before base are never read: their table entries may be
 *     anything (a cache may free them).
 *   - Partials: rows are (sequence, query token, query head), laid out
 *     [num_seqs][Q][num_q_heads]; m[row][j] is the maximum logit over the
 *     tokens of split j the row's query token attends (natural-log units),
 *     l[row][j] = sum exp(z - m), acc[row][j][:] = sum exp(z - m) v (not
 *     divided by l). A split with no such token stores m = -inf, l = 0,
 *     acc = 0. Entries past the sequence's split count are not written.
 *   - Pointers: every array argument is a device pointer owned by the caller;
 *     the library never allocates, frees or synchronises. q, k/v, k_cache,
 *     v_cache must be 16-byte aligned and contiguous in the layouts above.
 *   - Streams: work is enqueued on `stream` and nothing else, so a call can be
 *     captured in a HIP graph.
 *   - Errors: host-detectable problems return a negative PA_ERR_* code before
 *     anything is enqueued; a failed launch returns PA_ERR_LAUNCH. Device data
 *     is trusted for meaning but never read out of bounds: context lengths are
 *     clamped to [0, min(max_context_len, 16 * max_blocks_per_seq)], block ids
 *     to [0, num_blocks), and slots outside the pool are skipped, so bad data
 *     gives unspecified results, not memory faults.
 *   - Thread safety: the library keeps no mutable global state, except the
 *     per-device address table of paged_attn_decode_noalloc's fixed scratch
 *     (guarded by a mutex; see that call).
 *   - Launch trace (a debugging aid): PAGEDATTN_TRACE in the environment, read
 *     once per process, is a level. At 1 every entry point and kernel launch
 *     prints one line of its parameters and grid to stderr. At 2 the plan
 *     calls (paged_attn_plan, paged_decode_prepare and the calls built on
 *     them) also synchronise `stream` and copy the plan back to print its
 *     list, so level 2 breaks the no-synchronisation rule above and cannot
 *     run under graph capture. Unset or 0: no output and no effect.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_BLOCK_SIZE 16
#define PA_MAX_SPLIT_TOKENS 4096
#define PA_MAX_SEQS 65535
#define PA_MAX_QUERY_TOKENS 4096
#define PA_MAX_PACKED_QUERY_TOKENS (1 << 20)
#define PA_MAX_GROUP_MEMBERS 4
#define PA_MAX_SPLITS 65536  /* splits per sequence: the plan stores the split index in 16 bits */
/* Fixed device scratch of paged_attn_decode_noalloc, per GPU. */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Element types. PA_FP8 is OCP FP8 E4M3 (bias 7, no infinities, 0x7F / 0xFF
 * NaN, largest finite 448). */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_FP8 = 3 } pa_dtype;

/* Status codes. */
enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,      /* a required pointer is NULL */
  PA_ERR_DTYPE = -2,     /* unsupported dtype or dtype combination */
  PA_ERR_SHAPE = -3,     /* unsupported sizes (head_dim, head counts, ...) */
  PA_ERR_SPLIT = -4,     /* bad split_tokens, max_splits below what is needed, or more than
                            PA_MAX_SPLITS splits for the longest possible sequence */
  PA_ERR_WORKSPACE = -5, /* workspace smaller than pa_workspace_bytes() */
  PA_ERR_ALIGN = -6,     /* a pointer is not 16-byte aligned */
  PA_ERR_LAUNCH = -7,    /* the kernel launch failed (paged_attn_decode_noalloc: or its
                            device's fixed scratch could not be set up) */
  PA_ERR_SCRATCH = -8    /* paged_attn_decode_noalloc: the call needs more than
                            PA_NOALLOC_SCRATCH_BYTES of workspace */
};

/* Human-readable text for a status code (static storage). An auxiliary call
 * of this library's error convention; the pages define no interface, so it
 * follows no passage of theirs. */
const char *pa_strerror(int status);

/* Number of splits for a context of length context_len:
 * max(1, ceil(context_len / split_tokens)); 0 if split_tokens <= 0.
 * [EchoLLMServing notes, section 2, FlashDecoding split heuristic.] */
int32_t pa_num_splits(int32_t context_len, int32_t split_tokens);

/* Splits of the longest split range a sequence of length <= max_context_len
 * can have with num_query_tokens query tokens and the given window: the
 * max_splits the partials need [EchoLLMServing notes, section 2, FlashDecoding
 * split heuristic; section 4 for the window]. Without a window this is
 * pa_num_splits(max_context_len, split_tokens); with one the range is at
 * most min(max_context_len, Q + W + 14) tokens. 0 for bad arguments. */
int32_t pa_max_splits(int32_t max_context_len, int32_t num_query_tokens, int32_t sliding_window,
                      int32_t split_tokens);

/* Split size T (tokens) the library uses when a caller passes
 * split_tokens = 0 [EchoLLMServing notes, section 2: the split count follows
 * the context length, one split per 512 tokens in the notes' setting].
 * T starts at 256 KiB of K and V per (split, KV head) for every 8 query rows
 * of the KV head (rows = Q * g, g = num_q_heads / num_kv_heads; at least one
 * unit), i.e. 262144 * max(1, rows / 8) / (2 * head_dim * element bytes): 512
 * tokens for a 16-bit 128-dim cache and up to 15 rows, 1024 with 16 rows or
 * an INT8 cache, capped at 4096. With items = num_seqs * num_kv_heads *
 * ceil(Q * g / 64) * pa_max_splits(max_context_len, Q, W, T): T is halved,
 * down to 64, while items < 1024 (small batches
 * still fill the device); with more than 64 query rows per KV head it is then
 * doubled, up to 4096, while items stay >= 1024 (fewer partials to write);
 * with at most 8 query rows per KV head, or at most 16 with several query
 * tokens (a decode step, multi-token included) it then grows by 64 tokens at
 * a time, up to 4096, while items stay >= 2048 and
 * T * 2 * head_dim * element bytes (the K/V codes of a split and KV head)
 * stays <= 1 MiB.
 * Returns 0 for a head_dim other than 64 or 128, an unknown cache_dtype, bad
 * head counts or bad Q / W. Host-only arithmetic. */
int32_t pa_default_split_tokens(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t cache_dtype, int32_t max_context_len,
                                int32_t num_query_tokens, int32_t sliding_window);

/* Bytes of the plan paged_attn_plan writes (an int32 list of every split plus
 * a small header) [EchoLLMServing notes, section 2: one program per split of
 * every sequence, the split count following the context length]. */
size_t pa_sched_bytes(int32_t num_seqs, int32_t max_splits);

/* The same for packed queries (query_start given): the list then holds one
 * entry per (split, block of 64 query rows) of each sequence, at most
 * max_splits * (num_seqs + ceil(total_query_tokens * q_heads_per_kv / 64)). */
size_t pa_sched_bytes_packed(int32_t num_seqs, int32_t max_splits, int32_t total_query_tokens,
                             int32_t q_heads_per_kv);

/* Bytes of workspace paged_attn_decode needs [EchoLLMServing notes, section 2,
 * FlashDecoding: every split leaves temporaries (m, l, acc) for the reduce
 * kernel, and their size grows with the split count, which is why the split
 * count follows the context length]: scheduling scratch plus the partials
 * (m, l, acc) of num_seqs * num_query_tokens * num_q_heads rows of max_splits
 * splits each (fp32; acc has head_dim values per split). */
size_t pa_workspace_bytes(int32_t num_seqs, int32_t num_query_tokens, int32_t num_q_heads,
                          int32_t head_dim, int32_t max_splits);

/* The same for packed queries: partials of total_query_tokens * num_q_heads
 * rows and the packed plan. */
size_t pa_workspace_bytes_packed(int32_t num_seqs, int32_t total_query_tokens,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_splits);

/*
 * KV write ("reshape and cache") [ATOM article 5.1; Primer 8.1]: for every
 * token t < num_tokens with slot = slot_mapping[t] >= 0, copy k[t][h][:] and
 * v[t][h][:] into row slot % 16 of block slot / 16 for every KV head h.
 *   k, v          [num_tokens][num_kv_heads][head_dim] of in_dtype (PA_F32/PA_BF16)
 *   slot_mapping  [num_tokens] int64; negative entries are skipped
 *   k_cache, ...  pool of cache_dtype. cache_dtype == in_dtype: exact copy.
 *                 cache_dtype == PA_I8 [EchoLLMServing notes, section 3]: per
 *                 (token, head) a = max|x| (x widened to fp32), scale = a/127
 *                 (IEEE fp32 division), code = clamp(rint_half_even(x/scale),
 *                 -127, 127), a == 0 gives scale 0 and codes 0; the scale goes
 *                 to k_scale / v_scale (required for PA_I8 and PA_FP8, ignored
 *                 otherwise). cache_dtype == PA_FP8 [ATOM article, section 3]:
 *                 the same with scale = a/448 and code = the OCP E4M3 value
 *                 nearest to x/scale (ties to even, saturating at +-448).
 *   head_dim      64 or 128.
 * Duplicate slots in one call race (unspecified winner). Writing into a block
 * shared by several sequences is the caller's decision.
 */
int paged_kv_write(const void *k, const void *v, int32_t in_dtype, const int64_t *slot_mapping,
                   int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim, void *k_cache,
                   void *v_cache, float *k_scale, float *v_scale, int64_t num_blocks,
                   int32_t cache_dtype, hipStream_t stream);

/*
 * Plan of a decode step [EchoLLMServing notes, section 2: the split count of a
 * sequence follows its context length]: one small kernel reads context_lens on
 * the device and writes into `sched` the list of every split of the batch,
 * max(1, ceil((L_s - base_s) / T)) per sequence (see the split range above),
 * full splits first and then the last split of each sequence, longest first.
 * The list depends only on the lengths, the query counts, W, T and the length
 * bounds (and, with grouping, the tables), so one plan serves every attention
 * layer of a step that uses the same window.
 *   context_lens       [num_seqs] int32 (device)
 *   query_start        NULL: every sequence has num_query_tokens query tokens.
 *                      Else packed queries [EchoLLMServing notes, section 3,
 *                      chunked prefill: one call for a batch that mixes prefill
 *                      chunks and decodes, a decode being a chunk of length 1]:
 *                      [num_seqs + 1] int32 (device), 0 = query_start[0] <=
 *                      query_start[1] <= ... <= query_start[num_seqs] =
 *                      num_query_tokens; sequence s has Q_s = query_start[s+1]
 *                      - query_start[s] <= PA_MAX_QUERY_TOKENS query tokens (0
 *                      allowed), its last Q_s positions, packed as rows
 *                      query_start[s] .. query_start[s+1] - 1. Trusted device
 *                      data: spans are clamped into [0, num_query_tokens) so
 *                      that nothing is read or written out of bounds, and other
 *                      offsets give unspecified results.
 *   block_tables       [num_seqs][max_blocks_per_seq] int32 (device); read
 *                      only with group_members > 1, may be NULL otherwise
 *   max_blocks_per_seq, max_context_len   the bounds the decode call will use
 *   num_query_tokens   Q, 1 .. PA_MAX_QUERY_TOKENS; with query_start the total
 *                      N, 0 .. PA_MAX_PACKED_QUERY_TOKENS
 *   q_heads_per_kv     g = num_q_heads / num_kv_heads (1, 2, 4, 8 or 16); read
 *                      only with query_start (a packed plan lists blocks of 64
 *                      query rows, Q_s * g rows per sequence)
 *   sliding_window     W >= 0 (0: none)
 *   split_tokens       T, a positive multiple of 16 <= 4096 (the plan knows no
 *                      cache, so there is no default here: pass what the
 *                      decode call will use, e.g. pa_default_split_tokens())
 *   group_members      1, or up to PA_MAX_GROUP_MEMBERS [ATOM article 5.1-5.2:
 *                      blocks are reference counted and shared, e.g. a
 *                      prompt's prefix across its samples]: within aligned
 *                      runs of that many consecutive sequences, full splits j
 *                      that start on the same physical block as the previous
 *                      sequence's split j become one work item, its sequences
 *                      one per wave over shared, cached tile reads. Results do
 *                      not depend on it (each sequence still reads its own
 *                      table); it costs a few table reads per split in the plan.
 *                      Requires W = 0 and no query_start; a plan with groups
 *                      is used only when Q * g <= 16 rows (MFMA engine) or 8
 *                      (VALU engine), and is otherwise ignored like any
 *                      mismatched plan.
 *   sched              device scratch of pa_sched_bytes(num_seqs, max_splits)
 *                      bytes (pa_sched_bytes_packed(num_seqs, max_splits, N, g)
 *                      with query_start), max_splits >= pa_max_splits(
 *                      max_context_len, Q', W, T) with Q' = Q, or min(N, 4096)
 */
int paged_attn_plan(const int32_t *context_lens, const int32_t *query_start,
                    const int32_t *block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t max_context_len, int32_t num_query_tokens, int32_t q_heads_per_kv,
                    int32_t sliding_window, int32_t split_tokens, int32_t group_members,
                    int32_t *sched, hipStream_t stream);

/*
 * paged_kv_write followed by paged_attn_plan, in one launch: the two do not
 * depend on each other, so one kernel does both (its last workgroup plans, the
 * others write). Arguments, layouts and errors are those of the two calls
 * (split_tokens is required, as for the plan); the results are identical to
 * calling them in turn. Serves the start of a decode step, where the new tokens
 * (num_seqs * Q of them with several query tokens, N with packed queries) are
 * written and the batch's splits are listed.
 */
int paged_decode_prepare(const void *k, const void *v, int32_t in_dtype,
                         const int64_t *slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, void *k_cache, void *v_cache, float *k_scale,
                         float *v_scale, int64_t num_blocks, int32_t cache_dtype,
                         const int32_t *context_lens, const int32_t *query_start,
                         const int32_t *block_tables, int32_t num_seqs,
                         int32_t max_blocks_per_seq, int32_t max_context_len,
                         int32_t num_query_tokens, int32_t q_heads_per_kv,
                         int32_t sliding_window, int32_t split_tokens, int32_t group_members,
                         int32_t *sched, hipStream_t stream);

/*
 * Split-K decode kernel [EchoLLMServing notes, section 2]: for every sequence
 * s, query token i, query head h and split j of s, write the partials
 * (m, l, acc) of that split. The Q*g rows (query tokens x query heads) of a KV
 * head share every K/V load. Works through the split list of `sched`, which
 * paged_attn_plan must have written (on this stream, before this call) for the
 * same context_lens, query_start, num_seqs, max_blocks_per_seq,
 * max_context_len, Q (or N), W and split_tokens; a plan for another
 * split_tokens, num_seqs, length bound, query count, query layout or W is
 * ignored (nothing is written), other mismatches give unspecified results.
 *   q                 [num_seqs][num_query_tokens][num_q_heads][head_dim] of q_dtype
 *                     (PA_F32/PA_BF16); with query_start the packed
 *                     [num_query_tokens = N][num_q_heads][head_dim]
 *   k_cache, ...      pool as above; cache_dtype PA_F32 (q PA_F32), PA_BF16
 *                     (q PA_BF16), PA_I8 or PA_FP8 (q PA_BF16 or PA_F32;
 *                     k_scale and v_scale required). num_blocks < 2^31.
 *   block_tables      [num_seqs][max_blocks_per_seq] int32
 *   context_lens      [num_seqs] int32, each <= max_context_len
 *   query_start       NULL, or the packed query offsets (see paged_attn_plan)
 *   max_context_len   host bound on context_lens, sizes the launch grid
 *   sliding_window    W >= 0 (0: none)
 *   scale             logit scale (commonly 1/sqrt(head_dim))
 *   split_tokens      T, a positive multiple of 16 <= 4096, or 0 for
 *                     pa_default_split_tokens() (with Q' below for Q)
 *   max_splits        leading stride of the partials;
 *                     >= pa_max_splits(max_context_len, Q', W, T), Q' = Q, or
 *                     min(N, PA_MAX_QUERY_TOKENS) with query_start
 *   part_m, part_l    [num_seqs][num_query_tokens][num_q_heads][max_splits] fp32
 *                     ([N][num_q_heads][max_splits] with query_start)
 *   part_acc          [num_seqs][num_query_tokens][num_q_heads][max_splits][head_dim] fp32
 *                     ([N][num_q_heads][max_splits][head_dim]), 16-byte aligned
 *   sched             the plan (read only)
 * head_dim must be 64 or 128, num_q_heads / num_kv_heads one of 1, 2, 4, 8, 16,
 * num_query_tokens 1 .. PA_MAX_QUERY_TOKENS (N 0 .. PA_MAX_PACKED_QUERY_TOKENS
 * with query_start) and num_seqs at most PA_MAX_SEQS.
 */
int paged_attn_decode_partial(const void *q, int32_t q_dtype, int32_t num_seqs,
                              int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                              const void *k_cache, const void *v_cache, const float *k_scale,
                              const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
                              int32_t num_kv_heads, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              const int32_t *query_start, int32_t max_context_len,
                              int32_t sliding_window, float scale, int32_t split_tokens,
                              int32_t max_splits, float *part_m, float *part_l,
                              float *part_acc, const int32_t *sched, hipStream_t stream);

/*
 * Reduce kernel [EchoLLMServing notes, section 2]: merge the partials of every
 * row (sequence, query token, query head) over the splits of its sequence:
 *   M = max_j m_j over splits with l_j > 0, w_j = exp(m_j - M),
 *   out = sum_j w_j acc_j / sum_j w_j l_j   (0 when no split holds a token),
 * written as out_dtype (PA_F32, or PA_BF16 rounded to nearest even).
 *   part_*         as written by paged_attn_decode_partial with the same
 *                  query_start, num_query_tokens, sliding_window, split_tokens
 *                  (T > 0) and max_splits
 *   context_lens   [num_seqs] int32; each length is clamped to
 *                  [0, min(max_context_len, 16 * max_blocks_per_seq)] exactly
 *                  as the split kernel clamps it, so the reduce merges the
 *                  splits that call wrote and no others
 *   max_blocks_per_seq, max_context_len   the bounds given to the decode call
 *   query_start    NULL, or the packed query offsets (each packed row finds
 *                  its sequence by binary search over them)
 *   out            [num_seqs][num_query_tokens][num_q_heads][head_dim]
 *                  ([N][num_q_heads][head_dim] with query_start)
 */
int paged_attn_reduce(const float *part_m, const float *part_l, const float *part_acc,
                      const int32_t *context_lens, const int32_t *query_start, int32_t num_seqs,
                      int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                      int32_t max_blocks_per_seq, int32_t max_context_len,
                      int32_t sliding_window, int32_t split_tokens, int32_t max_splits,
                      void *out, int32_t out_dtype, hipStream_t stream);

/*
 * Whole decode step of one attention layer [EchoLLMServing notes, section 2,
 * FlashDecoding: the context is cut into splits whose count follows its
 * length, one program per split leaves (m, l, acc), a second reduce kernel
 * merges them; LLM Primer ch. 8, section 8.1: K and V are gathered through
 * the block table]: paged_attn_plan (no grouping) and
 * paged_attn_decode_partial into the caller's workspace, then
 * paged_attn_reduce into out (dtype = q_dtype). The partials live in the
 * workspace only for the length of the call.
 * The split count is pa_max_splits(max_context_len', Q, W, T) with
 * max_context_len' = min(max_context_len, 16 * max_blocks_per_seq) and
 * T = split_tokens (0: pa_default_split_tokens()). workspace must hold
 * pa_workspace_bytes(num_seqs, Q, num_q_heads, head_dim, that split count)
 * bytes (pa_workspace_bytes_packed(num_seqs, N, num_q_heads, num_kv_heads,
 * head_dim, that split count) with query_start, where Q' = min(N, 4096)
 * stands for Q), 256-byte aligned.
 */
int paged_attn_decode(const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_query_tokens,
                      int32_t num_q_heads, int32_t head_dim, const void *k_cache,
                      const void *v_cache, const float *k_scale, const float *v_scale,
                      int32_t cache_dtype, int64_t num_blocks, int32_t num_kv_heads,
                      const int32_t *block_tables, int32_t max_blocks_per_seq,
                      const int32_t *context_lens, const int32_t *query_start,
                      int32_t max_context_len, int32_t sliding_window, float scale,
                      int32_t split_tokens, void *out, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code being captured into a HIP graph, tight serving
 * loops, and harnesses that forbid hipMalloc. Same arguments (minus workspace
 * and workspace_bytes), results and errors as paged_attn_decode, the same
 * kernels; the plan and the partials go to a fixed scratch array of
 * PA_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on each GPU it is
 * called for, from that GPU's first call until the process ends.
 *   - The call allocates nothing: no hipMalloc, hipFree or allocating library
 *     routine. Its first call for a GPU looks up that GPU's copy of the array
 *     (hipGetSymbolAddress, with that GPU current), which loads it; make that
 *     first call outside a graph capture.
 *   - A call whose plan and partials need more than PA_NOALLOC_SCRATCH_BYTES
 *     (pa_workspace_bytes for its sizes) returns PA_ERR_SCRATCH before anything
 *     is enqueued; a GPU whose scratch cannot be set up gives PA_ERR_LAUNCH.
 *   - The GPU is the one `stream` belongs to. Every call on a GPU shares its
 *     array, and the array keeps the last call's contents: nothing in it has
 *     to start cleared (the plan kernel writes every word the split kernel
 *     reads, the split kernel every partial the reduce reads). Calls that
 *     overlap on one GPU (different streams, or host threads without an
 *     order between their streams) race on the array: order them.
 */
int paged_attn_decode_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs,
                              int32_t num_query_tokens, int32_t num_q_heads, int32_t head_dim,
                              const void *k_cache, const void *v_cache, const float *k_scale,
                              const float *v_scale, int32_t cache_dtype, int64_t num_blocks,
                              int32_t num_kv_heads, const int32_t *block_tables,
                              int32_t max_blocks_per_seq, const int32_t *context_lens,
                              const int32_t *query_start, int32_t max_context_len,
                              int32_t sliding_window, float scale, int32_t split_tokens,
                              void *out, hipStream_t stream);

/*
 * Measurement aid (not part of the attention path): read `bytes` (a multiple
 * of 16) from device buffer `src` once, using sink_words / 256 workgroups of
 * 256 threads (four waves; each wave reads whole 8 KiB chunks, two in flight);
 * each thread writes one word of its XOR to sink[sink_words]. Used to measure
 * the device's practical HBM read bandwidth next to the decode kernel's
 * (about 1024 to 3072 workgroups suit MI355X).
 */
int pa_hbm_read_probe(const void *src, size_t bytes, uint32_t *sink, int32_t sink_words,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
