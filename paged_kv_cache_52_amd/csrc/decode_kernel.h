// Split-K paged decode attention kernel for gfx950.
//
// One workgroup handles one (split j, KV head, sequence). Its NW wavefronts
// share the split's blocks; each wave streams whole (block, KV head) tiles of
// 16 x head_dim elements with 16-byte loads and keeps an online softmax
// [EchoLLMServing notes, section 2, PagedAttention V2] for every query head of
// the KV head's group, so each K/V byte is read from HBM once for all g query
// heads. K/V are gathered through the block table [LLM Primer ch. 8, 8.1].
//
// Lane layout inside a wave (for one 16-token tile of one KV head):
//   E   = elements per 16-byte load (8 bf16, 4 fp32, 16 int8)
//   LPR = head_dim / E   lanes that together hold one token row
//   RPI = 64 / LPR       token rows one load instruction covers
//   NI  = 16 / RPI       load instructions per tile (per K or per V)
// Lane l holds dims [E*(l % LPR), E*(l % LPR) + E) of tokens l / LPR + RPI*i,
// i < NI. One load instruction therefore reads 64 x 16 = 1024 contiguous bytes
// of the tile. q.k partial sums are combined across the LPR lanes of a row
// with DPP; the LPR lanes of a row then hold identical logits, and each of the
// RPI row groups keeps its own running (m, l, acc) over the tokens it owns.
// Row groups and waves are merged once, at the end of the split.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pa_common.h"

namespace pa {

struct DecodeParams {
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const float *k_scale;
  const float *v_scale;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *part_m;
  float *part_l;
  float *part_acc;
  const int32_t *sched;  // work list from the plan kernel (see kSchedHeader)
  int32_t num_bins;      // bins the first items are dealt over (one per compute unit)
  int32_t bin_wgs;       // workgroups per bin resident at launch
  int64_t num_blocks;
  int32_t num_seqs, num_q_heads, num_kv_heads, head_dim;
  int32_t max_blocks_per_seq, max_context_len;
  int32_t split_tokens, max_splits;
  int32_t num_query_tokens;  // Q query tokens per sequence (its last Q positions), or
                             // the packed total with query_start
  int32_t window;            // sliding window in tokens, 0 = none
  int32_t group;             // g = num_q_heads / num_kv_heads
  int32_t group_shift;       // log2(g) (g is a power of two)
  int32_t head_groups;  // uniform Q: workgroups per (split, KV head), rw row groups each
  int32_t rw;           // uniform Q: row groups of G rows per workgroup (1, 2 or 4)
  const int32_t *query_start;  // [num_seqs + 1] packed query offsets, or nullptr
  float scale_log2;     // scale * log2(e)
  // The divisors of a work item's set-up (split_tokens, num_kv_heads, items
  // per plan entry, num_bins) as multiply-and-shift constants: at launch every
  // resident wave runs that set-up at once on its compute unit's scalar unit,
  // before its first tile can be requested.
  FastDiv fd_split, fd_kv_heads, fd_entry, fd_bins;
};

// Row R (0 <= R < Q_s*g) of KV head kvh of a sequence whose query token 0 is
// packed row `first` is query token R / g, query head kvh*g + R % g; its q,
// out and partials row in [tokens][Hq].
__device__ __forceinline__ int64_t query_row(const DecodeParams &p, int first, int kvh, int R) {
  const int g = p.group;
  return ((int64_t)first + (R >> p.group_shift)) * p.num_q_heads + kvh * g + (R & (g - 1));
}

// Token ranges of the rows a workgroup handles. Query token i of the sequence
// attends [lo(i), hi(i)] (empty when its position is negative); the group's
// rows together attend [ulo, uhi], and a 16-token tile inside
// [lo_max, hi_min] is attended in full by every row (no mask needed).
struct RowRanges {
  int q0;      // position of query token 0: L - Q
  int window;  // W, 0 = none
  int first;   // q row (token index) of query token 0
  int ulo, uhi, lo_max, hi_min;

  __device__ __forceinline__ int lo(int i) const {
    const int pos = q0 + i;
    return window > 0 ? max(0, pos - window + 1) : 0;
  }
  __device__ __forceinline__ int hi(int i) const { return q0 + i; }
  __device__ __forceinline__ bool needs_mask(int tb) const {
    return tb < lo_max || tb + kBlock - 1 > hi_min;
  }
  // Rows [R0, R0 + nrows) with 2^gs query heads per KV head.
  __device__ __forceinline__ static RowRanges make(int L, int Q, int W, int gs, int R0, int nrows,
                                                  int first) {
    RowRanges r;
    r.q0 = L - Q;
    r.window = W;
    r.first = first;
    const int i0 = R0 >> gs, i1 = (R0 + nrows - 1) >> gs;
    r.ulo = r.lo(i0);
    r.uhi = r.hi(i1);
    r.lo_max = r.lo(i1);
    r.hi_min = r.hi(i0);
    return r;
  }
};

// Layout of the scheduling scratch written by the plan kernel:
//   [0] number of splits of the batch
//   [1] split_tokens, [2] num_seqs, [3] clamped max length, [4] query tokens
//   (per sequence, or the packed total), [5] window the plan was made for,
//   [6] group members (0: no group entries), [7] g with packed queries, else 0
//   then two words per entry, full splits first: (sequence << 16 | split),
//   read as unsigned (negative as int32 from sequence 32768 on), and
//   the sequence's clamped context length (minus the member count for a group
//   entry; the row block index with packed queries).
constexpr int kSchedHeader = 8;
// Largest number of bins the split kernel deals its first items over (one
// bin per compute unit).
constexpr int kMaxBins = 1024;

template <int QT, int CT, int D, int G>
struct DecodeShape {
  static constexpr int ELT = DtypeBytes<CT>::value;
  static constexpr int E = 16 / ELT;
  static constexpr int LPR = D / E;
  static constexpr int RPI = kWave / LPR;
  static constexpr int NI = kBlock / RPI;
  static constexpr int ROW_BYTES = D * ELT;
  static constexpr int TILE_BYTES = kBlock * ROW_BYTES;
  static constexpr bool DOT2 = (QT == PA_BF16 && CT == PA_BF16);
  static constexpr int QW = DOT2 ? E / 2 : E;  // q registers per head per lane
  static_assert(LPR >= 1 && LPR <= kWave && RPI * LPR == kWave && NI * RPI == kBlock, "layout");
};

// Registers of one in-flight tile: K and V rows plus INT8 per-token scales.
template <class S>
struct Tile {
  u32x4 k[S::NI];
  u32x4 v[S::NI];
  float ks[S::NI];
  float vs[S::NI];
};

template <int QT, int CT, int D, int G, int NW>
struct DecodeWave {
  using S = DecodeShape<QT, CT, D, G>;

  float qr[G][S::QW];  // q slice (fp32, pre-scaled) or packed bf16 pairs (DOT2)
  float m[G];          // running max of this row group, log2 units
  float l[G];          // running sum of exp2(z - m) over this lane's tokens
  float acc[G][S::E];  // running sum of exp2(z - m) * v, this lane's dims

  // Tile loads go through buffer descriptors built per tile in SGPRs: the
  // lane offset stays a 32-bit VGPR (no 64-bit address pairs), and the record
  // count is the tile size, so an offset outside the tile reads zeros.
  template <int POL>
  __device__ __forceinline__ void load_tile(Tile<S> &t, const DecodeParams &p, int blk, int kvh,
                                            int lane_off, int scale_off) {
    const int64_t tile = (int64_t)blk * p.num_kv_heads + kvh;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc((const char *)p.k_cache + tile * S::TILE_BYTES,
                                                S::TILE_BYTES);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc((const char *)p.v_cache + tile * S::TILE_BYTES,
                                                S::TILE_BYTES);
    // K (and its scales) first, then V: the q.k step waits only for K while
    // V and the next tile stay in flight.
#pragma unroll
    for (int i = 0; i < S::NI; ++i)
      t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + i * S::RPI * S::ROW_BYTES, 0,
                                                     POL);
    if constexpr (Quantised<CT>::value) {
      const __amdgpu_buffer_rsrc_t ksr = make_rsrc(p.k_scale + tile * kBlock, kBlock * 4);
#pragma unroll
      for (int i = 0; i < S::NI; ++i)
        t.ks[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                ksr, scale_off + i * S::RPI * 4, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < S::NI; ++i)
      t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off + i * S::RPI * S::ROW_BYTES, 0,
                                                     POL);
    if constexpr (Quantised<CT>::value) {
      const __amdgpu_buffer_rsrc_t vsr = make_rsrc(p.v_scale + tile * kBlock, kBlock * 4);
#pragma unroll
      for (int i = 0; i < S::NI; ++i)
        t.vs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                vsr, scale_off + i * S::RPI * 4, 0, 0));
    }
  }

  // 16 dims of an 8-bit row chunk (INT8 codes, or FP8 E4M3 codes decoded by
  // v_cvt_pk_f32_fp8), widened to fp32.
  __device__ __forceinline__ static void widen8(const u32x4 &w, float (&x)[16]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (CT == PA_FP8) {
        const uint32_t wk = w[k];
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wk, false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wk, true);
        x[4 * k + 0] = lo[0];
        x[4 * k + 1] = lo[1];
        x[4 * k + 2] = hi[0];
        x[4 * k + 3] = hi[1];
      } else {
        const int32_t v = (int32_t)w[k];
        x[4 * k + 0] = (float)((v << 24) >> 24);
        x[4 * k + 1] = (float)((v << 16) >> 24);
        x[4 * k + 2] = (float)((v << 8) >> 24);
        x[4 * k + 3] = (float)(v >> 24);
      }
    }
  }

  // Fold one tile (first token tb) into the running state. With need_mask,
  // row h keeps only the tokens in [lo[h], hi[h]] and the V rows of tokens
  // outside the group's [ulo, uhi] are dropped by select.
  __device__ __forceinline__ void consume(const Tile<S> &t, bool need_mask, int tb,
                                         const int (&lo)[G], const int (&hi)[G], int ulo,
                                         int uhi, int lane, float scale_log2) {
    const int r0 = lane / S::LPR;
    float z[S::NI][G];
    // q . k over this lane's E dims, for each owned token row and query head.
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
      if constexpr (S::DOT2) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int k = 0; k < S::E / 2; ++k) {
            // Copy the vector element to a scalar first: a bit cast applied
            // directly to an ext-vector element reads element 0 (clang).
            const uint32_t kw = t.k[i][k];
            const float qw = qr[h][k];
            a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, kw),
                                                __builtin_bit_cast(bf16x2, qw), a, false);
          }
          z[i][h] = a;
        }
      } else if constexpr (CT == PA_F32) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < S::E; ++e) a = fmaf(qr[h][e], __uint_as_float(t.k[i][e]), a);
          z[i][h] = a;
        }
      } else {  // 8-bit codes; the per-token scale multiplies the finished sum
        float x[16];
        widen8(t.k[i], x);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) a = fmaf(qr[h][e], x[e], a);
          z[i][h] = a;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < S::NI; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) z[i][h] = group_sum<S::LPR>(z[i][h]);
    if constexpr (S::DOT2) {
#pragma unroll
      for (int i = 0; i < S::NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) z[i][h] *= scale_log2;
    }
    if constexpr (Quantised<CT>::value) {
#pragma unroll
      for (int i = 0; i < S::NI; ++i)
#pragma unroll
        for (int h = 0; h < G; ++h) z[i][h] *= t.ks[i];
    }
    bool valid[S::NI];  // token inside the group's union
#pragma unroll
    for (int i = 0; i < S::NI; ++i) valid[i] = true;
    if (need_mask) {  // uniform
#pragma unroll
      for (int i = 0; i < S::NI; ++i) {
        const int tok = tb + r0 + i * S::RPI;
        valid[i] = tok >= ulo && tok <= uhi;
#pragma unroll
        for (int h = 0; h < G; ++h)
          z[i][h] = (tok >= lo[h] && tok <= hi[h]) ? z[i][h] : -INFINITY;
      }
    }

    // Online softmax update of this row group.
    float mnew[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = z[0][h];
#pragma unroll
      for (int i = 1; i < S::NI; ++i) bm = fmaxf(bm, z[i][h]);
      mnew[h] = fmaxf(m[h], bm);
      grow |= mnew[h] > m[h];
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float alpha = fast_exp2(m[h] - mnew[h]);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < S::E; ++e) acc[h][e] *= alpha;
        m[h] = mnew[h];
      }
    }
    float pr[S::NI][G];
#pragma unroll
    for (int i = 0; i < S::NI; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        pr[i][h] = fast_exp2(z[i][h] - m[h]);
        l[h] += pr[i][h];
      }

    // P . V over this lane's tokens and dims.
#pragma unroll
    for (int i = 0; i < S::NI; ++i) {
      float vf[S::E];
      if constexpr (CT == PA_BF16) {
#pragma unroll
        for (int k = 0; k < S::E / 2; ++k) {
          vf[2 * k] = bf16_lo(t.v[i][k]);
          vf[2 * k + 1] = bf16_hi(t.v[i][k]);
        }
      } else if constexpr (CT == PA_F32) {
#pragma unroll
        for (int e = 0; e < S::E; ++e) vf[e] = __uint_as_float(t.v[i][e]);
      } else {
        widen8(t.v[i], vf);
      }
      float w[G];
#pragma unroll
      for (int h = 0; h < G; ++h) w[h] = pr[i][h];
      if constexpr (Quantised<CT>::value) {
        const float vs = valid[i] ? t.vs[i] : 0.f;  // a poisoned scale must not leak
#pragma unroll
        for (int h = 0; h < G; ++h) w[h] *= vs;
      }
      // NaN * 0 would leak (an FP8 code can be NaN): select, not scale.
      if (CT != PA_I8 && need_mask && !valid[i]) {
#pragma unroll
        for (int e = 0; e < S::E; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < S::E; ++e) acc[h][e] = fmaf(w[h], vf[e], acc[h][e]);
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA engine (bf16 q; bf16 or INT8 cache; head_dim 128; any group g <= 16).
//
// The g query heads of a KV head make q.k^T and P.V small dense products, so
// one wave computes them on the matrix cores:
//   S[16 tokens][16 heads] = K_tile . q^T   4 x v_mfma_f32_16x16x32_bf16
//   O[16 heads][128 dims] += P . V_tile     8 x 2 x v_mfma_f32_16x16x16_bf16
// with the query heads padded to 16 (zero q). Lane l (c = l % 16, g = l / 16):
//   - K operand: token c, 8 dims per MFMA (bf16: dims 32i + 8g .. +8, so one
//     load instruction reads 64 contiguous bytes of each of the 16 rows;
//     INT8: dims 32g + 8i .. +8, two 16-byte loads per lane);
//   - q operand: head c, the same dims as K;
//   - S: head c, tokens 4g .. 4g+3 -- exactly how P must be laid out as the A
//     operand of P.V (rows heads, k = tokens 4g..4g+3), so P never moves
//     between lanes;
//   - V: rows 4g .. 4g+3, dims 8c .. 8c+7; v_perm (bf16) or byte conversion
//     (INT8) gathers, for output column block jj, element jj of the four rows
//     into the B operand;
//   - O: heads 4g .. 4g+3, dims 8c + jj.
// P is split into bf16 hi + lo parts (two MFMAs) so that the softmax weights
// keep ~16 significant bits. The reference max is shared by the four lane
// groups of a head and is only moved when a tile's max exceeds it by more than
// kRescaleSlack (exp2 arguments stay <= that slack). Each lane tests its own
// tokens against it, so the cross-row max steps run only when some lane's
// logits pass the limit; the true max is tracked per lane on the side, and
// at the end of the split the head's true max (across its four lanes) is the
// one the state is renormalised to.
//
// INT8 codes x are fed as u = x + 128 (x ^ 0x80 per byte), which bf16 holds
// exactly, and the bias is removed algebraically: q.x = q.u - 128 sum(q) per
// head, and sum_t w_t x_t = sum_t w_t u_t - 128 sum_t w_t with w_t = p_t *
// vscale_t; the per-token K scale multiplies the finished logit.
// ---------------------------------------------------------------------------

constexpr float kRescaleSlack = 8.0f;  // log2 units: weights stay below 2^8

template <int CT, int D>
struct MfmaEligible {
  static constexpr bool value = (CT == PA_BF16 || CT == PA_I8 || CT == PA_FP8) && D == 128;
};

template <int CT>
struct MfmaTile;
template <>
struct MfmaTile<PA_BF16> {
  u32x4 k[4];  // K operand fragments
  u32x4 v[4];  // V rows 4g + i, dims 8c .. 8c+7
};
template <>
struct MfmaTile<PA_I8> {
  u32x4 k[2];  // K codes: token c, dims 32g .. 32g+31
  u32x2 v[4];  // V codes: rows 4g + i, dims 8c .. 8c+7
  float ks1;   // K scale of token 4g + c % 4 (as loaded)
  float vs1;   // V scale of token 4g + c % 4
  f32x4 ks;    // K scales of tokens 4g .. 4g+3 (handed out from ks1 within the quad)
  f32x4 vs;    // V scales of tokens 4g .. 4g+3
};
template <>
struct MfmaTile<PA_FP8> : MfmaTile<PA_I8> {};  // same layout, E4M3 codes

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Unsigned byte k of w as fp32 (selected as v_cvt_f32_ubyte<k>).
template <int K>
__device__ __forceinline__ float ubyte_f32(uint32_t w) {
  return (float)((w >> (8 * K)) & 0xffu);
}

// E4M3 codes in bytes 0, 1 (HI = false) or 2, 3 (HI = true) of w as a bf16
// pair (v_cvt_scalef32_pk_bf16_fp8 with scale 1: exact, E4M3 fits bf16).
template <bool HI>
__device__ __forceinline__ uint32_t fp8pair_to_bf16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Biased INT8 codes (u = x + 128) of bytes 2h and 2h+1 of w, as a bf16 pair.
template <int H>
__device__ __forceinline__ uint32_t u8pair_to_bf16(uint32_t w) {
  return pack_bf16(ubyte_f32<2 * H>(w), ubyte_f32<2 * H + 1>(w));
}

// Byte K of each of two words, as biased codes, packed as a bf16 pair.
template <int K>
__device__ __forceinline__ uint32_t u8col_to_bf16(uint32_t w0, uint32_t w1) {
  return pack_bf16(ubyte_f32<K>(w0), ubyte_f32<K>(w1));
}

// LDS staging of the MFMA engine (bf16 cache): a 16-token K or V tile is 16
// rows of 256 bytes, stored kStageRow bytes apart to spread the lanes'
// 16-byte operand reads over the banks; two tiles (K and V) per buffer, two
// buffers. Measured on the prefill chunk batch: rows 256 bytes apart spend
// 50% of the busy cycles in bank conflicts, 272 bytes 22%, 288 bytes 12%
// (and 288 is the fastest of 272 .. 384).
constexpr int kStageRow = 288;
constexpr int kStageTile = kBlock * kStageRow;   // one K or V tile
constexpr int kStageBytes = 4 * kStageTile;      // 2 buffers x (K, V)

// LDS transpose read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 4a + e receives element e of the 8-byte rows addressed by lanes a,
// a + 4, a + 8 and a + 12 (measured lane layout on gfx950).
__device__ __forceinline__ s16x4 lds_read_tr16(const char *ptr) {
#if __HIP_DEVICE_COMPILE__
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(char *)ptr);
#else
  (void)ptr;
  return s16x4{0, 0, 0, 0};
#endif
}

template <int CT, int G>
struct MfmaWave {
  static constexpr int ELT = DtypeBytes<CT>::value;
  static constexpr int ROW = 128 * ELT;  // bytes per token row
  static constexpr int TILE = kBlock * ROW;
  u32x4 qB[4];   // q operand: head c (zero beyond the group), the K operand's dims
  f32x4 acc[8];  // O: heads 4g + r, dims 8c + jj
  float m;       // reference max (log2 units) of head c
  float mlim;    // m + kRescaleSlack: logits above it move m
  float mtrue;   // true running max of head c over this lane's tokens
  float l;       // sum of exp2(z - m) over this lane's tokens of head c
  float wsum;    // INT8: sum of exp2(z - m) * vscale over this lane's tokens
  float qbias;   // INT8: 128 * sum_d q[c][d]

  // Loads one tile. With live == false the descriptors have size 0: every
  // load is out of range, returns zeros and reads no memory.
  template <int POL>
  __device__ __forceinline__ void load_tile(MfmaTile<CT> &t, const DecodeParams &p, int blk,
                                            int kvh, int koff, int voff, int soff,
                                            bool live = true) {
    const int64_t tile = (int64_t)blk * p.num_kv_heads + kvh;
    const int tb = live ? TILE : 0;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc((const char *)p.k_cache + tile * TILE, tb);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc((const char *)p.v_cache + tile * TILE, tb);
    if constexpr (CT == PA_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 64 * i, 0, POL);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff + ROW * i, 0, POL);
    } else {
      const int sb = live ? kBlock * 4 : 0;
      const __amdgpu_buffer_rsrc_t ksr = make_rsrc(p.k_scale + tile * kBlock, sb);
      const __amdgpu_buffer_rsrc_t vsr = make_rsrc(p.v_scale + tile * kBlock, sb);
#pragma unroll
      for (int i = 0; i < 2; ++i)
        t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 16 * i, 0, POL);
      t.ks1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksr, soff, 0, 0));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        t.v[i] = __builtin_amdgcn_raw_buffer_load_b64(vr, voff + ROW * i, 0, POL);
      t.vs1 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsr, soff, 0, 0));
    }
  }

  // Logits of one tile for this lane's row (head c) and tokens 4g .. 4g+3, in
  // log2 units: S = K q^T on the matrix cores, then the K scale (INT8 / FP8)
  // and the softmax scale.
  __device__ __forceinline__ void scores(const MfmaTile<CT> &t, float (&z)[4],
                                         float scale_log2) const {
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (CT == PA_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, t.k[i]),
                                                    __builtin_bit_cast(bf16x8, qB[i]), sc, 0, 0,
                                                    0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // 8 codes: dims 32g + 8i .. +8 = bytes 8i .. 8i+7 of the lane's 32.
        u32x4 kb;
        if constexpr (CT == PA_I8) {
          const uint32_t w0 = t.k[i / 2][2 * (i % 2)] ^ 0x80808080u;
          const uint32_t w1 = t.k[i / 2][2 * (i % 2) + 1] ^ 0x80808080u;
          kb = u32x4{u8pair_to_bf16<0>(w0), u8pair_to_bf16<1>(w0), u8pair_to_bf16<0>(w1),
                     u8pair_to_bf16<1>(w1)};
        } else {  // E4M3 values are exact in bf16
          const uint32_t w0 = t.k[i / 2][2 * (i % 2)], w1 = t.k[i / 2][2 * (i % 2) + 1];
          kb = u32x4{fp8pair_to_bf16<false>(w0), fp8pair_to_bf16<true>(w0),
                     fp8pair_to_bf16<false>(w1), fp8pair_to_bf16<true>(w1)};
        }
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb),
                                                    __builtin_bit_cast(bf16x8, qB[i]), sc, 0, 0,
                                                    0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (CT == PA_BF16)
        z[r] = sc[r] * scale_log2;
      else if constexpr (CT == PA_I8)
        z[r] = (sc[r] - qbias) * t.ks[r] * scale_log2;
      else
        z[r] = sc[r] * t.ks[r] * scale_log2;
    }
  }

  // A tile at an edge of some row's range (tokens tb ..): this lane's row
  // keeps only tokens in [lo, hi]; V rows of tokens outside the group's
  // [ulo, uhi] are dropped by select (NaN * 0 would leak).
  __device__ __forceinline__ static void mask(MfmaTile<CT> &t, float (&z)[4], int tb, int lo,
                                              int hi, int ulo, int uhi, int g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tb + 4 * g + r;
      z[r] = (tok >= lo && tok <= hi) ? z[r] : -INFINITY;
      const bool used = tok >= ulo && tok <= uhi;
      if constexpr (CT == PA_BF16) {
        if (!used) t.v[r] = u32x4{0u, 0u, 0u, 0u};
      } else {
        if (!used) t.vs[r] = 0.f;
        if constexpr (CT == PA_FP8) {  // a NaN code must not meet a zero weight
          if (!used) t.v[r] = u32x2{0u, 0u};
        }
      }
    }
  }

  // Running max of head c over a step's logits (bm: this lane's maximum, of
  // logits that still need the factor `scale` > 0). The lane's true max takes
  // it as it is; only when some lane passes the reference by more than the
  // slack does the wave form each head's maximum over its four lane groups
  // (scaling commutes with the maximum, as rounding is monotonic) and rescale
  // the heads that passed.
  __device__ __forceinline__ void update_max(float bm, int g, float scale = 1.f) {
    bm *= scale;
    mtrue = max_raw(mtrue, bm);
    if (__any(bm > mlim)) {  // uniform
      bm = xor_max_raw<32>(xor_max_raw<16>(bm));
      rescale(bm > mlim ? bm : m, g);
    }
  }

  // Softmax weights of one tile's logits, added to l (and, INT8, wsum); for
  // INT8 / FP8 the V scale is folded in. P = hi + lo as bf16 pairs (tokens
  // (0, 1) and (2, 3) of the lane's four).
  __device__ __forceinline__ void weights(const MfmaTile<CT> &t, const float (&z)[4],
                                          uint32_t (&hi)[2], uint32_t (&lo)[2]) {
    float pz[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pz[r] = fast_exp2(z[r] - m);
    l += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    if constexpr (Quantised<CT>::value) {
#pragma unroll
      for (int r = 0; r < 4; ++r) pz[r] *= t.vs[r];
      if constexpr (CT == PA_I8) wsum += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    }
    hi[0] = pack_bf16(pz[0], pz[1]);
    hi[1] = pack_bf16(pz[2], pz[3]);
    lo[0] = pack_bf16(pz[0] - bf16_lo(hi[0]), pz[1] - bf16_hi(hi[0]));
    lo[1] = pack_bf16(pz[2] - bf16_lo(hi[1]), pz[3] - bf16_hi(hi[1]));
  }

  // FP8: V bytes of rows (0, 1) and (2, 3) interleaved per column pair, so
  // that one conversion yields a column's bf16 pair of two rows.
  __device__ __forceinline__ static void fp8_rows(const MfmaTile<CT> &t, uint32_t (&x01)[4],
                                                  uint32_t (&x23)[4]) {
    if constexpr (CT == PA_FP8) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        x01[2 * w] = __builtin_amdgcn_perm(t.v[1][w], t.v[0][w], 0x05010400u);
        x01[2 * w + 1] = __builtin_amdgcn_perm(t.v[1][w], t.v[0][w], 0x07030602u);
        x23[2 * w] = __builtin_amdgcn_perm(t.v[3][w], t.v[2][w], 0x05010400u);
        x23[2 * w + 1] = __builtin_amdgcn_perm(t.v[3][w], t.v[2][w], 0x07030602u);
      }
    }
  }

  // B operand of output column block JJ from one tile: element JJ (dim
  // 8c + JJ) of V rows (0, 1) and (2, 3) of the lane's four, as bf16 pairs.
  template <int JJ>
  __device__ __forceinline__ static void v_cols(const MfmaTile<CT> &t, const uint32_t (&x01)[4],
                                                const uint32_t (&x23)[4], uint32_t &b01,
                                                uint32_t &b23) {
    if constexpr (CT == PA_FP8) {
      // column JJ = byte JJ % 4 of word JJ / 4; x*[JJ / 2] holds columns
      // 2(JJ/2) and 2(JJ/2) + 1 in its low and high halves.
      b01 = fp8pair_to_bf16<(JJ & 1) != 0>(x01[JJ >> 1]);
      b23 = fp8pair_to_bf16<(JJ & 1) != 0>(x23[JJ >> 1]);
    } else if constexpr (CT == PA_BF16) {
      constexpr uint32_t sel = (JJ & 1) ? 0x07060302u : 0x05040100u;
      b01 = __builtin_amdgcn_perm(t.v[1][JJ >> 1], t.v[0][JJ >> 1], sel);
      b23 = __builtin_amdgcn_perm(t.v[3][JJ >> 1], t.v[2][JJ >> 1], sel);
    } else {
      constexpr int w = JJ >> 2;  // dims 8c + JJ live in byte JJ % 4 of word JJ / 4
      const uint32_t v0 = t.v[0][w] ^ 0x80808080u, v1 = t.v[1][w] ^ 0x80808080u;
      const uint32_t v2 = t.v[2][w] ^ 0x80808080u, v3 = t.v[3][w] ^ 0x80808080u;
      b01 = u8col_to_bf16<JJ & 3>(v0, v1);
      b23 = u8col_to_bf16<JJ & 3>(v2, v3);
    }
  }

  // O column block JJ += P . V over one tile (16 tokens, 16x16x16 MFMAs).
  template <int JJ>
  __device__ __forceinline__ void pv16(const MfmaTile<CT> &t, const uint32_t (&x01)[4],
                                       const uint32_t (&x23)[4], s16x4 phi, s16x4 plo) {
    uint32_t b01, b23;
    v_cols<JJ>(t, x01, x23, b01, b23);
    const s16x4 bv = __builtin_bit_cast(s16x4, u32x2{b01, b23});
    acc[JJ] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, bv, acc[JJ], 0, 0, 0);
    acc[JJ] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, bv, acc[JJ], 0, 0, 0);
  }

  // Fold one tile (first token tb) into the running state; need_mask: the
  // tile is at an edge of some row's range.
  __device__ __forceinline__ void consume(MfmaTile<CT> &t, bool need_mask, int tb, int lo,
                                          int hi, int ulo, int uhi, int g, float scale_log2) {
    if constexpr (Quantised<CT>::value) {
      // Each lane loaded the scales of one token of its quad's four (4g + c % 4);
      // every lane takes all four from its quad.
      t.ks = f32x4{dpp<0x00>(t.ks1), dpp<0x55>(t.ks1), dpp<0xAA>(t.ks1), dpp<0xFF>(t.ks1)};
      t.vs = f32x4{dpp<0x00>(t.vs1), dpp<0x55>(t.vs1), dpp<0xAA>(t.vs1), dpp<0xFF>(t.vs1)};
    }
    float z[4];
    scores(t, z, scale_log2);
    if (need_mask) mask(t, z, tb, lo, hi, ulo, uhi, g);  // uniform
    update_max(max3_raw(z[0], z[1], max_raw(z[2], z[3])), g);
    uint32_t h[2], lw[2];
    weights(t, z, h, lw);
    const s16x4 phi = __builtin_bit_cast(s16x4, u32x2{h[0], h[1]});
    const s16x4 plo = __builtin_bit_cast(s16x4, u32x2{lw[0], lw[1]});
    [[maybe_unused]] uint32_t x01[4], x23[4];
    fp8_rows(t, x01, x23);
    pv16<0>(t, x01, x23, phi, plo);
    pv16<1>(t, x01, x23, phi, plo);
    pv16<2>(t, x01, x23, phi, plo);
    pv16<3>(t, x01, x23, phi, plo);
    pv16<4>(t, x01, x23, phi, plo);
    pv16<5>(t, x01, x23, phi, plo);
    pv16<6>(t, x01, x23, phi, plo);
    pv16<7>(t, x01, x23, phi, plo);
  }

  // Staged tiles (bf16 K/V rows in LDS, kStageRow bytes apart).
  // Raw q.k sums of the two staged tiles whose K rows start at k0 and k1.
  __device__ __forceinline__ void scores2_lds(const char *k0, const char *k1, float (&z0)[4],
                                              float (&z1)[4], int c, int g) const {
    u32x4 a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = *reinterpret_cast<const u32x4 *>(k0 + c * kStageRow + 64 * i + 16 * g);
      b[i] = *reinterpret_cast<const u32x4 *>(k1 + c * kStageRow + 64 * i + 16 * g);
    }
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                  __builtin_bit_cast(bf16x8, qB[i]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b[i]),
                                                  __builtin_bit_cast(bf16x8, qB[i]), s1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z0[r] = s0[r];
      z1[r] = s1[r];
    }
  }

  // B operand of output column block JJ (dims 16JJ .. 16JJ + 15) from the V
  // tile at vb: this lane's column (dim 16JJ + c), tokens 4g .. 4g + 3. Lane
  // (c, g) addresses 4 dims of token 4g + c / 4, so that the transpose read
  // hands every lane its column.
  template <int JJ>
  __device__ __forceinline__ static s16x4 v_tr(const char *vb, int c, int g) {
    return lds_read_tr16(vb + (4 * g + (c >> 2)) * kStageRow + (16 * JJ + 4 * (c & 3)) * 2);
  }

  template <int JJ>
  __device__ __forceinline__ void pv32_lds(const char *v0, const char *v1, int c, int g,
                                           bf16x8 phi, bf16x8 plo) {
    const s16x4 a = v_tr<JJ>(v0, c, g), b = v_tr<JJ>(v1, c, g);
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{ua[0], ua[1], ub[0], ub[1]});
    acc[JJ] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, bv, acc[JJ], 0, 0, 0);
    acc[JJ] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, bv, acc[JJ], 0, 0, 0);
  }

  // Fold the staged tile pair (K0, V0) and (K1, V1), first tokens tb and
  // tb + 16, as one 32-token step. in0 / in1: the tile is in this wave's range
  // (else its logits are -inf); m0 / m1: it is at an edge of some row's range.
  // O column block JJ holds dims 16JJ .. 16JJ + 15 here (lane c: dim 16JJ + c).
  // V rows no row of the workgroup attends are zero in LDS, so a zero weight
  // never meets a NaN.
  template <int PRIO = 0>
  __device__ __forceinline__ void consume_pair_lds(const char *k0, const char *v0,
                                                   const char *k1, const char *v1, bool in0,
                                                   bool in1, bool m0, bool m1, int tb, int lo,
                                                   int hi, int c, int g, float scale_log2) {
    float z0[4], z1[4];
    // The matrix-core blocks (logits, then P.V) run one wave-priority level
    // above the walk's own (PRIO) and the softmax between them at PRIO, so
    // that a SIMD's waves tend to alternate between the two phases instead of
    // bunching up in one.
    // Both tiles' logits are computed (two independent MFMA chains); a tile
    // outside this wave's range then gets -inf by select, so whatever its
    // LDS rows hold never reaches a weight. The logits stay raw q.k sums (q
    // carries the scale's sign, so scale_log2 > 0 here): the maximum is taken
    // on them and scaled once, and each weight is exp2(fma(sum, scale, -m)).
    __builtin_amdgcn_s_setprio(PRIO + 1);
    scores2_lds(k0, k1, z0, z1, c, g);
    __builtin_amdgcn_s_setprio(PRIO);
    if (!(in0 && in1) || m0 || m1) {  // uniform
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z0[r] = in0 ? z0[r] : -INFINITY;
        z1[r] = in1 ? z1[r] : -INFINITY;
      }
      if (m0) mask_z(z0, tb, lo, hi, g);
      if (m1) mask_z(z1, tb + kBlock, lo, hi, g);
    }
    update_max(max3_raw(max3_raw(z0[0], z0[1], z0[2]), max3_raw(z0[3], z1[0], z1[1]),
                        max_raw(z1[2], z1[3])),
               g, scale_log2);
    uint32_t h0[2], l0[2], h1[2], l1[2];
    weights_plain(z0, h0, l0, scale_log2);
    weights_plain(z1, h1, l1, scale_log2);
    const bf16x8 phi = __builtin_bit_cast(bf16x8, u32x4{h0[0], h0[1], h1[0], h1[1]});
    const bf16x8 plo = __builtin_bit_cast(bf16x8, u32x4{l0[0], l0[1], l1[0], l1[1]});
    __builtin_amdgcn_s_setprio(PRIO + 1);
    pv32_lds<0>(v0, v1, c, g, phi, plo);
    pv32_lds<1>(v0, v1, c, g, phi, plo);
    pv32_lds<2>(v0, v1, c, g, phi, plo);
    pv32_lds<3>(v0, v1, c, g, phi, plo);
    pv32_lds<4>(v0, v1, c, g, phi, plo);
    pv32_lds<5>(v0, v1, c, g, phi, plo);
    pv32_lds<6>(v0, v1, c, g, phi, plo);
    pv32_lds<7>(v0, v1, c, g, phi, plo);
    __builtin_amdgcn_s_setprio(PRIO);
  }

  // Tokens of this lane's row outside [lo, hi] get -inf (tile at tb).
  __device__ __forceinline__ static void mask_z(float (&z)[4], int tb, int lo, int hi, int g) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tb + 4 * g + r;
      z[r] = (tok >= lo && tok <= hi) ? z[r] : -INFINITY;
    }
  }

  // weights() without cache scales (bf16 cache), from raw sums z: exp2(z *
  // scale - m) with one rounding.
  __device__ __forceinline__ void weights_plain(const float (&z)[4], uint32_t (&hi)[2],
                                                uint32_t (&lo)[2], float scale) {
    float pz[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pz[r] = fast_exp2(fmaf(z[r], scale, -m));
    l += (pz[0] + pz[1]) + (pz[2] + pz[3]);
    hi[0] = pack_bf16(pz[0], pz[1]);
    hi[1] = pack_bf16(pz[2], pz[3]);
    lo[0] = pack_bf16(pz[0] - bf16_lo(hi[0]), pz[1] - bf16_hi(hi[0]));
    lo[1] = pack_bf16(pz[2] - bf16_lo(hi[1]), pz[3] - bf16_hi(hi[1]));
  }

  // Move the reference max of head c to mnew (per lane) and rescale l (and
  // wsum) and the O rows (heads 4g + r get the factor computed in lane 4g + r).
  // All lanes of the wave must call it together.
  __device__ __forceinline__ void rescale(float mnew, int g) {
    const float alpha = fast_exp2(m - mnew);
    l *= alpha;
    wsum *= alpha;
    m = mnew;
    mlim = mnew + kRescaleSlack;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[jj][r] *= ar;
    }
  }
};


// Per-wave pass of the MFMA engine over tiles [wb0, wb1) of the split (tile n
// starts at token (b0 + n) * 16); leaves the wave's (m, l, acc) for the rows
// R0 .. R0 + nrows - 1 in LDS row `wave`.
// STAGED (bf16 cache, every wave of the workgroup on the same sequence and
// split, one row group per wave): the workgroup walks the union [sb0, sb1) of
// its waves' tiles together; each tile is loaded from memory once, by all
// 256 threads, into LDS (aliasing sm_acc, which is written only after the
// walk), and every wave reads its K and V operands from there, for the tiles
// of its own range. The tiles go two at a time: V rows of tokens outside the
// workgroup's [ulo_wg, uhi_wg] are stored as zeros, and P.V runs on 16x16x32
// instructions with V read by LDS transpose reads; the next pair's loads fly
// (in registers) while the current pair is consumed, two barriers per pair.
template <int QT, int CT, int D, int G, int NW, int POL, bool STAGED = false>
__device__ __forceinline__ void wave_pass_mfma(const DecodeParams &p, int s, int kvh, int R0,
                                               int nrows, const RowRanges &rr, int b0, int wb0,
                                               int wb1, int lane, int wave,
                                               float (&sm_m)[NW][G], float (&sm_l)[NW][G],
                                               float (&sm_acc)[NW][G][D], int sb0 = 0,
                                               int sb1 = 0, int ulo_wg = 0, int uhi_wg = -1,
                                               int s_own = -1, int pre_staged = 0,
                                               int pre_own = 0) {
  // Group entry (s_own >= 0, uniform): the workgroup stages sequence s's
  // blocks and this wave's rows belong to sequence s_own.
  const bool grouped = STAGED && s_own >= 0;
  using Wv = MfmaWave<CT, G>;
  Wv st;
  const int c = lane % 16, g = lane / 16;
  // This lane's S row: row R0 + c (padding rows beyond nrows keep zero q and
  // the group's token range).
  const bool row_ok = c < G && c < nrows;
  const int qi = (R0 + c) >> p.group_shift;
  const int lo = row_ok ? rr.lo(qi) : rr.ulo, hi = row_ok ? rr.hi(qi) : rr.uhi;
  const int64_t qrow = row_ok ? query_row(p, rr.first, kvh, R0 + c) : 0;
  float qs = 0.f;
  // Staged walks: the scale's sign goes into q (exact for bf16) and every
  // tile of the walk uses |scale| > 0 (a zero scale becomes the smallest
  // normal float, which leaves every weight at exactly 1).
  const uint32_t qsign = STAGED && p.scale_log2 < 0.f ? 0x80008000u : 0u;
  const float sl2 = STAGED ? fmaxf(fabsf(p.scale_log2), 1.17549435e-38f) : p.scale_log2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.qB[i] = u32x4{0u, 0u, 0u, 0u};
    if (row_ok) {
      const int dim0 = CT == PA_BF16 ? 32 * i + 8 * g : 32 * g + 8 * i;
      st.qB[i] = *(const u32x4 *)((const uint16_t *)p.q + qrow * D + dim0);
      if constexpr (STAGED) {
#pragma unroll
        for (int w = 0; w < 4; ++w) st.qB[i][w] ^= qsign;
      }
    }
    if constexpr (CT == PA_I8) {
#pragma unroll
      for (int k = 0; k < 4; ++k) qs += bf16_lo(st.qB[i][k]) + bf16_hi(st.qB[i][k]);
    }
  }
  if constexpr (CT == PA_I8) {
    qs = xor_sum<16>(qs);
    qs = xor_sum<32>(qs);
  }
  st.qbias = 128.f * qs;
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) st.acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = kNegBig;
  st.mlim = kNegBig + kRescaleSlack;
  st.mtrue = kNegBig;
  st.l = 0.f;
  st.wsum = 0.f;

  const int last_block = (int)(p.num_blocks - 1);
  const int koff = CT == PA_BF16 ? c * Wv::ROW + 16 * g : c * Wv::ROW + 32 * g;
  const int voff = 4 * g * Wv::ROW + 8 * Wv::ELT * c;
  // Scales: this lane reads token 4g + c % 4's (its quad shares them out).
  const int soff = CT == PA_BF16 ? 0 : 4 * (4 * g + c % 4);
  auto eat = [&](MfmaTile<CT> &t, int n) {
    const int tb = (b0 + n) * kBlock;
    st.consume(t, rr.needs_mask(tb), tb, lo, hi, rr.ulo, rr.uhi, g, sl2);
  };
  if constexpr (STAGED) {
    static_assert(CT == PA_BF16 && sizeof(float) * NW * G * D >= kStageBytes, "staging space");
    char *stage = reinterpret_cast<char *>(&sm_acc[0][0][0]);
    char *const K0 = stage, *const V0 = stage + kStageTile;
    char *const K1 = stage + 2 * kStageTile, *const V1 = stage + 3 * kStageTile;
    const int tid = threadIdx.x;  // NW * 64 = 256 threads, 16 bytes of a tile each
    const int srow = tid / 16, scol = (tid % 16) * 16;
    constexpr int TB = kBlock * 256;  // bytes of a bf16 K or V tile in memory
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // The walk, instantiated twice: a group entry's walk holds a raised wave
    // priority throughout (2, and 3 around its matrix-core blocks). Its items
    // are the launch's longest and share the SIMDs with plain decode items;
    // favouring them shortens the launch. Other staged walks use 0 and 1.
    auto walk = [&](auto prio) {
      constexpr int PRIO = decltype(prio)::value;
      constexpr bool kGroup = PRIO > 0;  // walk<2> runs group entries only
      __builtin_amdgcn_s_setprio(PRIO);
      for (int c0 = sb0; c0 < sb1; c0 += kWave) {
        const int c1 = min(sb1, c0 + kWave);
        // Lane i describes tile c0 + i of the chunk: its byte offset in the
        // pools and, as bits of wave-wide masks, whether this wave takes it,
        // whether its rows need no mask on it and whether it lies wholly inside
        // the workgroup's staged tokens. Each pair step then tests two bits.
        const int nl = c0 + lane;
        const bool lane_ok = nl < c1;
        int my_id = 0, own_id = 0;
        if (kGroup && c0 == 0) {  // a group walk's first chunk: read with the lengths
          my_id = lane_ok ? pre_staged : 0;
          own_id = lane_ok ? pre_own : 0;
        } else if (lane_ok) {
          my_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + b0 + nl];
          if (kGroup) own_id = p.block_tables[(int64_t)s_own * p.max_blocks_per_seq + b0 + nl];
        }
        const int tbl = (b0 + nl) * kBlock;
        // Group entry: this wave takes staged tile n only when it is its own
        // block too and lies wholly inside its rows' tokens and the staged
        // (unzeroed) tokens; the other tiles of its range follow the loop.
        const bool took_l = lane_ok && nl >= wb0 && nl < wb1 &&
                            (!kGroup || (own_id == my_id && tbl >= max(rr.ulo, ulo_wg) &&
                                          tbl + kBlock - 1 <= min(rr.uhi, uhi_wg)));
        const uint64_t took = __ballot(took_l);
        const uint64_t plain = __ballot(!rr.needs_mask(tbl));
        const uint64_t whole = __ballot(lane_ok && tbl >= ulo_wg && tbl + kBlock - 1 <= uhi_wg);
        // Physical block (clamped: a corrupt table entry reads a wrong but
        // existing block instead of faulting) as a byte offset into the pools;
        // with the clamp every fetch below stays inside the pool, so it is a
        // plain load rather than one through a tile-sized buffer descriptor.
        const uint64_t off_l =
            ((uint64_t)min(max(my_id, 0), last_block) * p.num_kv_heads + kvh) * (uint64_t)TB;
        const uint32_t off_lo = (uint32_t)off_l, off_hi = (uint32_t)(off_l >> 32);
        u32x4 kr0 = zero, vr0 = zero, kr1 = zero, vr1 = zero;
        auto fetch = [&](int i, u32x4 &kr, u32x4 &vr) {  // tile c0 + i
          const uint64_t off = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(off_hi, i) << 32) |
                               (uint32_t)__builtin_amdgcn_readlane(off_lo, i);
          kr = *reinterpret_cast<const u32x4 *>((const char *)p.k_cache + off + tid * 16);
          vr = *reinterpret_cast<const u32x4 *>((const char *)p.v_cache + off + tid * 16);
        };
        fetch(0, kr0, vr0);
        if (c0 + 1 < c1) fetch(1, kr1, vr1);
        for (int n = c0; n < c1; n += 2) {
          const int i = n - c0;
          // The loaded rows are stored as they are; at the workgroup's range
          // edges the rows outside it (and a missing second tile) are then
          // overwritten with zeros (a thread's two LDS stores land in order).
          *reinterpret_cast<u32x4 *>(K0 + srow * kStageRow + scol) = kr0;
          *reinterpret_cast<u32x4 *>(V0 + srow * kStageRow + scol) = vr0;
          *reinterpret_cast<u32x4 *>(K1 + srow * kStageRow + scol) = kr1;
          *reinterpret_cast<u32x4 *>(V1 + srow * kStageRow + scol) = vr1;
          if (((whole >> i) & 3u) != 3u) {  // uniform
            const int tok0 = (b0 + n) * kBlock + srow, tok1 = tok0 + kBlock;
            if (!(tok0 >= ulo_wg && tok0 <= uhi_wg)) {
              *reinterpret_cast<u32x4 *>(K0 + srow * kStageRow + scol) = zero;
              *reinterpret_cast<u32x4 *>(V0 + srow * kStageRow + scol) = zero;
            }
            if (!(n + 1 < c1 && tok1 >= ulo_wg && tok1 <= uhi_wg)) {
              *reinterpret_cast<u32x4 *>(K1 + srow * kStageRow + scol) = zero;
              *reinterpret_cast<u32x4 *>(V1 + srow * kStageRow + scol) = zero;
            }
          }
          __syncthreads();  // the pair is in LDS
          if (n + 2 < c1) fetch(i + 2, kr0, vr0);
          if (n + 3 < c1) fetch(i + 3, kr1, vr1);
          const uint32_t tk = (uint32_t)(took >> i) & 3u;
          if (tk != 0u) {  // uniform
            const uint32_t pl = (uint32_t)(plain >> i);
            st.template consume_pair_lds<PRIO>(K0, V0, K1, V1, tk & 1u, tk >> 1, !(pl & 1u),
                                               !(pl & 2u), (b0 + n) * kBlock, lo, hi, c, g, sl2);
          }
          __syncthreads();  // every wave is done with the pair
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    if (grouped)
      walk(std::integral_constant<int, 2>{});
    else
      walk(std::integral_constant<int, 0>{});
    if (grouped) {
      // O's columns leave the staged loop in the transpose-read order (block
      // jj = dims 16jj .. 16jj+15, lane c: dim 16jj + c); the unstaged tiles
      // below add in the register order (lane c: dims 8c .. 8c+7). Reorder
      // through this wave's own LDS slot (the staging space is free now).
      float *slot = &sm_acc[wave][0][0];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) slot[(4 * g + r) * D + 16 * jj + c] = st.acc[jj][r];
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) st.acc[jj][r] = slot[(4 * g + r) * D + 8 * c + jj];
      // The tiles of this wave's range it did not take from LDS, from its own
      // blocks (same test as in the staged loop, one lane per tile; the wave
      // then visits only the tiles it did not take).
      for (int c0 = wb0; c0 < wb1; c0 += kWave) {
        const int nl = c0 + lane;
        const bool lane_ok = nl < min(wb1, c0 + kWave);
        int mine = 0, staged_id = -1;
        if (lane_ok) {
          mine = p.block_tables[(int64_t)s_own * p.max_blocks_per_seq + b0 + nl];
          if (nl >= sb0 && nl < sb1)
            staged_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + b0 + nl];
        }
        const int tbl = (b0 + nl) * kBlock;
        const bool took_l = nl >= sb0 && nl < sb1 && mine == staged_id &&
                            tbl >= max(rr.ulo, ulo_wg) && tbl + kBlock - 1 <= min(rr.uhi, uhi_wg);
        for (uint64_t rest = __ballot(lane_ok && !took_l); rest != 0; rest &= rest - 1) {
          const int i = __builtin_ctzll(rest);
          MfmaTile<CT> t;
          st.template load_tile<0>(t, p, min(max(__builtin_amdgcn_readlane(mine, i), 0), last_block),
                                   kvh, koff, voff, soff);
          eat(t, c0 + i);
        }
      }
    }
  } else
  // Tiles in chunks of 64: the chunk's physical block ids sit one per lane.
  for (int c0 = wb0; c0 < wb1; c0 += kWave) {
    const int c1 = min(wb1, c0 + kWave);
    int my_id = 0;
    if (lane < c1 - c0) my_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + b0 + c0 + lane];
    // Physical block of tile n (clamped: a corrupt table entry reads a wrong
    // but existing block instead of faulting).
    auto block_of = [&](int n) {
      return min(max(__builtin_amdgcn_readlane(my_id, min(n - c0, kWave - 1)), 0), last_block);
    };
    MfmaTile<CT> t;
    for (int n = c0; n < c1; ++n) {
      st.template load_tile<POL>(t, p, block_of(n), kvh, koff, voff, soff);
      eat(t, n);
    }
  }
  // Renormalise to the head's true max, the largest of its four lanes' (every
  // lane takes part: rescale reads other lanes' factors), then sum l over the
  // four lane groups.
  st.rescale(fmaxf(xor_max_raw<32>(xor_max_raw<16>(st.mtrue)), st.m), g);
  const float lt = xor_sum<32>(xor_sum<16>(st.l));
  if constexpr (CT == PA_I8) {
    // Remove the code bias from O: row 4g + r loses 128 * (its head's wsum).
    const float wt = xor_sum<32>(xor_sum<16>(st.wsum));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float bias = 128.f * __shfl(wt, 4 * g + r);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) st.acc[jj][r] -= bias;
    }
  }
  if (lane < G) {
    sm_m[wave][lane] = st.m;
    sm_l[wave][lane] = lt;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * g + r;
    if (h < G) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        sm_acc[wave][h][STAGED && !grouped ? 16 * jj + c : 8 * c + jj] = st.acc[jj][r];
    }
  }
}

// Per-wave pass of the VALU engine (every dtype and head_dim); same contract.
template <int QT, int CT, int D, int G, int NW, int POL>
__device__ __forceinline__ void wave_pass_valu(const DecodeParams &p, int s, int kvh, int R0,
                                               int nrows, const RowRanges &rr, int b0, int wb0,
                                               int wb1, int lane, int wave,
                                               float (&sm_m)[NW][G], float (&sm_l)[NW][G],
                                               float (&sm_acc)[NW][G][D]) {
  using S = DecodeShape<QT, CT, D, G>;
  using W = DecodeWave<QT, CT, D, G, NW>;
  W st;
  // Token range of each row (padding rows past nrows take the group's).
  int lo[G], hi[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int qi = (R0 + h) >> p.group_shift;
    lo[h] = h < nrows ? rr.lo(qi) : rr.ulo;
    hi[h] = h < nrows ? rr.hi(qi) : rr.uhi;
  }
  // q slice for this lane's dims (zero for padding rows).
  {
    const int c = lane % S::LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = (h < nrows ? query_row(p, rr.first, kvh, R0 + h) : 0) * D;
      if (h >= nrows) {
#pragma unroll
        for (int k = 0; k < S::QW; ++k) st.qr[h][k] = 0.f;
      } else if constexpr (S::DOT2) {
        const u32x4 w = *(const u32x4 *)((const uint16_t *)p.q + row + c * S::E);
#pragma unroll
        for (int k = 0; k < S::E / 2; ++k) st.qr[h][k] = __uint_as_float(w[k]);
      } else if constexpr (QT == PA_F32) {
#pragma unroll
        for (int e = 0; e < S::E; e += 4) {
          const u32x4 w = *(const u32x4 *)((const float *)p.q + row + c * S::E + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) st.qr[h][e + k] = __uint_as_float(w[k]) * p.scale_log2;
        }
      } else {  // bf16 q against a non-bf16 cache: widen
#pragma unroll
        for (int e = 0; e < S::E; e += 8) {
          const u32x4 w = *(const u32x4 *)((const uint16_t *)p.q + row + c * S::E + e);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            st.qr[h][e + 2 * k] = bf16_lo(w[k]) * p.scale_log2;
            st.qr[h][e + 2 * k + 1] = bf16_hi(w[k]) * p.scale_log2;
          }
        }
      }
      st.m[h] = kNegBig;
      st.l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < S::E; ++e) st.acc[h][e] = 0.f;
    }
  }

  const int last_block = (int)(p.num_blocks - 1);  // the host checks 0 < num_blocks < 2^31
  auto eat = [&](const Tile<S> &t, int n) {
    const int tb = (b0 + n) * kBlock;
    st.consume(t, rr.needs_mask(tb), tb, lo, hi, rr.ulo, rr.uhi, lane, p.scale_log2);
  };
  const int lane_off = (lane / S::LPR) * S::ROW_BYTES + (lane % S::LPR) * 16;
  const int scale_off = (lane / S::LPR) * 4;
  // Tiles in chunks of 64: the chunk's physical block ids sit one per lane.
  Tile<S> t;
  for (int c0 = wb0; c0 < wb1; c0 += kWave) {
    const int c1 = min(wb1, c0 + kWave);
    int my_id = 0;
    if (lane < c1 - c0) my_id = p.block_tables[(int64_t)s * p.max_blocks_per_seq + b0 + c0 + lane];
    for (int n = c0; n < c1; ++n) {
      const int blk = min(max(__builtin_amdgcn_readlane(my_id, n - c0), 0), last_block);
      st.template load_tile<POL>(t, p, blk, kvh, lane_off, scale_off);
      eat(t, n);
    }
  }

  // Merge the RPI row groups of the wave.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = stride_max<S::LPR>(st.m[h]);
    const float f = fast_exp2(st.m[h] - M);
    st.l[h] = stride_sum<S::LPR>(st.l[h] * f);
#pragma unroll
    for (int e = 0; e < S::E; ++e) st.acc[h][e] = stride_sum<S::LPR>(st.acc[h][e] * f);
    st.m[h] = M;
  }
  if (lane < S::LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < S::E; ++e) sm_acc[wave][h][lane * S::E + e] = st.acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = st.m[h];
      sm_l[wave][h] = st.l[h];
    }
  }
}

// One work item for KV head kvh: split j of sequence s for the rw row groups
// of G rows starting at row R0 (rows R0 .. min(R_end, R0 + rw*G) - 1 of the
// KV head's Q_s*g rows), or, for a group entry (group > 0), split j of the
// `group` sequences s, s+1, ... whose splits share tiles, one row group (all
// Q*g <= G rows) each, rw = NW. The NW waves split into rw row groups of
// tw = NW / rw waves: the tw waves of a row group divide the tiles of the
// split that its rows reach, and merge their states in LDS; different row
// groups read their tiles at about the same time (with rw > 1 through the
// caches, not streamed) and write their own partials. len is the sequence's
// clamped length (not used for group entries). Contains two workgroup
// barriers.
template <int QT, int CT, int D, int G, int NW>
__device__ __forceinline__ void process_split(const DecodeParams &p, int s, int len, int j,
                                              int kvh, int R0, int R_end, int rw, int group,
                                              int lane, int wave, float (&sm_m)[NW][G],
                                              float (&sm_l)[NW][G], float (&sm_acc)[NW][G][D]) {
  // rw and NW are powers of two: tw = NW / rw waves per row group.
  const int tws = __builtin_ctz(NW) - __builtin_ctz(rw);
  const int tw = 1 << tws;
  const int rg = wave >> tws, tp = wave & (tw - 1);  // this wave's row group and tile share
  const int W = p.window;
  // Context length, clamped so that no read leaves the table or the pool.
  const int lmax = (int)min((int64_t)p.max_context_len, (int64_t)p.max_blocks_per_seq * kBlock);
  // The row group's sequence, rows and split range.
  auto seq_of = [&](int g) { return group > 0 ? s + g : s; };
  const int s_rg = min(seq_of(rg), p.num_seqs - 1);
  const QuerySpan qsp = query_span(p.query_start, s_rg, p.num_query_tokens, p.num_query_tokens);
  const int Q = qsp.count;
  auto rows_of = [&](int g) {  // rows of row group g (<= 0: a padding row group)
    if (group > 0) return g < group ? min(G, Q * p.group) : 0;
    return min(G, R_end - (R0 + g * G));
  };
  // A group entry (made only without a window) walks split j from block
  // j * T / 16 whatever the lengths, so the first 64 table words of the
  // staged sequence and of this wave's own are read before the lengths, in
  // the same round trip (each read stays inside its table row).
  int pre_staged = 0, pre_own = 0;
  if (group > 0) {
    const int col = j * (p.split_tokens / kBlock) + lane;
    if (col < p.max_blocks_per_seq) {
      pre_staged = p.block_tables[(int64_t)s * p.max_blocks_per_seq + col];
      pre_own = p.block_tables[(int64_t)s_rg * p.max_blocks_per_seq + col];
    }
  }
  const int L = group > 0 ? max(0, min(p.context_lens[s_rg], lmax)) : len;
  const int base = split_base(L, Q, W);
  const bool has_split = Q > 0 && j < splits_of(L, Q, W, p.fd_split);
  const int t0 = base + j * p.split_tokens;  // a multiple of 16
  const int t1 = min(t0 + p.split_tokens, L);
  const int b0 = t0 / kBlock;
  const int Rg = group > 0 ? 0 : R0 + rg * G;  // first row of this wave's row group
  const int nrows = has_split ? rows_of(rg) : 0;
  // Tiles of the split the row group's rows reach: tokens [ta, tz].
  RowRanges rr{};
  int wb0 = 0, wb1 = 0;
  if (nrows > 0) {
    rr = RowRanges::make(L, Q, W, p.group_shift, Rg, nrows, qsp.first);
    const int ta = max(t0, rr.ulo), tz = min(t1 - 1, rr.uhi);
    if (tz >= ta) {
      const int first = (ta - t0) / kBlock, count = (tz - t0) / kBlock - first + 1;
      const int per = (count + tw - 1) >> tws;
      wb0 = first + min(count, tp * per);
      wb1 = first + min(count, tp * per + per);
    }
  }
  // Tiles that several row groups read stay cached; a lone row group streams.
  // Four row groups of one sequence (bf16, 16 rows each: prefill chunks)
  // share each tile through LDS.
  constexpr bool kStageable = QT == PA_BF16 && CT == PA_BF16 && D == 128 &&
                              G == 16 && NW == 4;
  if constexpr (QT == PA_BF16 && MfmaEligible<CT, D>::value) {
    if (kStageable && rw == NW) {
      // The workgroup's tiles: those any of its rows reach; for a group
      // entry, the blocks of the split the group's first sequence holds (each
      // member takes those it shares).
      int sb0 = 0, sb1 = 0, ulo = 0, uhi = -1;
      const int all = min(R_end - R0, rw * G);
      if (group > 0) {
        const int t1s = min(t0 + p.split_tokens, max(0, min(p.context_lens[s], lmax)));
        if (t1s > t0) {
          sb1 = (t1s - t0 + kBlock - 1) / kBlock;
          ulo = t0;
          uhi = t1s - 1;
        }
      } else if (has_split && all > 0) {
        const RowRanges ru = RowRanges::make(L, Q, W, p.group_shift, R0, all, qsp.first);
        ulo = max(t0, ru.ulo);
        uhi = min(t1 - 1, ru.uhi);
        if (uhi >= ulo) {
          sb0 = (ulo - t0) / kBlock;
          sb1 = (uhi - t0) / kBlock + 1;
        }
      }
      wave_pass_mfma<QT, CT, D, G, NW, 0, kStageable>(
          p, group > 0 ? s : s_rg, kvh, Rg, nrows, rr, b0, wb0, wb1, lane, wave, sm_m, sm_l,
          sm_acc, sb0, sb1, ulo, uhi, group > 0 ? s_rg : -1, pre_staged, pre_own);
    } else if (rw > 1)
      wave_pass_mfma<QT, CT, D, G, NW, 0>(p, s_rg, kvh, Rg, nrows, rr, b0, wb0, wb1, lane, wave,
                                          sm_m, sm_l, sm_acc);
    else
      wave_pass_mfma<QT, CT, D, G, NW, kStreamPolicy>(p, s_rg, kvh, Rg, nrows, rr, b0, wb0, wb1,
                                                      lane, wave, sm_m, sm_l, sm_acc);
  } else {
    if (rw > 1)
      wave_pass_valu<QT, CT, D, G, NW, 0>(p, s_rg, kvh, Rg, nrows, rr, b0, wb0, wb1, lane, wave,
                                          sm_m, sm_l, sm_acc);
    else
      wave_pass_valu<QT, CT, D, G, NW, kStreamPolicy>(p, s_rg, kvh, Rg, nrows, rr, b0, wb0, wb1,
                                                      lane, wave, sm_m, sm_l, sm_acc);
  }
  __syncthreads();

  // Merge the tw waves of each row group and write the split's partials: one
  // thread per row finds the row's common max, turns sm_m into the waves'
  // factors 2^(m_w - M) and writes (m, l); then all threads sum the rows'
  // dims, four per thread. A row group without the split writes nothing.
  // Group entries come from uniform-Q plans only: member g's rows start at
  // packed row (s + g) * Q.
  auto out_row = [&](int g, int h) {
    const int first = group > 0 ? (s + g) * p.num_query_tokens : qsp.first;
    return query_row(p, first, kvh, (group > 0 ? 0 : R0 + g * G) + h) * p.max_splits + j;
  };
  auto live = [&](int g) {  // rows of row group g that have this split
    if (group == 0) return has_split ? rows_of(g) : 0;
    if (g >= group || s + g >= p.num_seqs) return 0;
    const int Lg = max(0, min(p.context_lens[s + g], lmax));
    return j < splits_of(Lg, Q, W, p.fd_split) ? rows_of(g) : 0;
  };
  // The row threads also leave each row's partials index in sm_row (-1: the
  // row has no split here), so that the dims loop below needs no table reads
  // or divisions of its own.
  __shared__ int64_t sm_row[NW][G];
  if ((int)threadIdx.x < rw * G) {
    const int g = threadIdx.x / G, h = threadIdx.x % G;
    int64_t row = -1;
    if (h < live(g)) {
      const int w0 = g * tw;
      float M = sm_m[w0][h];
      for (int w = 1; w < tw; ++w) M = fmaxf(M, sm_m[w0 + w][h]);
      float lsum = 0.f;
      for (int w = 0; w < tw; ++w) {
        const float f = fast_exp2(sm_m[w0 + w][h] - M);
        sm_m[w0 + w][h] = f;
        lsum = fmaf(f, sm_l[w0 + w][h], lsum);
      }
      row = out_row(g, h);
      p.part_l[row] = lsum;
      p.part_m[row] = lsum > 0.f ? M * kLn2 : -INFINITY;
    }
    sm_row[g][h] = row;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < rw * G * (D / 4); idx += NW * kWave) {
    const int g = idx / (G * (D / 4));
    const int h = idx / (D / 4) % G, d = (idx % (D / 4)) * 4;
    const int64_t row = sm_row[g][h];
    if (row < 0) continue;
    const int w0 = g * tw;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < tw; ++w) {
      const float f = sm_m[w0 + w][h];
      const f32x4 v = *(const f32x4 *)&sm_acc[w0 + w][h][d];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = fmaf(f, v[e], a[e]);
    }
    *(f32x4 *)(p.part_acc + row * D + d) = a;
  }
}

// The MFMA engine on 16-bit and FP8 caches fits 128 VGPRs, i.e. four waves per
// SIMD (16 per CU) for latency hiding; the INT8 one needs more and runs three.
constexpr int kMfmaWavesPerEu = 4;

template <int QT, int CT, int D, int G, int NW>
__device__ __forceinline__ void decode_split_body(const DecodeParams &p);

template <int QT, int CT, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_split_kernel(
    const DecodeParams p) {
  decode_split_body<QT, CT, D, G, NW>(p);
}

// The same kernel with the MFMA engine's occupancy bound (bf16 q, bf16 or FP8
// cache, head_dim 128).
template <int QT, int CT, int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(
    kMfmaWavesPerEu))) void decode_split_kernel_mfma(const DecodeParams p) {
  decode_split_body<QT, CT, D, G, NW>(p);
}

// Work item k of the list (k < the list's item count): split j of sequence s
// for KV head kvh (and, uniform Q, its row set), or a group entry. Contains
// workgroup barriers; every thread of the workgroup calls it with the same k.
template <int QT, int CT, int D, int G, int NW>
__device__ __forceinline__ void decode_item(const DecodeParams &p, int k,
                                            float (&sm_m)[NW][G], float (&sm_l)[NW][G],
                                            float (&sm_acc)[NW][G][D]) {
  const bool packed = p.query_start != nullptr;
  const int lmax = (int)min((int64_t)p.max_context_len, (int64_t)p.max_blocks_per_seq * kBlock);
  const int lane = lane_id();
  // Wave index as a scalar, so that per-wave ranges and loop counters stay in
  // SGPRs and the tile loop runs without exec masking.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // k = entry * per_entry + e, e = set * Hkv + kvh (per_entry items per entry).
  const int ent = p.fd_entry.div(k);
  const int e = k - ent * (int)p.fd_entry.d;
  const int kvh = p.fd_kv_heads.mod(e);
  const int packed_entry = p.sched[kSchedHeader + 2 * ent];
  const int word1 = p.sched[kSchedHeader + 2 * ent + 1];
  // The sequence index is clamped so that no entry can send a read out of
  // bounds; process_split ignores a split index past a sequence's end.
  const int s = min((int)((uint32_t)packed_entry >> 16), p.num_seqs - 1);
  const int j = packed_entry & 0xffff;
  if (!packed) {
    // word1 is the sequence's length, or minus the member count of a group
    // entry (made only with one row group per KV head).
    const int group = word1 < 0 ? min(-word1, NW) : 0;
    const int rows = p.num_query_tokens * p.group;
    const int R0 = p.fd_kv_heads.div(e) * p.rw * G;
    process_split<QT, CT, D, G, NW>(p, s, max(word1, 0), j, kvh, R0, rows,
                                    group > 0 ? NW : p.rw, group, lane, wave, sm_m, sm_l,
                                    sm_acc);
  } else {
    // word1 is the row block: rows [rb * kPackedRows, ...) of the sequence's
    // Q_s * g rows, in passes of up to NW row groups.
    const int L = max(0, min(p.context_lens[s], lmax));
    const QuerySpan qsp = query_span(p.query_start, s, p.num_query_tokens, p.num_query_tokens);
    const int rows = qsp.count * p.group;
    const int r0 = max(word1, 0) * kPackedRows;
    const int r1 = min(rows, r0 + kPackedRows);
    for (int R0 = r0; R0 < r1; R0 += NW * G) {
      const int nr = min(NW * G, r1 - R0);
      int rw = 1;
      while (rw < NW && rw * G < nr) rw <<= 1;
      if (R0 > r0) __syncthreads();  // the previous pass has read the LDS state
      process_split<QT, CT, D, G, NW>(p, s, L, j, kvh, R0, r1, rw, 0, lane, wave, sm_m, sm_l,
                                      sm_acc);
    }
  }
}

// Items are dealt over num_bins bins in snake order (round r of num_bins
// consecutive items goes to bins 0, 1, ... for even r and back for odd r), so
// that, with the plan's list running from the longest items to the shortest,
// every bin gets about the same number of bytes. Item i of bin b:
__device__ __forceinline__ int64_t bin_item(int b, int i, int nb) {
  return (int64_t)i * nb + ((i & 1) ? nb - 1 - b : b);
}


// Split kernel. Work item k is entry sched[kSchedHeader + 2*(k / per_entry)]
// of the list the plan kernel wrote, for KV head k % Hkv and (uniform Q) the
// set (k % per_entry) / Hkv of rw row groups of the KV head's Q*g rows
// (per_entry = Hkv * head_groups); with packed queries an entry names its
// block of kPackedRows rows itself and per_entry = Hkv. A plan made for
// another split size, batch, length bound, query count, window or query
// layout counts as an empty list.
//
// Which workgroup runs which item. The grid has a workgroup per possible
// item. The first num_bins * bin_wgs of them are resident at launch, and the
// dispatcher places workgroups w, w + num_bins, ... on one compute unit (one
// bin per compute unit). Those take the first num_bins * bin_wgs items of the
// list dealt over the bins in snake order (workgroup w: item
// bin_item(w % num_bins, w / num_bins)), so that, with the list running from
// the longest items to the shortest, every compute unit starts with about
// the same bytes: they read at about the same rate when all are busy, and a
// unit dealt the longest items would otherwise set the kernel's length. Each
// later workgroup w, started when a slot frees up, takes item w (as does
// every workgroup of a plan with group entries). Every item has exactly one
// workgroup whatever the placement, which only decides the balance;
// workgroups past the list exit at once.
template <int QT, int CT, int D, int G, int NW>
__device__ __forceinline__ void decode_split_body(const DecodeParams &p) {
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  __shared__ __align__(16) float sm_acc[NW][G][D];

  const bool packed = p.query_start != nullptr;
  const int per_entry = packed ? p.num_kv_heads : p.num_kv_heads * p.head_groups;
  const int lmax = (int)min((int64_t)p.max_context_len, (int64_t)p.max_blocks_per_seq * kBlock);
  // A plan made with group entries needs uniform query counts, every
  // sequence's rows in one row group (Q*g <= G), and a wave per member.
  static_assert(NW >= PA_MAX_GROUP_MEMBERS, "a group entry takes one wave per member");
  // The header's words are read together and compared without short
  // circuits, so that no read waits for the one before it.
  int hd[kSchedHeader];
#pragma unroll
  for (int i = 0; i < kSchedHeader; ++i) hd[i] = p.sched[i];
  const bool plan_ok = (hd[1] == p.split_tokens) & (hd[2] == p.num_seqs) & (hd[3] == lmax) &
                       (hd[4] == p.num_query_tokens) & (hd[5] == p.window) &
                       (hd[7] == (packed ? p.group : 0)) &
                       ((hd[6] <= 1) | (!packed & (p.num_query_tokens * p.group <= G)));
  const int n_items = plan_ok ? hd[0] * per_entry : 0;
  const int w = blockIdx.x;
  const int nb = p.num_bins;
  // Group entries keep the list order: the entries of the groups that share
  // one prompt's blocks follow each other and run side by side.
  const bool dealt = hd[6] <= 1 && w < nb * p.bin_wgs;
  const int64_t k = dealt ? bin_item(p.fd_bins.mod(w), p.fd_bins.div(w), nb) : (int64_t)w;
  if (k >= n_items) return;
  decode_item<QT, CT, D, G, NW>(p, (int)k, sm_m, sm_l, sm_acc);
}

// Launch helper instantiated per (q dtype, cache dtype) in the decode_*.hip units.
// Waves per workgroup (they share one split).
constexpr int kDecodeWaves = 4;

// Compute units of the device `stream` runs on (cached per device: a fixed
// property).
int compute_units(hipStream_t stream);

// Resident workgroups per compute unit of a kernel (its registers and LDS
// decide; cached per kernel by the caller).
int resident_per_cu(const void *kernel, int threads);

// Launch tracing: PAGEDATTN_TRACE in the environment (read once per process)
// is the level. At 1 every entry point and kernel launch prints one line of
// its parameters and grid to stderr; at 2 a plan is also waited for and its
// list printed. 0 or unset: silent.
int trace_level();
void trace(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
const char *dtype_name(int dtype);

template <int QT, int CT, int D, int G>
hipError_t launch_decode(DecodeParams p, int64_t max_items, hipStream_t stream) {
  constexpr int NW = kDecodeWaves;
  constexpr bool kMfmaBound = QT == PA_BF16 && (CT == PA_BF16 || CT == PA_FP8) && D == 128;
  const void *kernel;
  if constexpr (kMfmaBound)
    kernel = reinterpret_cast<const void *>(&decode_split_kernel_mfma<QT, CT, D, G, NW>);
  else
    kernel = reinterpret_cast<const void *>(&decode_split_kernel<QT, CT, D, G, NW>);
  // A bin per compute unit (at most one per possible item) and as many
  // workgroups per bin as fit on a compute unit at once (so that the dealt
  // workgroups are those resident at launch); a workgroup per possible item.
  static std::atomic<int> known{0};  // a property of the kernel: computed once
  int per_cu = known.load(std::memory_order_relaxed);
  if (per_cu == 0) {
    per_cu = resident_per_cu(kernel, NW * kWave);
    known.store(per_cu, std::memory_order_relaxed);
  }
  const int64_t nb = std::min<int64_t>({compute_units(stream), kMaxBins, max_items});
  const int64_t w = std::max<int64_t>(1, std::min<int64_t>(per_cu, max_items / nb));
  p.num_bins = (int32_t)nb;
  p.bin_wgs = (int32_t)w;
  p.fd_bins = FastDiv::make((uint32_t)nb);
  p.fd_entry = FastDiv::make((uint32_t)(p.query_start != nullptr ? p.num_kv_heads
                                                                  : p.num_kv_heads * p.head_groups));
  if (trace_level() > 0)
    trace("split kernel: %s engine, q %s, cache %s, D %d, %d rows per row group; %lld "
          "workgroups of %d waves (one per possible item), %lld bins x %lld dealt, %d resident "
          "per CU",
          MfmaEligible<CT, D>::value && QT == PA_BF16 ? "MFMA" : "VALU", dtype_name(QT),
          dtype_name(CT), D, G, (long long)max_items, NW, (long long)nb, (long long)w, per_cu);
  if constexpr (kMfmaBound)
    hipLaunchKernelGGL((decode_split_kernel_mfma<QT, CT, D, G, NW>), dim3((unsigned)max_items),
                       dim3(NW * kWave), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<QT, CT, D, G, NW>), dim3((unsigned)max_items),
                       dim3(NW * kWave), 0, stream, p);
  return hipGetLastError();
}

// Dispatch on (head_dim, rows per KV head) for one (q dtype, cache dtype)
// pair. A KV head has Q*g query rows (query tokens x the heads of its group).
// The MFMA engine takes up to 16 rows per row group, the VALU engine up to 8;
// with a uniform query count, more rows are split into sets of up to four
// row groups handled by separate workgroups. With packed queries the row
// group size follows the largest possible count, min(total, PA_MAX_QUERY_TOKENS).
// max_entries bounds the plan's list (its capacity).
inline int pow2_at_least(int x) {
  int r = 1;
  while (r < x) r <<= 1;
  return r;
}

template <int QT, int CT>
hipError_t dispatch_decode(DecodeParams p, int64_t max_entries, hipStream_t stream) {
  const bool packed = p.query_start != nullptr;
  const int qmax = packed ? min(p.num_query_tokens, PA_MAX_QUERY_TOKENS) : p.num_query_tokens;
  const int rows = max(1, qmax * p.group);
  auto by_rows = [&](auto dtag) -> hipError_t {
    constexpr int D = decltype(dtag)::value;
    constexpr int kMaxRows = (QT == PA_BF16 && MfmaEligible<CT, D>::value) ? 16 : 8;
    const int G = min(kMaxRows, pow2_at_least(rows));
    const int row_groups = (rows + G - 1) / G;
    p.rw = row_groups >= 4 ? 4 : row_groups >= 2 ? 2 : 1;
    p.head_groups = packed ? 1 : (row_groups + p.rw - 1) / p.rw;
    const int64_t items = max_entries * p.num_kv_heads * p.head_groups;
    switch (G) {
      case 1: return launch_decode<QT, CT, D, 1>(p, items, stream);
      case 2: return launch_decode<QT, CT, D, 2>(p, items, stream);
      case 4: return launch_decode<QT, CT, D, 4>(p, items, stream);
      default: break;
    }
    if (G == 8 && kMaxRows == 16) return launch_decode<QT, CT, D, 8>(p, items, stream);
    return launch_decode<QT, CT, D, kMaxRows>(p, items, stream);
  };
  if (p.head_dim == 64) return by_rows(std::integral_constant<int, 64>{});
  return by_rows(std::integral_constant<int, 128>{});
}

}  // namespace pa
