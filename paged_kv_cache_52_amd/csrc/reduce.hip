// Reduce kernel of split-K decode [EchoLLMServing notes, section 2,
// FlashDecoding]: merges the per-split (m, l, acc) of every (sequence, query
// head) into the attention output.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kReduceWaves = 4;       // waves per workgroup
constexpr int kReduceManySplits = 32;  // from this many splits, 4 waves share one head
constexpr int kReduceU = 4;            // splits whose acc rows are loaded together
constexpr int kReduceRowsForFour = 16384;  // from this many rows (and at most kReduceU
                                           // splits), each wave reduces four
constexpr int kReduceManyU = 16;  // many splits: acc rows loaded together per wave

__device__ __forceinline__ float lane_value(float x, int j) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), j));
}

template <int OT>
__device__ __forceinline__ void store_out(const ReduceParams &p, int64_t idx, float o) {
  if constexpr (OT == PA_BF16) {
    ((uint16_t *)p.out)[idx] = (uint16_t)f32_to_bf16_rne(o);
  } else {
    ((float *)p.out)[idx] = o;
  }
}

// Few splits (fewer than kReduceManySplits, so lane j holds split j): each
// wave reduces R consecutive rows (query token, query head) on its own. All
// loads that do not depend on a row's sequence go first: lane j loads every
// row's (m_j, l_j), and the acc rows of splits 0 .. U-1; with packed queries
// the R rows' sequences are then found together by a 16-ary search (lanes
// 16r .. 16r+15 for row r; ceil(log16(num_seqs)) rounds of one load per lane),
// and the rows' split counts follow. Per row, M = the largest m_j of its
// non-empty splits, w_j = exp(m_j - M) (0 for an empty or absent split, so
// the contents of its acc never matter), out = sum_j w_j acc_j / sum_j w_j
// l_j, each lane owning head_dim / 64 output dims. Rows are [num_seqs][Q][Hq]
// (grid y = sequence) or, with packed queries, [N][Hq] (grid y = 1).
template <int OT, int D, int R>
__global__ __launch_bounds__(kReduceWaves *kWave) void reduce_rows_kernel(const ReduceParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  constexpr int U = kReduceU;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int rows = p.num_query_tokens * p.num_q_heads;
  const int hq0 = (blockIdx.x * kReduceWaves + wave) * R;
  if (hq0 >= rows) return;
  const int S = p.max_splits;
  int64_t row0[R];
  float m0[R], l0[R], r0[R][U][DPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    row0[r] = ((int64_t)blockIdx.y * rows + min(hq0 + r, rows - 1)) * S;
    m0[r] = lane < S ? p.part_m[row0[r] + lane] : -INFINITY;
    l0[r] = lane < S ? p.part_l[row0[r] + lane] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        r0[r][u][k] = u < S ? p.part_acc[(row0[r] + u) * D + lane + k * kWave] : 0.f;
  }
  int seq[R];
#pragma unroll
  for (int r = 0; r < R; ++r) seq[r] = blockIdx.y;
  if (p.query_start != nullptr) {
    static_assert(R * 16 <= kWave, "16 lanes per row");
    const int grp = min(lane >> 4, R - 1), sub = lane & 15;
    const int t = min(hq0 + grp, rows - 1) / p.num_q_heads;
    int lo = 0, hi = p.num_seqs;  // the last s with qs[s] <= t lies in [lo, hi)
    while (__any(hi - lo > 1)) {
      const int step = (hi - lo + 15) / 16;
      const int idx = lo + sub * step;
      const unsigned long long le = __ballot(idx < hi && p.query_start[idx] <= t);
      const unsigned bits = (unsigned)(le >> (16 * (lane >> 4))) & 0xffffu;
      const int j = bits ? 31 - __clz(bits) : 0;
      lo += j * step;
      hi = min(hi, lo + step);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) seq[r] = __builtin_amdgcn_readlane(lo, 16 * r);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int Q = p.query_start ? query_span(p.query_start, seq[r], 0, p.num_query_tokens).count
                                : p.num_query_tokens;
    const int L = min(max(0, p.context_lens[seq[r]]), p.len_bound);
    const int ns = Q > 0 ? min(splits_of(L, Q, p.window, p.split_tokens), S) : 0;
    const bool live = lane < ns && l0[r] > 0.f;
    const float M = group_max<kWave>(live ? m0[r] : -INFINITY);
    const float w = live ? __expf(m0[r] - M) : 0.f;
    const float den = group_sum<kWave>(live ? w * l0[r] : 0.f);
    float acc[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < ns) {
        const float wu = lane_value(w, u);
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wu, wu != 0.f ? r0[r][u][k] : 0.f, acc[k]);
      }
    }
    const float *arow = p.part_acc + row0[r] * D + lane;
    for (int i = U; i < ns; i += U) {
      float v[U][DPL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k)
          v[u][k] = i + u < ns ? arow[(int64_t)(i + u) * D + k * kWave] : 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = i + u < ns ? lane_value(w, i + u) : 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wu, wu != 0.f ? v[u][k] : 0.f, acc[k]);
      }
    }
    if (hq0 + r < rows) {
      const int64_t orow = ((int64_t)blockIdx.y * rows + hq0 + r) * D;
#pragma unroll
      for (int k = 0; k < DPL; ++k)
        store_out<OT>(p, orow + lane + k * kWave, den > 0.f ? acc[k] / den : 0.f);
    }
  }
}

// Many splits: the kReduceWaves waves of a workgroup share one row. Each wave
// finds the maximum M of the split maxima (lane-parallel), then sums its
// contiguous range of splits: lane j of a 64-split chunk turns split j's
// (m_j, l_j) into w_j = exp(m_j - M) (0 for an empty split), and the chunk's
// acc rows are added with those weights, 16 rows loaded at a time. The
// waves' sums meet in LDS. Rows as in reduce_rows_kernel; with packed queries
// the row's sequence is found by a 64-ary search.
template <int OT, int D>
__global__ __launch_bounds__(kReduceWaves *kWave) void reduce_kernel(const ReduceParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  constexpr int WPH = kReduceWaves;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int part = wave;
  const bool packed = p.query_start != nullptr;
  const int rows = p.num_query_tokens * p.num_q_heads;
  const int hq = blockIdx.x;  // grid x = rows
  const int64_t row0 = ((int64_t)blockIdx.y * rows + hq) * p.max_splits;
  int s = blockIdx.y, Q = p.num_query_tokens;
  if (packed) {
    s = seq_of_token_wave(p.query_start, p.num_seqs, hq / p.num_q_heads);
    Q = query_span(p.query_start, s, 0, p.num_query_tokens).count;
  }
  const int L = min(max(0, p.context_lens[s]), p.len_bound);
  const int ns = Q > 0 ? min(splits_of(L, Q, p.window, p.split_tokens), p.max_splits) : 0;

  float M = -INFINITY;
  for (int j = lane; j < ns; j += kWave) {
    if (p.part_l[row0 + j] > 0.f) M = fmaxf(M, p.part_m[row0 + j]);
  }
  M = group_max<kWave>(M);

  const int per = (ns + WPH - 1) / WPH;
  const int j0 = min(ns, part * per), j1 = min(ns, j0 + per);
  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float den = 0.f;
  for (int base = j0; base < j1; base += kWave) {
    const int j = base + lane;
    float w = 0.f, lj = 0.f;
    if (j < j1) {
      lj = p.part_l[row0 + j];
      w = lj > 0.f ? __expf(p.part_m[row0 + j] - M) : 0.f;
    }
    den += group_sum<kWave>(w * lj);
    const int cnt = min(kWave, j1 - base);
    const float *arow = p.part_acc + (row0 + base) * D + lane;
    // kReduceManyU acc rows requested at a time (the last group masked).
    for (int i = 0; i < cnt; i += kReduceManyU) {
      float r[kReduceManyU][DPL];
#pragma unroll
      for (int u = 0; u < kReduceManyU; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k) r[u][k] = i + u < cnt ? arow[(i + u) * D + k * kWave] : 0.f;
#pragma unroll
      for (int u = 0; u < kReduceManyU; ++u) {
        const float wu = i + u < cnt ? lane_value(w, (i + u) & (kWave - 1)) : 0.f;
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wu, wu != 0.f ? r[u][k] : 0.f, acc[k]);
      }
    }
  }

  __shared__ float sm_acc[kReduceWaves][D];
  __shared__ float sm_den[kReduceWaves];
#pragma unroll
  for (int k = 0; k < DPL; ++k) sm_acc[wave][lane + k * kWave] = acc[k];
  if (lane == 0) sm_den[wave] = den;
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kReduceWaves * kWave) {
    float a = 0.f, dn = 0.f;
#pragma unroll
    for (int w = 0; w < WPH; ++w) {
      a += sm_acc[w][d];
      dn += sm_den[w];
    }
    store_out<OT>(p, ((int64_t)blockIdx.y * rows + hq) * D + d, dn > 0.f ? a / dn : 0.f);
  }
}

namespace {

template <int OT, int D>
void launch_reduce_t(const ReduceParams &p, hipStream_t stream) {
  const dim3 block(kReduceWaves * kWave);
  const int rows = p.num_query_tokens * p.num_q_heads;
  const int grid_y = p.query_start ? 1 : p.num_seqs;
  if (p.max_splits >= kReduceManySplits) {
    hipLaunchKernelGGL((reduce_kernel<OT, D>), dim3(rows, grid_y), block, 0, stream, p);
  } else if ((int64_t)rows * grid_y >= kReduceRowsForFour && p.max_splits <= kReduceU) {
    // Many rows whose splits are all loaded up front: four per wave, fewer
    // and fuller workgroups (with more splits the rows' remaining loads would
    // run one row after another).
    const dim3 grid((rows + 4 * kReduceWaves - 1) / (4 * kReduceWaves), grid_y);
    hipLaunchKernelGGL((reduce_rows_kernel<OT, D, 4>), grid, block, 0, stream, p);
  } else {
    const dim3 grid((rows + kReduceWaves - 1) / kReduceWaves, grid_y);
    hipLaunchKernelGGL((reduce_rows_kernel<OT, D, 1>), grid, block, 0, stream, p);
  }
}

}  // namespace

hipError_t launch_reduce(const ReduceParams &p, hipStream_t stream) {
  if (p.out_dtype == PA_BF16) {
    if (p.head_dim == 64) launch_reduce_t<PA_BF16, 64>(p, stream);
    else launch_reduce_t<PA_BF16, 128>(p, stream);
  } else {
    if (p.head_dim == 64) launch_reduce_t<PA_F32, 64>(p, stream);
    else launch_reduce_t<PA_F32, 128>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
