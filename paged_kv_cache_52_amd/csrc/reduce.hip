// Reduce kernel of split-K decode [EchoLLMServing notes, section 2,
// FlashDecoding]: merges the per-split (m, l, acc) of every (sequence, query
// head) into the attention output.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

constexpr int kReduceWaves = 4;       // waves per workgroup
constexpr int kReduceManySplits = 32;  // from this many splits, 4 waves share one head

// Every workgroup has kReduceWaves waves. WPH waves work on one row (query
// token, query head): WPH = 1 gives four rows per workgroup (few splits per head),
// WPH = 4 one head whose splits the waves divide (long contexts). Each wave
// finds the maximum M of the split maxima (lane-parallel), then sums a
// contiguous range of splits: lane j of a 64-split chunk turns split j's
// (m_j, l_j) into w_j = exp(m_j - M) (0 for an empty split, so the contents of
// its acc never matter), and the chunk's acc rows are added with those weights,
// each lane owning head_dim / 64 output dims, four rows loaded at a time. With
// WPH > 1 the waves' sums meet in LDS. Rows are [num_seqs][Q][Hq] (grid y =
// sequence) or, with packed queries, [N][Hq] (grid y = 1; a row's sequence is
// found from the query offsets).
template <int OT, int D, int WPH>
__global__ __launch_bounds__(kReduceWaves *kWave) void reduce_kernel(const ReduceParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  constexpr int U = 4;            // splits whose rows are loaded together
  constexpr int HPW = kReduceWaves / WPH;  // heads per workgroup
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int part = wave % WPH;
  const bool packed = p.query_start != nullptr;
  // (query token, head) rows per grid row: per sequence, or all packed rows.
  const int rows = p.num_query_tokens * p.num_q_heads;
  const int hq = blockIdx.x * HPW + wave / WPH;
  if (WPH == 1 && hq >= rows) return;  // no barrier below in that case
  int s = blockIdx.y, Q = p.num_query_tokens;
  if (packed) {
    s = seq_of_token(p.query_start, p.num_seqs, min(hq, rows - 1) / p.num_q_heads);
    Q = query_span(p.query_start, s, 0, p.num_query_tokens).count;
  }
  const int L = max(0, p.context_lens[s]);
  const int ns = Q > 0 ? min(splits_of(L, Q, p.window, p.split_tokens), p.max_splits) : 0;
  const int64_t row0 = ((int64_t)blockIdx.y * rows + hq) * p.max_splits;

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
    const float *rows = p.part_acc + (row0 + base) * D + lane;
    int i = 0;
    for (; i + U <= cnt; i += U) {
      float r[U][DPL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < DPL; ++k) r[u][k] = rows[(i + u) * D + k * kWave];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wu = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i + u));
#pragma unroll
        for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wu, wu != 0.f ? r[u][k] : 0.f, acc[k]);
      }
    }
    for (; i < cnt; ++i) {
      const float wi =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i));
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[k] = fmaf(wi, wi != 0.f ? rows[i * D + k * kWave] : 0.f,
                                                  acc[k]);
    }
  }

  auto store = [&](int64_t idx, float o) {
    if constexpr (OT == PA_BF16) {
      ((uint16_t *)p.out)[idx] = (uint16_t)f32_to_bf16_rne(o);
    } else {
      ((float *)p.out)[idx] = o;
    }
  };
  if constexpr (WPH == 1) {
    const int64_t orow = ((int64_t)blockIdx.y * rows + hq) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) store(orow + lane + k * kWave, den > 0.f ? acc[k] / den : 0.f);
  } else {
    __shared__ float sm_acc[kReduceWaves][D];
    __shared__ float sm_den[kReduceWaves];
#pragma unroll
    for (int k = 0; k < DPL; ++k) sm_acc[wave][lane + k * kWave] = acc[k];
    if (lane == 0) sm_den[wave] = den;
    __syncthreads();
    for (int idx = threadIdx.x; idx < HPW * D; idx += kReduceWaves * kWave) {
      const int h = idx / D, d = idx % D;
      const int hh = blockIdx.x * HPW + h;
      if (hh >= rows) continue;
      float a = 0.f, dn = 0.f;
#pragma unroll
      for (int w = 0; w < WPH; ++w) {
        a += sm_acc[h * WPH + w][d];
        dn += sm_den[h * WPH + w];
      }
      store(((int64_t)blockIdx.y * rows + hh) * D + d, dn > 0.f ? a / dn : 0.f);
    }
  }
}

namespace {

template <int OT, int D>
void launch_reduce_t(const ReduceParams &p, hipStream_t stream) {
  const dim3 block(kReduceWaves * kWave);
  const int rows = p.num_query_tokens * p.num_q_heads;
  const int grid_y = p.query_start ? 1 : p.num_seqs;
  if (p.max_splits >= kReduceManySplits) {
    hipLaunchKernelGGL((reduce_kernel<OT, D, kReduceWaves>), dim3(rows, grid_y), block, 0,
                       stream, p);
  } else {
    const dim3 grid((rows + kReduceWaves - 1) / kReduceWaves, grid_y);
    hipLaunchKernelGGL((reduce_kernel<OT, D, 1>), grid, block, 0, stream, p);
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
