// Reduce kernel of split-K decode [EchoLLMServing notes, section 2,
// FlashDecoding]: merges the per-split (m, l, acc) of every (sequence, query
// head) into the attention output.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

// One wavefront per (query head, sequence). Lane j first turns split j's
// (m_j, l_j) into its weight w_j = exp(m_j - M) (0 for an empty split, so the
// contents of its acc never matter), then the splits' acc rows are summed with
// those weights, each lane owning head_dim / 64 output dims. The row loads do
// not depend on each other, so the compiler can keep several in flight.
template <int OT, int D>
__global__ __launch_bounds__(kWave) void reduce_kernel(const ReduceParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
  constexpr int U = 4;            // splits whose rows are loaded together
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int lane = lane_id();
  const int L = max(0, p.context_lens[s]);
  const int ns = min(max(1, (L + p.split_tokens - 1) / p.split_tokens), p.max_splits);
  const int64_t row0 = ((int64_t)s * p.num_q_heads + hq) * p.max_splits;

  float M = -INFINITY;
  for (int j = lane; j < ns; j += kWave) {
    if (p.part_l[row0 + j] > 0.f) M = fmaxf(M, p.part_m[row0 + j]);
  }
  M = group_max<kWave>(M);

  float acc[DPL];
#pragma unroll
  for (int k = 0; k < DPL; ++k) acc[k] = 0.f;
  float den = 0.f;
  for (int base = 0; base < ns; base += kWave) {
    const int j = base + lane;
    float w = 0.f, lj = 0.f;
    if (j < ns) {
      lj = p.part_l[row0 + j];
      w = lj > 0.f ? __expf(p.part_m[row0 + j] - M) : 0.f;
    }
    den += group_sum<kWave>(w * lj);
    const int cnt = min(kWave, ns - base);
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
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t orow = ((int64_t)s * p.num_q_heads + hq) * D;
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const float o = acc[k] * inv;
    if constexpr (OT == PA_BF16) {
      ((uint16_t *)p.out)[orow + lane + k * kWave] = (uint16_t)f32_to_bf16_rne(o);
    } else {
      ((float *)p.out)[orow + lane + k * kWave] = o;
    }
  }
}

hipError_t launch_reduce(const ReduceParams &p, hipStream_t stream) {
  dim3 grid(p.num_q_heads, p.num_seqs);
  if (p.out_dtype == PA_BF16) {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((reduce_kernel<PA_BF16, 64>), grid, dim3(kWave), 0, stream, p);
    else
      hipLaunchKernelGGL((reduce_kernel<PA_BF16, 128>), grid, dim3(kWave), 0, stream, p);
  } else {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((reduce_kernel<PA_F32, 64>), grid, dim3(kWave), 0, stream, p);
    else
      hipLaunchKernelGGL((reduce_kernel<PA_F32, 128>), grid, dim3(kWave), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
