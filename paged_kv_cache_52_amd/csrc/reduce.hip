// Reduce kernel of split-K decode [EchoLLMServing notes, section 2,
// FlashDecoding]: merges the per-split (m, l, acc) of every (sequence, query
// head) into the attention output.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

// One wavefront per (query head, sequence). Lanes first scan the split maxima
// in parallel, then walk the splits in order, each lane owning head_dim/64
// output dims.
template <int OT, int D>
__global__ __launch_bounds__(kWave) void reduce_kernel(const ReduceParams p) {
  constexpr int DPL = D / kWave;  // dims per lane
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
  for (int j = 0; j < ns; ++j) {
    const float lj = p.part_l[row0 + j];
    if (!(lj > 0.f)) continue;  // empty split: its acc is never read
    const float w = __expf(p.part_m[row0 + j] - M);
    den = fmaf(w, lj, den);
    const float *a = p.part_acc + (row0 + j) * D;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[k] = fmaf(w, a[lane + k * kWave], acc[k]);
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
