// KV write ("reshape and cache") kernels [AMD ATOM article, section 5.1;
// LLM Primer ch. 8, 8.1]: each new token's K and V rows go to the physical slot
// its slot_mapping entry names; an INT8 pool quantises per (token, KV head)
// with one fp32 scale [EchoLLMServing notes, section 3].
#include "pa_common.h"
#include "pa_internal.h"
#include "plan_device.h"

namespace pa {

// Exact copy: one thread moves one 16-byte chunk of a K row and of a V row.
__device__ __forceinline__ void kv_copy_thread(const WriteParams &p, int row_bytes, int64_t gid) {
  const int cpr = row_bytes / 16;  // chunks per (token, head) row
  const int64_t total = p.num_tokens * p.num_kv_heads * cpr;
  if (gid >= total) return;
  const int64_t row = gid / cpr;
  const int chunk = (int)(gid - row * cpr);
  const int64_t t = row / p.num_kv_heads;
  const int h = (int)(row - t * p.num_kv_heads);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_blocks * kBlock) return;
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t dst = ((b * p.num_kv_heads + h) * kBlock + o) * row_bytes + chunk * 16;
  const int64_t src = row * row_bytes + chunk * 16;
  *(u32x4 *)((char *)p.k_cache + dst) = *(const u32x4 *)((const char *)p.k + src);
  *(u32x4 *)((char *)p.v_cache + dst) = *(const u32x4 *)((const char *)p.v + src);
}

__global__ __launch_bounds__(kPlanThreads) void kv_copy_kernel(const WriteParams p, int row_bytes) {
  kv_copy_thread(p, row_bytes, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// INT8 quantiser: a group of D/8 lanes owns one (token, head) row, 8 values
// per lane. absmax is combined across the group with DPP; the division by the
// scale is IEEE fp32 (correctly rounded) and rintf rounds half to even.
template <int IT, int D>
__device__ __forceinline__ void quantise_row(const void *src, int64_t src_row, int part,
                                             int8_t *dst, float *scale_dst, bool write_scale) {
  constexpr int LPG = D / 8;
  float x[8];
  if constexpr (IT == PA_BF16) {
    const u32x4 w = *(const u32x4 *)((const uint16_t *)src + src_row * D + part * 8);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_lo(w[k]);
      x[2 * k + 1] = bf16_hi(w[k]);
    }
  } else {
    const float *f = (const float *)src + src_row * D + part * 8;
    const u32x4 w0 = *(const u32x4 *)f;
    const u32x4 w1 = *(const u32x4 *)(f + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = __uint_as_float(w0[k]);
      x[4 + k] = __uint_as_float(w1[k]);
    }
  }
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(x[k]));
  a = group_max<LPG>(a);
  const float sc = a / 127.0f;
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float r = 0.f;
    if (a != 0.f) {
      r = rintf(x[k] / sc);
      r = fminf(fmaxf(r, -127.f), 127.f);
    }
    const uint32_t code = (uint32_t)((int32_t)r) & 0xffu;
    packed[k / 4] |= code << (8 * (k % 4));
  }
  u32x2 out;
  out[0] = packed[0];
  out[1] = packed[1];
  *(u32x2 *)(dst + part * 8) = out;
  if (write_scale) *scale_dst = sc;
}

template <int IT, int D>
__device__ __forceinline__ void kv_quant_thread(const WriteParams &p, int64_t gid) {
  constexpr int LPG = D / 8;
  const int64_t total = p.num_tokens * p.num_kv_heads * LPG;
  if (gid >= total) return;  // whole lane groups leave together (total % LPG == 0)
  const int64_t row = gid / LPG;
  const int part = (int)(gid % LPG);
  const int64_t t = row / p.num_kv_heads;
  const int h = (int)(row - t * p.num_kv_heads);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_blocks * kBlock) return;  // same for the whole group
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t srow = (b * p.num_kv_heads + h) * kBlock + o;  // scale index
  quantise_row<IT, D>(p.k, row, part, (int8_t *)p.k_cache + srow * D, p.k_scale + srow, part == 0);
  quantise_row<IT, D>(p.v, row, part, (int8_t *)p.v_cache + srow * D, p.v_scale + srow, part == 0);
}

template <int IT, int D>
__global__ __launch_bounds__(kPlanThreads) void kv_quant_kernel(const WriteParams p) {
  kv_quant_thread<IT, D>(p, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// KV write and plan of one decode step in one launch (they do not depend on
// each other): the last workgroup plans, the others write. Variant 0 copies,
// variants 1..4 quantise ({bf16, fp32} input x head_dim {64, 128}).
template <int VARIANT>
__global__ __launch_bounds__(kPlanThreads) void prepare_kernel(const WriteParams w,
                                                               const PlanParams pl,
                                                               int row_bytes) {
  if (blockIdx.x == gridDim.x - 1) {
    plan_workgroup(pl);
    return;
  }
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if constexpr (VARIANT == 0) kv_copy_thread(w, row_bytes, gid);
  if constexpr (VARIANT == 1) kv_quant_thread<PA_BF16, 64>(w, gid);
  if constexpr (VARIANT == 2) kv_quant_thread<PA_BF16, 128>(w, gid);
  if constexpr (VARIANT == 3) kv_quant_thread<PA_F32, 64>(w, gid);
  if constexpr (VARIANT == 4) kv_quant_thread<PA_F32, 128>(w, gid);
}

namespace {

// Write variant, row bytes (copy) and number of write workgroups.
struct WriteShape {
  int variant, row_bytes;
  int64_t blocks;
};

WriteShape write_shape(const WriteParams &p) {
  if (p.cache_dtype != PA_I8) {
    const int row_bytes = p.head_dim * (p.cache_dtype == PA_F32 ? 4 : 2);
    const int64_t total = p.num_tokens * p.num_kv_heads * (row_bytes / 16);
    return {0, row_bytes, (total + kPlanThreads - 1) / kPlanThreads};
  }
  const int64_t total = p.num_tokens * p.num_kv_heads * (p.head_dim / 8);
  const int variant = (p.in_dtype == PA_BF16 ? 1 : 3) + (p.head_dim == 128 ? 1 : 0);
  return {variant, 0, (total + kPlanThreads - 1) / kPlanThreads};
}

}  // namespace

hipError_t launch_kv_write(const WriteParams &p, hipStream_t stream) {
  const WriteShape ws = write_shape(p);
  const dim3 grid((unsigned)ws.blocks), block(kPlanThreads);
  switch (ws.variant) {
    case 0: hipLaunchKernelGGL(kv_copy_kernel, grid, block, 0, stream, p, ws.row_bytes); break;
    case 1: hipLaunchKernelGGL((kv_quant_kernel<PA_BF16, 64>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((kv_quant_kernel<PA_BF16, 128>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((kv_quant_kernel<PA_F32, 64>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((kv_quant_kernel<PA_F32, 128>), grid, block, 0, stream, p); break;
  }
  return hipGetLastError();
}

hipError_t launch_prepare(const WriteParams &w, const PlanParams &pl, hipStream_t stream) {
  const WriteShape ws = write_shape(w);
  const dim3 grid((unsigned)(ws.blocks + 1)), block(kPlanThreads);
  switch (ws.variant) {
    case 0: hipLaunchKernelGGL(prepare_kernel<0>, grid, block, 0, stream, w, pl, ws.row_bytes); break;
    case 1: hipLaunchKernelGGL(prepare_kernel<1>, grid, block, 0, stream, w, pl, 0); break;
    case 2: hipLaunchKernelGGL(prepare_kernel<2>, grid, block, 0, stream, w, pl, 0); break;
    case 3: hipLaunchKernelGGL(prepare_kernel<3>, grid, block, 0, stream, w, pl, 0); break;
    default: hipLaunchKernelGGL(prepare_kernel<4>, grid, block, 0, stream, w, pl, 0); break;
  }
  return hipGetLastError();
}

}  // namespace pa
