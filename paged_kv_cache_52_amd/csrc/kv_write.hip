// KV write ("reshape and cache") kernels [AMD ATOM article, section 5.1;
// LLM Primer ch. 8, 8.1]: each new token's K and V rows go to the physical slot
// its slot_mapping entry names; an INT8 pool quantises per (token, KV head)
// with one fp32 scale [EchoLLMServing notes, section 3].
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

// Exact copy: one thread moves one 16-byte chunk of a K row and of a V row.
__global__ __launch_bounds__(256) void kv_copy_kernel(const WriteParams p, int row_bytes) {
  const int cpr = row_bytes / 16;  // chunks per (token, head) row
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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
__global__ __launch_bounds__(256) void kv_quant_kernel(const WriteParams p) {
  constexpr int LPG = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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

hipError_t launch_kv_write(const WriteParams &p, hipStream_t stream) {
  const int threads = 256;
  if (p.cache_dtype != PA_I8) {
    const int row_bytes = p.head_dim * (p.cache_dtype == PA_F32 ? 4 : 2);
    const int64_t total = p.num_tokens * p.num_kv_heads * (row_bytes / 16);
    const int64_t blocks = (total + threads - 1) / threads;
    hipLaunchKernelGGL(kv_copy_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, p,
                       row_bytes);
    return hipGetLastError();
  }
  const int64_t total = p.num_tokens * p.num_kv_heads * (p.head_dim / 8);
  const dim3 grid((unsigned)((total + threads - 1) / threads));
  if (p.in_dtype == PA_BF16) {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((kv_quant_kernel<PA_BF16, 64>), grid, dim3(threads), 0, stream, p);
    else
      hipLaunchKernelGGL((kv_quant_kernel<PA_BF16, 128>), grid, dim3(threads), 0, stream, p);
  } else {
    if (p.head_dim == 64)
      hipLaunchKernelGGL((kv_quant_kernel<PA_F32, 64>), grid, dim3(threads), 0, stream, p);
    else
      hipLaunchKernelGGL((kv_quant_kernel<PA_F32, 128>), grid, dim3(threads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace pa
