// KV write ("reshape and cache") kernels [AMD ATOM article, section 5.1;
// LLM Primer ch. 8, 8.1]: each new token's K and V rows go to the physical slot
// its slot_mapping entry names; an INT8 pool quantises per (token, KV head)
// with one fp32 scale [EchoLLMServing notes, section 3], and an FP8 pool
// (OCP E4M3, the ATOM article's FP8 KV cache) likewise.
#include <type_traits>

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
  // The source chunk is read with the slot, not after it (one round trip).
  const int64_t src = row * row_bytes + chunk * 16;
  const u32x4 kx = *(const u32x4 *)((const char *)p.k + src);
  const u32x4 vx = *(const u32x4 *)((const char *)p.v + src);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_blocks * kBlock) return;
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t dst = ((b * p.num_kv_heads + h) * kBlock + o) * row_bytes + chunk * 16;
  *(u32x4 *)((char *)p.k_cache + dst) = kx;
  *(u32x4 *)((char *)p.v_cache + dst) = vx;
}

// OCP E4M3 code of x: the nearest value (ties to the even mantissa) among
// +-m * 2^-9 (subnormals, m < 8) and +-(8 + m) * 2^(e - 10) (e = 1 .. 15, not
// e = 15 with m = 7, which is NaN); finite values beyond 448 saturate to +-448.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a == a)) return 0x7Fu;
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | (uint32_t)rintf(a * 512.0f);  // m * 2^-9; m = 8 is 2^-6
  int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;         // a = 1.f * 2^e, e in [-6, 8]
  int q = (int)rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));  // 8 .. 16 eighths
  if (q == 16) {
    q = 8;
    e += 1;
  }
  return sign | (uint32_t)(((e + 7) << 3) | (q - 8));
}

// Lane `part`'s 8 values of source row src_row, widened to fp32.
template <int IT, int D>
__device__ __forceinline__ void load_row_part(const void *src, int64_t src_row, int part,
                                              float (&x)[8]) {
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
}

// INT8 / FP8 quantiser: a group of D/8 lanes owns one (token, head) row, 8
// values per lane. absmax is combined across the group with DPP; the scale is
// absmax / 127 (INT8) or absmax / 448 (FP8), the division by it is IEEE fp32
// (correctly rounded), and both roundings are to nearest, ties to even.
template <int CT, int D>
__device__ __forceinline__ void quantise_row(const float (&x)[8], int part, uint8_t *dst,
                                             float *scale_dst, bool write_scale) {
  constexpr int LPG = D / 8;
  float a = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) a = fmaxf(a, fabsf(x[k]));
  a = group_max<LPG>(a);
  const float sc = a / (CT == PA_FP8 ? 448.0f : 127.0f);
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t code = 0u;
    if (a != 0.f) {
      if constexpr (CT == PA_FP8) {
        code = e4m3_code(x[k] / sc);
      } else {
        const float r = fminf(fmaxf(rintf(x[k] / sc), -127.f), 127.f);
        code = (uint32_t)((int32_t)r) & 0xffu;
      }
    }
    packed[k / 4] |= code << (8 * (k % 4));
  }
  u32x2 out;
  out[0] = packed[0];
  out[1] = packed[1];
  *(u32x2 *)(dst + part * 8) = out;
  if (write_scale) *scale_dst = sc;
}

template <int CT, int IT, int D>
__device__ __forceinline__ void kv_quant_thread(const WriteParams &p, int64_t gid) {
  constexpr int LPG = D / 8;
  const int64_t total = p.num_tokens * p.num_kv_heads * LPG;
  if (gid >= total) return;  // whole lane groups leave together (total % LPG == 0)
  const int64_t row = gid / LPG;
  const int part = (int)(gid % LPG);
  const int64_t t = row / p.num_kv_heads;
  const int h = (int)(row - t * p.num_kv_heads);
  // The source values are read with the slot, not after it (one round trip).
  float xk[8], xv[8];
  load_row_part<IT, D>(p.k, row, part, xk);
  load_row_part<IT, D>(p.v, row, part, xv);
  const int64_t slot = p.slot_mapping[t];
  if (slot < 0 || slot >= p.num_blocks * kBlock) return;  // same for the whole group
  const int64_t b = slot / kBlock;
  const int o = (int)(slot - b * kBlock);
  const int64_t srow = (b * p.num_kv_heads + h) * kBlock + o;  // scale index
  quantise_row<CT, D>(xk, part, (uint8_t *)p.k_cache + srow * D, p.k_scale + srow, part == 0);
  quantise_row<CT, D>(xv, part, (uint8_t *)p.v_cache + srow * D, p.v_scale + srow, part == 0);
}

// Write variants: 0 copies; 1..4 quantise to INT8 and 5..8 to FP8, each for
// ({bf16, fp32} input) x (head_dim {64, 128}).
template <int VARIANT>
__device__ __forceinline__ void write_variant(const WriteParams &w, int row_bytes, int64_t gid) {
  constexpr int CT = VARIANT >= 5 ? PA_FP8 : PA_I8;
  constexpr int V = VARIANT >= 5 ? VARIANT - 4 : VARIANT;
  constexpr int IT = V <= 2 ? PA_BF16 : PA_F32;
  constexpr int D = (V % 2) ? 64 : 128;
  if constexpr (VARIANT == 0)
    kv_copy_thread(w, row_bytes, gid);
  else
    kv_quant_thread<CT, IT, D>(w, gid);
}

template <int VARIANT>
__global__ __launch_bounds__(kPlanThreads) void kv_write_kernel(const WriteParams p,
                                                                int row_bytes) {
  write_variant<VARIANT>(p, row_bytes, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// KV write and plan of one decode step in one launch (they do not depend on
// each other): the last workgroup plans, the others write.
template <int VARIANT>
__global__ __launch_bounds__(kPlanThreads) void prepare_kernel(const WriteParams w,
                                                               const PlanParams pl,
                                                               int row_bytes) {
  if (blockIdx.x == gridDim.x - 1) {
    plan_workgroup(pl);
    return;
  }
  write_variant<VARIANT>(w, row_bytes, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

namespace {

// Write variant, row bytes (copy) and number of write workgroups.
struct WriteShape {
  int variant, row_bytes;
  int64_t blocks;
};

WriteShape write_shape(const WriteParams &p) {
  if (p.cache_dtype != PA_I8 && p.cache_dtype != PA_FP8) {
    const int row_bytes = p.head_dim * (p.cache_dtype == PA_F32 ? 4 : 2);
    const int64_t total = p.num_tokens * p.num_kv_heads * (row_bytes / 16);
    return {0, row_bytes, (total + kPlanThreads - 1) / kPlanThreads};
  }
  const int64_t total = p.num_tokens * p.num_kv_heads * (p.head_dim / 8);
  const int variant = (p.cache_dtype == PA_FP8 ? 4 : 0) + (p.in_dtype == PA_BF16 ? 1 : 3) +
                      (p.head_dim == 64 ? 0 : 1);
  return {variant, 0, (total + kPlanThreads - 1) / kPlanThreads};
}

}  // namespace

hipError_t launch_kv_write(const WriteParams &p, hipStream_t stream) {
  const WriteShape ws = write_shape(p);
  const dim3 grid((unsigned)ws.blocks), block(kPlanThreads);
  auto go = [&](auto v) {
    hipLaunchKernelGGL(kv_write_kernel<decltype(v)::value>, grid, block, 0, stream, p,
                       ws.row_bytes);
  };
  switch (ws.variant) {
    case 0: go(std::integral_constant<int, 0>{}); break;
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

hipError_t launch_prepare(const WriteParams &w, const PlanParams &pl, hipStream_t stream) {
  const WriteShape ws = write_shape(w);
  const dim3 grid((unsigned)(ws.blocks + 1)), block(kPlanThreads);
  auto go = [&](auto v) {
    hipLaunchKernelGGL(prepare_kernel<decltype(v)::value>, grid, block, 0, stream, w, pl,
                       ws.row_bytes);
  };
  switch (ws.variant) {
    case 0: go(std::integral_constant<int, 0>{}); break;
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 5: go(std::integral_constant<int, 5>{}); break;
    case 6: go(std::integral_constant<int, 6>{}); break;
    case 7: go(std::integral_constant<int, 7>{}); break;
    default: go(std::integral_constant<int, 8>{}); break;
  }
  return hipGetLastError();
}

}  // namespace pa
