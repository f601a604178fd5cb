// HBM read probe: streams a buffer once with 16-byte loads, as a measured
// ceiling for read-dominated kernels on this device.
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4 *__restrict__ src,
                                                         int64_t n16, uint32_t *__restrict__ sink) {
  constexpr int U = 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  // One word per thread keeps the loads live; the sink holds gridDim*blockDim words.
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream, (const u32x4 *)src,
                     (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace pa
