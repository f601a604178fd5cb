// HBM read probe: streams a buffer once, as a measured ceiling for
// read-dominated kernels on this device. Each wave of a persistent grid reads
// whole 8 KiB chunks (eight 16-byte loads per lane, consecutive lanes on
// consecutive addresses), two chunks in flight; chunks are dealt round-robin
// over the waves. This was the fastest of the read patterns tried on MI355X
// (grid-stride 16-byte loads reach about 15% less).
#include "pa_common.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kChunk = 512;      // 16-byte words per chunk (8 KiB)
constexpr int kProbeWaves = 4;   // waves per workgroup

__device__ __forceinline__ uint32_t xor4(const u32x4 &v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

}  // namespace

__global__ __launch_bounds__(kProbeWaves *kWave) void read_probe_kernel(
    const u32x4 *__restrict__ src, int64_t n16, uint32_t *__restrict__ sink) {
  constexpr int PER_LANE = kChunk / kWave;  // loads per lane per chunk
  const int lane = lane_id();
  const int64_t nwaves = (int64_t)gridDim.x * kProbeWaves;
  int64_t w = (int64_t)blockIdx.x * kProbeWaves + threadIdx.x / kWave;
  const int64_t nchunks = n16 / kChunk;
  uint32_t acc = 0;
  for (; w + nwaves < nchunks; w += 2 * nwaves) {  // chunks w and w + nwaves
    u32x4 a[PER_LANE], b[PER_LANE];
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      a[k] = __builtin_nontemporal_load(src + w * kChunk + k * kWave + lane);
      b[k] = __builtin_nontemporal_load(src + (w + nwaves) * kChunk + k * kWave + lane);
    }
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) acc ^= xor4(a[k]) ^ xor4(b[k]);
  }
  if (w < nchunks) {  // at most one chunk left for this wave
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k)
      acc ^= xor4(__builtin_nontemporal_load(src + w * kChunk + k * kWave + lane));
  }
  // Words past the last whole chunk.
  for (int64_t i = nchunks * kChunk + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    acc ^= xor4(src[i]);
  // One word per thread keeps the loads live; the sink holds gridDim*blockDim words.
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_read_probe(const void *src, size_t bytes, uint32_t *sink, int blocks,
                             hipStream_t stream) {
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeWaves * kWave), 0, stream,
                     (const u32x4 *)src, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace pa
