// Streaming-read probe: the bandwidth a plain read of device memory reaches on
// this chip, measured beside the verify kernels so their fractions can be
// given against it as well as against the nominal HBM peak.  Not part of the
// verify path.
//
// Each wave reads 8 KB per step as eight 16-byte nontemporal loads per lane
// (1 KB contiguous per instruction, all eight in flight), the waves of the
// grid striding over the buffer; an XOR of everything read is written per
// workgroup so no load can be dropped.

#include "common.h"

namespace sv {

constexpr int kProbeThreads = 256;
constexpr int kProbeStep = 8;          // 16-byte loads per lane per step

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const u32x4_t* __restrict__ a,
                                                              long long nchunks,
                                                              uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const long long wave = ((long long)blockIdx.x * kProbeThreads + threadIdx.x) >> 6;
  const long long nwaves = ((long long)gridDim.x * kProbeThreads) >> 6;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (long long c = wave; c < nchunks; c += nwaves) {
    const u32x4_t* p = a + c * (64 * kProbeStep) + lane;
    u32x4_t v[kProbeStep];
#pragma unroll
    for (int u = 0; u < kProbeStep; ++u) v[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
    for (int u = 0; u < kProbeStep; ++u) acc ^= v[u];
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= (uint32_t)__shfl_xor((int)x, off, 64);
  __shared__ uint32_t s_x[kProbeThreads / 64];
  if (lane == 0) s_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kProbeThreads / 64; ++w) t ^= s_x[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace sv

extern "C" int spec_read_probe(const void* buf, size_t bytes, uint32_t* sink, int grid,
                               void* hip_stream) {
  constexpr size_t kChunk = (size_t)64 * sv::kProbeStep * 16;   // 8 KB per wave step
  if (!buf || !sink || grid < 1 || grid > (1 << 20) || bytes == 0 || bytes % kChunk != 0)
    return SV_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(buf) & 15) return SV_ERR_INVALID_ARG;
  hipLaunchKernelGGL(sv::k_read_probe, dim3(grid), dim3(sv::kProbeThreads), 0,
                     static_cast<hipStream_t>(hip_stream),
                     static_cast<const sv::u32x4_t*>(buf), (long long)(bytes / kChunk), sink);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
