// Streaming-read probe for gfx950: the HBM read rate a plain, fully
// sequential read of one large buffer reaches on this device.  It is the
// measured ceiling the decode's KV read rate is compared with, beside the
// nominal HBM peak; it is not part of the attention path.
//
// Each lane reads 16-byte chunks with non-temporal loads, eight independent
// loads in flight per iteration; consecutive lanes read consecutive chunks,
// so every wave load covers 1 KiB of contiguous memory.  What a wave read is
// folded (xor) into one word that lane 0 stores, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {
namespace {

typedef unsigned u32x4p __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(
    const u32x4p* __restrict__ src, size_t n16, unsigned* __restrict__ sink) {
  unsigned acc = 0;
  const size_t chunk = (size_t)kProbeThreads * kProbeUnroll;  // per workgroup step
  const size_t step = (size_t)gridDim.x * chunk;
  size_t i = (size_t)blockIdx.x * chunk + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < n16; i += step) {
    u32x4p v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the last partial step: each chunk index checked on its own
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) {
    const size_t j = i + u * kProbeThreads;
    if (j < n16) {
      const u32x4p v = __builtin_nontemporal_load(src + j);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0)
    sink[(size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace
}  // namespace pa

extern "C" pa_status pa_stream_read(const void* buf, size_t bytes,
                                    uint32_t* sink, int32_t grid,
                                    hipStream_t stream) {
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes == 0 || grid <= 0 || grid > 65535) return PA_ERR_SHAPE;
  if (bytes % 16 || (uintptr_t)buf % 16 || (uintptr_t)sink % 4) return PA_ERR_ALIGN;
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(grid), dim3(pa::kProbeThreads), 0,
                     stream, static_cast<const pa::u32x4p*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}
