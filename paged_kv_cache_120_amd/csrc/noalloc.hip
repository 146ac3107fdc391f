// The fused decode step for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): pa_decode_step with its range counters and partial states in
// a static device array instead of a caller-provided workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "api_internal.h"
#include "pa.h"

namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchPairs = PA_NOALLOC_MAX_PAIRS;
constexpr size_t kScratchCounterBytes = kScratchPairs * 4;
static_assert(kScratchCounterBytes % 256 == 0 && kScratchCounterBytes < kScratchBytes,
              "states start 256-byte aligned after the counters");

// Range counters (the first kScratchCounterBytes, zero between calls) and
// partial states of pa_decode_step_noalloc.  Each device the library runs
// on holds its own copy until the process ends.  In host code this name is
// only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void clear_words(unsigned* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
unsigned char* g_scratch[kMaxDevices];   // device address, per device

// Device address of the current device's scratch.  The first call on a
// device resolves it and clears the counters, waiting on `stream` for the
// clear (so that first call must not be captured into a graph).
pa_status scratch_address(hipStream_t stream, unsigned char** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return PA_ERR_HIP;
    hipLaunchKernelGGL(clear_words, dim3(64), dim3(256), 0, stream,
                       static_cast<unsigned*>(p), kScratchCounterBytes / 4);
    if (hipGetLastError() != hipSuccess || hipStreamSynchronize(stream) != hipSuccess)
      return PA_ERR_HIP;
    g_scratch[dev] = static_cast<unsigned char*>(p);
  }
  *addr = g_scratch[dev];
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_decode_step_noalloc(
    void* out, const void* query, const void* key, const void* value,
    void* key_cache, void* value_cache, int32_t* slot_mapping,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t grid, hipStream_t stream) {
  if (num_seqs > 0 && (!key || !value)) return PA_ERR_NULL;
  constexpr size_t kStateBytes = kScratchBytes - kScratchCounterBytes;
  // every argument, the size limits included, is checked before the device
  // is touched
  pa_status st = pa::balanced_run(
      out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
      context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
      num_blocks, scale, grid, nullptr, kScratchPairs, nullptr, kStateBytes, key,
      value, slot_mapping, stream, 2, 1.f, 1.f, false);
  if (st != PA_OK || num_seqs == 0) return st;
  unsigned char* base = nullptr;
  st = scratch_address(stream, &base);
  if (st != PA_OK) return st;
  return pa::balanced_run(
      out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
      context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
      num_blocks, scale, grid, reinterpret_cast<int*>(base), kScratchPairs,
      reinterpret_cast<float*>(base + kScratchCounterBytes), kStateBytes, key,
      value, slot_mapping, stream, 2, 1.f, 1.f, true);
}
