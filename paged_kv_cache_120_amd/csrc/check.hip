// PA_CHECK=1 validation pass: the device-side preconditions of the decode
// and cache-write calls, checked on the device before anything else is
// launched (used only when the PA_CHECK environment variable is 1).
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <mutex>

#include "api_internal.h"
#include "pa.h"

namespace {

// Bits of failed checks of one validation pass (PA_CHECK_* in pa.h).  In
// host code this name is only a stand-in; the device address comes from
// hipGetSymbolAddress.
static __device__ unsigned check_flags;

__device__ __forceinline__ void flag(unsigned* f, unsigned bit) {
  atomicOr(f, bit);
}

// One workgroup per sequence: its context length against the table width,
// and every table entry that a decode reads against the pool.
__global__ __launch_bounds__(256) void check_tables_kernel(
    const int32_t* block_tables, int32_t M, const int32_t* context_lens,
    int32_t nb, int32_t B, unsigned* flags) {
  const int i = blockIdx.x;
  const int64_t n = context_lens[i];
  const int64_t max_tok = (int64_t)M * B;
  if (threadIdx.x == 0 && n > max_tok) flag(flags, PA_CHECK_CONTEXT);
  const int64_t used = ((n < max_tok ? n : max_tok) + B - 1) / B;
  for (int64_t j = threadIdx.x; j < used; j += blockDim.x) {
    const int32_t id = block_tables[(int64_t)i * M + j];
    if (id < 0 || id >= nb) flag(flags, PA_CHECK_TABLE);
  }
}

// Slot of list entry k: explicit (slots[k]) or the slot a fused step writes
// for sequence k (position context_lens[k] - 1); -1 for none.
struct SlotList {
  const int32_t* slots;          // explicit list, or null
  const int32_t* block_tables;   // derived: tables and lengths
  const int32_t* context_lens;
  int32_t M, B, nb;
  __device__ int64_t at(int k) const {
    if (slots) return slots[k];
    const int64_t n = context_lens[k];
    if (n <= 0 || n > (int64_t)M * B) return -1;
    const int32_t id = block_tables[(int64_t)k * M + (n - 1) / B];
    if (id < 0 || id >= nb) return -1;
    return (int64_t)id * B + (n - 1) % B;
  }
};

// Each thread takes one entry: in range, and no later entry equal to it
// (all pairs, in LDS tiles of 1024).
__global__ __launch_bounds__(256) void check_slots_kernel(SlotList L, int32_t n,
                                                          int64_t num_slots,
                                                          unsigned* flags) {
  __shared__ int64_t tile[1024];
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = k < n ? L.at(k) : -1;
  if (s >= num_slots) flag(flags, PA_CHECK_SLOT_RANGE);
  const int first = blockIdx.x * blockDim.x;
  for (int c0 = first; c0 < n; c0 += 1024) {
    __syncthreads();
    for (int j = threadIdx.x; j < 1024 && c0 + j < n; j += blockDim.x)
      tile[j] = L.at(c0 + j);
    __syncthreads();
    if (s >= 0) {
      const int lim = n - c0 < 1024 ? n - c0 : 1024;
      for (int j = 0; j < lim; ++j)
        if (c0 + j > k && tile[j] == s) {
          flag(flags, PA_CHECK_DUPLICATE_SLOT);
          break;
        }
    }
  }
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
unsigned* g_flags[kMaxDevices];
thread_local unsigned g_last;

unsigned* flags_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_flags[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_flags)) != hipSuccess) return nullptr;
    g_flags[dev] = static_cast<unsigned*>(p);
  }
  return g_flags[dev];
}

}  // namespace

namespace pa {

bool check_mode() {
  const char* e = getenv("PA_CHECK");
  return e && e[0] == '1' && e[1] == '\0';
}

pa_status device_check(const int32_t* block_tables, int32_t M,
                       const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_blocks, int32_t block_size, bool derived_slots,
                       const int32_t* slots, int32_t num_slots, hipStream_t stream) {
  unsigned* f = flags_address();
  if (!f) return PA_ERR_HIP;
  static const unsigned zero = 0;
  if (hipMemcpyAsync(f, &zero, sizeof(zero), hipMemcpyHostToDevice, stream) != hipSuccess)
    return PA_ERR_HIP;
  if (block_tables && num_seqs > 0) {
    hipLaunchKernelGGL(check_tables_kernel, dim3(num_seqs), dim3(256), 0, stream,
                       block_tables, M, context_lens, num_blocks, block_size, f);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  SlotList L = {slots, block_tables, context_lens, M, block_size, num_blocks};
  const int32_t n = slots ? num_slots : (derived_slots ? num_seqs : 0);
  if (n > 0) {
    hipLaunchKernelGGL(check_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                       L, n, (int64_t)num_blocks * block_size, f);
    if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
  }
  unsigned got = 0;
  if (hipMemcpyAsync(&got, f, sizeof(got), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return PA_ERR_HIP;
  g_last = got;
  return got ? PA_ERR_CHECK : PA_OK;
}

unsigned last_check() { return g_last; }

}  // namespace pa

extern "C" uint32_t pa_last_check(void) { return pa::last_check(); }
