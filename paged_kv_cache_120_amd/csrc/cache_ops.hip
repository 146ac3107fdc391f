// Write side of the paged KV cache for gfx950: slot mapping, the per-token
// cache write, copy-on-write block copies and block swaps between pools.
//
// vLLM book ch.4 "PagedAttention：虚拟内存的启示" §4.4.3 (slot_mapping) and
// §4.3.2 / §4.5 (1) (reshape_and_cache: write each new token's K/V rows to
// its slot); "PagedAttention：KV Cache的虚拟内存" copy-on-write paragraph and
// "PagedAttention原理（下）" §4.3 (copy the shared block, then repoint) and
// §4.4 (move the blocks of a paused request out to CPU memory and back);
// ch.4 §4.8 (a lower-precision KV cache: the fp8 cache write).
//
// All three move whole 16-byte chunks; consecutive lanes touch consecutive
// chunks of a token row (cache write) or of a block (copy), so every wave
// issues fully coalesced 1 KiB loads and stores.
#include "common.h"
#include "decode.h"

namespace pa {

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int* __restrict__ out, const int* __restrict__ bt, int M, int rows,
    const int* __restrict__ seq, const int* __restrict__ pos, int n, int B) {
  for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) {
    const int rr = seq[j];
    const int pp = pos[j];
    int s = -1;
    if (rr >= 0 && rr < rows && pp >= 0 && pp < M * B) {
      const int blk = bt[(size_t)rr * M + pp / B];
      const long long v = (long long)blk * B + pp % B;
      if (blk >= 0 && v <= 0x7fffffffLL) s = (int)v;
    }
    out[j] = s;
  }
}

// grid.y strides over tokens, x/threads over the 16-byte chunks of a row
__global__ __launch_bounds__(256) void cache_write_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value,
    u32x4* __restrict__ kc, u32x4* __restrict__ vc,
    const int* __restrict__ slots, int n, long long num_slots, int cpr) {
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int s = slots[j];
    if (s < 0 || (long long)s >= num_slots) continue;
    const size_t src = (size_t)j * cpr;
    const size_t dst = (size_t)s * cpr;
    for (int cc = blockIdx.x * 256 + threadIdx.x; cc < cpr; cc += gridDim.x * 256) {
      kc[dst + cc] = key[src + cc];
      vc[dst + cc] = value[src + cc];
    }
  }
}

// As cache_write_kernel, into an fp8 pool: each lane turns one 16-byte
// chunk of 8 fp16 values into 8 one-byte codes.
__global__ __launch_bounds__(256) void cache_write_fp8_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value,
    u32x2* __restrict__ kc, u32x2* __restrict__ vc,
    const int* __restrict__ slots, int n, long long num_slots, int cpr,
    float inv_k, float inv_v) {
  for (int j = blockIdx.y; j < n; j += gridDim.y) {
    const int s = slots[j];
    if (s < 0 || (long long)s >= num_slots) continue;
    const size_t src = (size_t)j * cpr;
    const size_t dst = (size_t)s * cpr;
    for (int cc = blockIdx.x * 256 + threadIdx.x; cc < cpr; cc += gridDim.x * 256) {
      kc[dst + cc] = f16x8_to_fp8x8(key[src + cc], inv_k);
      vc[dst + cc] = f16x8_to_fp8x8(value[src + cc], inv_v);
    }
  }
}

__global__ __launch_bounds__(256) void copy_blocks_kernel(
    u32x4* __restrict__ kc, u32x4* __restrict__ vc,
    const int* __restrict__ src, const int* __restrict__ dst, int pairs,
    int nb, long long cpb) {
  for (int k = blockIdx.y; k < pairs; k += gridDim.y) {
    const int a = src[k];
    const int b = dst[k];
    if ((unsigned)a >= (unsigned)nb || (unsigned)b >= (unsigned)nb) continue;
    const size_t sa = (size_t)a * cpb;
    const size_t sb = (size_t)b * cpb;
    for (long long cc = (long long)blockIdx.x * 256 + threadIdx.x; cc < cpb;
         cc += (long long)gridDim.x * 256) {
      kc[sb + cc] = kc[sa + cc];
      vc[sb + cc] = vc[sa + cc];
    }
  }
}

// Block moves between two pools (device memory or pinned host memory the
// device maps): block src[k] of (sk, sv) to block dst[k] of (dk, dv).  Each
// workgroup row streams one pair; with host memory on either side the moves
// go over the host link, 1 KiB per wave instruction.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const u32x4* __restrict__ sk, const u32x4* __restrict__ sv, int snb,
    u32x4* __restrict__ dk, u32x4* __restrict__ dv, int dnb,
    const int* __restrict__ src, const int* __restrict__ dst, int pairs,
    long long cpb) {
  for (int k = blockIdx.y; k < pairs; k += gridDim.y) {
    const int a = src[k];
    const int b = dst[k];
    if ((unsigned)a >= (unsigned)snb || (unsigned)b >= (unsigned)dnb) continue;
    const size_t sa = (size_t)a * cpb;
    const size_t sb = (size_t)b * cpb;
    for (long long cc = (long long)blockIdx.x * 256 + threadIdx.x; cc < cpb;
         cc += (long long)gridDim.x * 256) {
      dk[sb + cc] = sk[sa + cc];
      dv[sb + cc] = sv[sa + cc];
    }
  }
}

static int clamp_grid(long long want, int cap) {
  if (want < 1) return 1;
  return want > cap ? cap : (int)want;
}

hipError_t launch_slot_mapping(int* out, const int* bt, int M, int rows,
                               const int* seq, const int* pos, int n, int B,
                               hipStream_t stream) {
  const int grid = clamp_grid((n + 255) / 256, 65535);
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(grid), dim3(256), 0, stream,
                     out, bt, M, rows, seq, pos, n, B);
  return hipGetLastError();
}

hipError_t launch_cache_write(const void* key, const void* value, void* kc,
                              void* vc, const int* slots, int n,
                              int64_t num_slots, int cpr, hipStream_t stream) {
  dim3 grid(clamp_grid((cpr + 255) / 256, 64), clamp_grid(n, 65535));
  hipLaunchKernelGGL(cache_write_kernel, grid, dim3(256), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x4*)kc,
                     (u32x4*)vc, slots, n, (long long)num_slots, cpr);
  return hipGetLastError();
}

hipError_t launch_cache_write_fp8(const void* key, const void* value, void* kc,
                                  void* vc, const int* slots, int n,
                                  int64_t num_slots, int cpr, float inv_k,
                                  float inv_v, hipStream_t stream) {
  dim3 grid(clamp_grid((cpr + 255) / 256, 64), clamp_grid(n, 65535));
  hipLaunchKernelGGL(cache_write_fp8_kernel, grid, dim3(256), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x2*)kc,
                     (u32x2*)vc, slots, n, (long long)num_slots, cpr, inv_k,
                     inv_v);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* kc, void* vc, const int* src,
                              const int* dst, int pairs, int nb,
                              int64_t cpb, hipStream_t stream) {
  dim3 grid(clamp_grid((cpb + 255) / 256, 64), clamp_grid(pairs, 65535));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream,
                     (u32x4*)kc, (u32x4*)vc, src, dst, pairs, nb,
                     (long long)cpb);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const void* sk, const void* sv, int snb, void* dk,
                              void* dv, int dnb, const int* src, const int* dst,
                              int pairs, int64_t cpb, hipStream_t stream) {
  dim3 grid(clamp_grid((cpb + 255) / 256, 64), clamp_grid(pairs, 65535));
  hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(256), 0, stream,
                     (const u32x4*)sk, (const u32x4*)sv, snb, (u32x4*)dk,
                     (u32x4*)dv, dnb, src, dst, pairs, (long long)cpb);
  return hipGetLastError();
}

}  // namespace pa
