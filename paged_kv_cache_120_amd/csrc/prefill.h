// Internal launch interface of the chunked-prefill kernel (not part of the
// C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct PrefillArgs {
  _Float16* out;             // [Q, H, D]
  const _Float16* query;     // [Q, H, D]
  const char* key_cache;     // [nb, B, H_kv, D] fp16
  const char* value_cache;
  const int* block_tables;   // [S, M]
  const int* context_lens;   // [S]
  const int* cu_seqlens_q;   // [S + 1]
  int num_q_tokens;
  int max_blocks_per_seq;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  float scale;
};

// query rows x heads of one workgroup (grid.y tiles them per sequence)
constexpr int kPrefillRows = 128;

// grid: (num_kv_heads, ceil(max_q_per_seq * group / kPrefillRows), num_seqs)
hipError_t launch_prefill(const PrefillArgs& a, int head_size, int block_size,
                          int group, dim3 grid, hipStream_t stream);

}  // namespace pa
