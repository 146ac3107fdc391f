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
  // split mode: one workgroup per (row tile, key partition) writes each
  // row's (max in natural-log units, sum, unnormalised out) for the
  // partition to [row, head, max_partitions] states (the split-K layout)
  float* ws_max;
  float* ws_sum;
  float* ws_out;
  int partition_size;        // keys, a multiple of 16
  int max_partitions;
  int num_seqs;
  int max_tokens;            // max_blocks_per_seq * block_size (the fold)
};

// query rows x heads of one workgroup (grid.y tiles them per sequence)
constexpr int kPrefillRows = 128;

// grid: (num_kv_heads, ceil(max_q_per_seq * group / kPrefillRows), num_seqs),
// and max_partitions * num_seqs in z (partition-major) for the split mode
hipError_t launch_prefill(const PrefillArgs& a, int head_size, int block_size,
                          int group, dim3 grid, bool split, hipStream_t stream);

// The fold after the split mode: out[row, head] from the partitions that
// hold keys 0 .. the row's position (one wave per row and head).
hipError_t launch_prefill_fold(const PrefillArgs& a, int head_size,
                               hipStream_t stream);

}  // namespace pa
