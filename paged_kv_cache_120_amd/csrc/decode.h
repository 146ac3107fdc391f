// Internal launch interface of the decode kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  _Float16* out;             // [S, H, D]      single-pass mode
  float* ws_max;             // [S, H, Pmax]   split mode
  float* ws_sum;             // [S, H, Pmax]
  float* ws_out;             // [S, H, Pmax, D]
  const _Float16* query;     // [S, H, D]
  const char* key_cache;     // [nb, B, H_kv, D] fp16
  const char* value_cache;
  const int* block_tables;   // [S, M]
  const int* context_lens;   // [S]
  int max_blocks_per_seq;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int partition_size;        // tokens; a multiple of B
  int max_partitions;        // Pmax (split mode)
  int split;
  int num_seqs;              // balanced split
  int* bal_count;            // [S*H_kv] range counters, zero between calls
  // fused step (all null unless the kernel also appends this step's token):
  // the token at position context_len-1 is taken from new_key/new_value
  // ([S, H_kv, D]), stored into its slot, and its slot written to slot_out
  const _Float16* new_key;
  const _Float16* new_value;
  int* slot_out;
  float scale;
  // multi-token queries: query row offsets [S+1] and query tiles per sequence
  const int* cu_seqlens_q;
  int q_tiles;
  int num_q_tokens;
  // fp8 pools: dequantisation scales (value = code * scale)
  float k_scale;
  float v_scale;
  float inv_k_scale;     // fused fp8 append: 1/scale rounded to fp32
  float inv_v_scale;
  // shared-prefix decode: per-sequence first partition left to the
  // partition kernel (earlier ones come from the prefix kernel), and the
  // groups (member lists in CSR form, shared full blocks per group)
  const int* part_start;
  const int* grp_offsets;
  const int* grp_members;
  const int* grp_blocks;
  int num_groups;
  int grp_max_parts;     // shared partitions per group at most (grid.z)
  int grp_max_members;   // members per group the prefix kernel covers
};


struct ReduceArgs {
  _Float16* out;
  const float* ws_max;
  const float* ws_sum;
  const float* ws_out;
  const int* context_lens;
  int num_heads;
  int max_partitions;
  int partition_size;
  int max_tokens;            // M * B
  const int* cu_seqlens_q;   // multi-token reduce: [S+1]
  int num_seqs;
};

hipError_t launch_decode(const DecodeArgs& a, int head_size, int block_size,
                         int group, dim3 grid, hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int head_size, int num_seqs,
                         hipStream_t stream);
// whole_line: the matrix-core body with split_columns() columns per tile
// instead of its 16-column form
hipError_t launch_multi(const DecodeArgs& a, int head_size, int block_size,
                        int group, dim3 grid, bool whole_line,
                        hipStream_t stream);
// multi-token queries on the balanced split (T*g <= 16 rows x heads per
// sequence, one kernel), always the whole-line body: whole_line true gives
// it split_columns() columns (T*g <= split_columns()), false 16 distinct
// columns with repeated score passes; grid = resident workgroups of that
// kernel
hipError_t launch_multi_balanced(const DecodeArgs& a, int head_size,
                                 int block_size, int group, int grid,
                                 bool whole_line, hipStream_t stream);
int multi_balanced_grid(int head_size, int block_size, int group,
                        bool whole_line);
// distinct (row, head) columns of the whole-line body for this shape
int split_columns(int head_size, int group);
hipError_t launch_multi_reduce(const ReduceArgs& a, int head_size,
                               int num_q_tokens, hipStream_t stream);
// shared-prefix decode: part_start from the groups, then the prefix
// partitions of every group (grid (H_kv, groups x member tiles, shared
// partitions)); the rest is launch_decode (split mode) + launch_reduce
hipError_t launch_prefix_marks(const DecodeArgs& a, int block_size,
                               int* part_start, hipStream_t stream);
hipError_t launch_prefix(const DecodeArgs& a, int head_size, int block_size,
                         int group, dim3 grid, bool whole_line,
                         hipStream_t stream);
// elem_bytes: 2 for an fp16 pool, 1 for an fp8 (e4m3) pool
hipError_t launch_balanced(const DecodeArgs& a, int head_size, int block_size,
                           int group, int grid, hipStream_t stream,
                           int elem_bytes = 2);
// workgroups of the balanced kernel resident at once on the current device
// (0 if it cannot be determined)
int balanced_grid(int head_size, int block_size, int group, int elem_bytes = 2);

// cache operations
hipError_t launch_slot_mapping(int* out, const int* block_tables, int M,
                               int rows, const int* seq, const int* pos, int n,
                               int block_size, hipStream_t stream);
hipError_t launch_cache_write(const void* key, const void* value, void* kc,
                              void* vc, const int* slots, int n,
                              int64_t num_slots, int chunks_per_row,
                              hipStream_t stream);
// fp16 rows -> e4m3 codes of x / scale (clamped to the finite range)
hipError_t launch_cache_write_fp8(const void* key, const void* value, void* kc,
                                  void* vc, const int* slots, int n,
                                  int64_t num_slots, int chunks_per_row,
                                  float inv_k_scale, float inv_v_scale,
                                  hipStream_t stream);
hipError_t launch_copy_blocks(void* kc, void* vc, const int* src,
                              const int* dst, int pairs, int num_blocks,
                              int64_t chunks_per_block, hipStream_t stream);
hipError_t launch_swap_blocks(const void* sk, const void* sv, int snb, void* dk,
                              void* dv, int dnb, const int* src, const int* dst,
                              int pairs, int64_t chunks_per_block,
                              hipStream_t stream);

}  // namespace pa
