// C ABI of the paged KV-cache library: argument validation, launch shapes
// and dispatch to the gfx950 kernels.  Declarations and contracts: pa.h.
#include "pa.h"

#include <math.h>
#include <stdint.h>

#include "api_internal.h"
#include "decode.h"
#include "prefill.h"

namespace {

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

bool supported_head(int32_t d) { return d == 64 || d == 128; }
bool supported_block(int32_t b) { return b == 16 || b == 32 || b == 64; }
bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

// Checks shared by the decode entry points.
pa_status check_decode(const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_size,
                       int32_t block_size, int32_t num_blocks, float scale) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || num_seqs > 65535 ||
      num_kv_heads > 65535 || num_heads % num_kv_heads != 0 || !isfinite(scale))
    return PA_ERR_SHAPE;
  if (!supported_head(head_size) || !supported_block(block_size) ||
      !supported_group(num_heads / num_kv_heads))
    return PA_ERR_UNSUPPORTED;
  // per-block buffer records are 32-bit; table positions are int32
  const uint64_t block_bytes =
      (uint64_t)block_size * num_kv_heads * head_size * 2;
  if (block_bytes >= (1ull << 31) ||
      (int64_t)max_blocks_per_seq * block_size >= (1ll << 31))
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!query || !key_cache || !value_cache || !block_tables || !context_lens)
    return PA_ERR_NULL;
  if (!aligned(query, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(block_tables, 4) ||
      !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  return PA_OK;
}

int64_t max_partitions(int32_t max_blocks_per_seq, int32_t block_size,
                       int32_t partition_size) {
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  return (tokens + partition_size - 1) / partition_size;
}

pa_status hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// PA_CHECK=1: the device-side preconditions of a decode over these tables
// (and, for a fused step, the slots it writes), checked before any launch
pa_status checked_tables(const int32_t* block_tables, int32_t M,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_blocks, int32_t block_size, bool appends,
                         hipStream_t stream) {
  if (!pa::check_mode()) return PA_OK;
  return pa::device_check(block_tables, M, context_lens, num_seqs, num_blocks,
                          block_size, appends, nullptr, 0, stream);
}

// Balanced-split workspaces: a fixed header of kCounterSlots int32 range
// counters (pair q = seq * H_kv + kv head uses counter q), then max, sum
// (fp32 [rows]) and out (fp32 [rows, D]), rows = (grid + S*H_kv) * columns
// per pair (g for decode, 16 for multi-token rows).  The header does not
// depend on the call's shape, so one zero-filled workspace can serve calls
// of any shape in any order: every counter is zero between calls, and no
// call ever stores partial states over a counter.
constexpr size_t kCounterSlots = PA_BALANCED_MAX_PAIRS;
constexpr size_t kCounterBytes = PA_BALANCED_COUNTER_BYTES;
static_assert(kCounterBytes == kCounterSlots * 4 && kCounterBytes % 16 == 0,
              "state region stays 16-byte aligned");

bool counters_fit(int32_t num_seqs, int32_t num_kv_heads) {
  return (uint64_t)num_seqs * (uint64_t)num_kv_heads <= kCounterSlots;
}

// state rows of a balanced-split workspace with `cols` columns per pair
uint64_t balanced_rows(int32_t num_seqs, int32_t num_kv_heads, int32_t grid,
                       int32_t cols) {
  return ((uint64_t)grid + (uint64_t)num_seqs * num_kv_heads) * (uint64_t)cols;
}

void set_balanced(pa::DecodeArgs& a, char* ws) {
  a.bal_count = reinterpret_cast<int*>(ws);
}

}  // namespace

extern "C" {

const char* pa_status_str(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_CHECK: return "PA_ERR_CHECK";
  }
  return "PA_ERR_UNKNOWN";
}

void pa_kv_cache_shape(int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_size,
                       int64_t out_shape[5]) {
  if (!out_shape) return;
  out_shape[0] = 2;
  out_shape[1] = num_blocks;
  out_shape[2] = block_size;
  out_shape[3] = num_kv_heads;
  out_shape[4] = head_size;
}

pa_status pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t num_rows,
                          const int32_t* seq_idx, const int32_t* positions,
                          int32_t num_tokens, int32_t block_size,
                          hipStream_t stream) {
  if (num_tokens < 0 || num_rows < 0 || max_blocks_per_seq <= 0 ||
      block_size <= 0 ||
      (int64_t)max_blocks_per_seq * block_size >= (1ll << 31))
    return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!slot_mapping || !block_tables || !seq_idx || !positions) return PA_ERR_NULL;
  if (!aligned(slot_mapping, 4) || !aligned(block_tables, 4) ||
      !aligned(seq_idx, 4) || !aligned(positions, 4))
    return PA_ERR_ALIGN;
  return hip_status(pa::launch_slot_mapping(slot_mapping, block_tables,
                                            max_blocks_per_seq, num_rows,
                                            seq_idx, positions, num_tokens,
                                            block_size, stream));
}

pa_status pa_cache_write(const void* key, const void* value, void* key_cache,
                         void* value_cache, const int32_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_size <= 0 || head_size % 8 != 0)
    return PA_ERR_SHAPE;
  const int64_t cpr = (int64_t)num_kv_heads * head_size / 8;  // 16-byte chunks
  if (cpr >= (1ll << 31)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return PA_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 4))
    return PA_ERR_ALIGN;
  if (pa::check_mode()) {
    const pa_status c = pa::device_check(nullptr, 0, nullptr, 0, num_blocks, block_size,
                                         false, slot_mapping, num_tokens, stream);
    if (c != PA_OK) return c;
  }
  return hip_status(pa::launch_cache_write(
      key, value, key_cache, value_cache, slot_mapping, num_tokens,
      (int64_t)num_blocks * block_size, (int)cpr, stream));
}

pa_status pa_cache_write_fp8(const void* key, const void* value,
                             void* key_cache, void* value_cache,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             int32_t num_blocks, int32_t block_size,
                             int32_t num_kv_heads, int32_t head_size,
                             float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_size <= 0 || head_size % 8 != 0 ||
      !(isfinite(k_scale) && k_scale > 0.f) ||
      !(isfinite(v_scale) && v_scale > 0.f))
    return PA_ERR_SHAPE;
  const int64_t cpr = (int64_t)num_kv_heads * head_size / 8;  // 8-element chunks
  if (cpr >= (1ll << 31)) return PA_ERR_SHAPE;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return PA_ERR_NULL;
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(key_cache, 16) ||
      !aligned(value_cache, 16) || !aligned(slot_mapping, 4))
    return PA_ERR_ALIGN;
  if (pa::check_mode()) {
    const pa_status c = pa::device_check(nullptr, 0, nullptr, 0, num_blocks, block_size,
                                         false, slot_mapping, num_tokens, stream);
    if (c != PA_OK) return c;
  }
  return hip_status(pa::launch_cache_write_fp8(
      key, value, key_cache, value_cache, slot_mapping, num_tokens,
      (int64_t)num_blocks * block_size, (int)cpr, 1.f / k_scale, 1.f / v_scale,
      stream));
}

pa_status pa_copy_blocks(void* key_cache, void* value_cache,
                         const int32_t* src, const int32_t* dst,
                         int32_t num_pairs, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, hipStream_t stream) {
  if (num_pairs < 0 || num_blocks <= 0 || block_size <= 0 ||
      num_kv_heads <= 0 || head_size <= 0 || head_size % 8 != 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!key_cache || !value_cache || !src || !dst) return PA_ERR_NULL;
  if (!aligned(key_cache, 16) || !aligned(value_cache, 16) ||
      !aligned(src, 4) || !aligned(dst, 4))
    return PA_ERR_ALIGN;
  const int64_t cpb = (int64_t)block_size * num_kv_heads * head_size / 8;
  return hip_status(pa::launch_copy_blocks(key_cache, value_cache, src, dst,
                                           num_pairs, num_blocks, cpb, stream));
}

pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                         int32_t src_num_blocks, void* dst_key_cache,
                         void* dst_value_cache, int32_t dst_num_blocks,
                         const int32_t* src_ids, const int32_t* dst_ids,
                         int32_t num_pairs, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_size,
                         hipStream_t stream) {
  if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 ||
      block_size <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      head_size % 8 != 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!src_key_cache || !src_value_cache || !dst_key_cache ||
      !dst_value_cache || !src_ids || !dst_ids)
    return PA_ERR_NULL;
  if (!aligned(src_key_cache, 16) || !aligned(src_value_cache, 16) ||
      !aligned(dst_key_cache, 16) || !aligned(dst_value_cache, 16) ||
      !aligned(src_ids, 4) || !aligned(dst_ids, 4))
    return PA_ERR_ALIGN;
  const int64_t cpb = (int64_t)block_size * num_kv_heads * head_size / 8;
  return hip_status(pa::launch_swap_blocks(
      src_key_cache, src_value_cache, src_num_blocks, dst_key_cache,
      dst_value_cache, dst_num_blocks, src_ids, dst_ids, num_pairs, cpb, stream));
}

pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_size, int32_t block_size, int32_t num_blocks,
                    float scale, hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK || num_seqs == 0) return st;
  if (!out) return PA_ERR_NULL;
  if (!aligned(out, 16)) return PA_ERR_ALIGN;
  pa::DecodeArgs a = {};
  a.out = static_cast<_Float16*>(out);
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.partition_size = max_blocks_per_seq * block_size;   // whole sequence
  a.max_partitions = 1;
  a.split = 0;
  a.scale = scale;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  dim3 grid(num_kv_heads, num_seqs, 1);
  return hip_status(pa::launch_decode(a, head_size, block_size,
                                      num_heads / num_kv_heads, grid, stream));
}

size_t pa_splitk_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t head_size, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || head_size <= 0 ||
      max_blocks_per_seq <= 0 || block_size <= 0 || partition_size <= 0)
    return 0;
  const int64_t pm = max_partitions(max_blocks_per_seq, block_size, partition_size);
  const uint64_t rows = (uint64_t)num_seqs * num_heads * pm;
  return (size_t)(rows * 4 * 2 + rows * head_size * 4);
}

pa_status pa_decode_splitk(const void* query, const void* key_cache,
                           const void* value_cache,
                           const int32_t* block_tables,
                           int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_size, int32_t block_size,
                           int32_t num_blocks, float scale,
                           int32_t partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % block_size != 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  const int64_t pm = max_partitions(max_blocks_per_seq, block_size, partition_size);
  if (pm > 65535) return PA_ERR_SHAPE;        // grid.z
  if (!workspace) return PA_ERR_NULL;
  if (!aligned(workspace, 16)) return PA_ERR_ALIGN;
  if (workspace_bytes < pa_splitk_workspace_size(num_seqs, num_heads, head_size,
                                                 max_blocks_per_seq, block_size,
                                                 partition_size))
    return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_seqs * num_heads * pm;
  pa::DecodeArgs a = {};
  a.ws_max = static_cast<float*>(workspace);
  a.ws_sum = a.ws_max + rows;
  a.ws_out = a.ws_sum + rows;
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.partition_size = partition_size;
  a.max_partitions = (int)pm;
  a.split = 1;
  a.scale = scale;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  dim3 grid(num_kv_heads, num_seqs, (unsigned)pm);
  return hip_status(pa::launch_decode(a, head_size, block_size,
                                      num_heads / num_kv_heads, grid, stream));
}

size_t pa_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t head_size, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t partition_size) {
  const size_t split = pa_splitk_workspace_size(num_seqs, num_heads, head_size,
                                                max_blocks_per_seq, block_size,
                                                partition_size);
  if (split == 0 && num_seqs != 0) return 0;
  return split + (((size_t)(num_seqs > 0 ? num_seqs : 0) * 4 + 15) & ~(size_t)15);
}

pa_status pa_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t partition_size,
    const int32_t* group_offsets, const int32_t* group_members,
    const int32_t* group_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_group_blocks, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (partition_size <= 0 || partition_size % block_size != 0 ||
      num_groups < 0 || max_group_size < 0 || max_group_blocks < 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  const int64_t pm = max_partitions(max_blocks_per_seq, block_size, partition_size);
  if (pm > 65535) return PA_ERR_SHAPE;        // grid.z
  const int32_t g = num_heads / num_kv_heads;
  // members per prefix tile: the narrow form of the matrix-core body
  // (split_columns/g members) when it needs no more tiles than the
  // 16-column form
  const int64_t per16 = 16 / g;
  const int64_t perw = pa::split_columns(head_size, g) / g;
  const int64_t tiles16 = (max_group_size + per16 - 1) / per16;
  const int64_t tilesw = perw > 0 ? (max_group_size + perw - 1) / perw : tiles16 + 1;
  const bool whole_line = tilesw <= tiles16;
  const int64_t per_tile = whole_line ? perw : per16;
  const int64_t tiles = whole_line ? tilesw : tiles16;
  if ((int64_t)num_groups * (tiles > 0 ? tiles : 1) > 65535) return PA_ERR_SHAPE;
  if (!out || !workspace) return PA_ERR_NULL;
  if (num_groups > 0 && (!group_offsets || !group_members || !group_blocks))
    return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(workspace, 16) ||
      (num_groups > 0 && (!aligned(group_offsets, 4) ||
                          !aligned(group_members, 4) || !aligned(group_blocks, 4))))
    return PA_ERR_ALIGN;
  if (workspace_bytes < pa_prefix_workspace_size(num_seqs, num_heads, head_size,
                                                 max_blocks_per_seq, block_size,
                                                 partition_size))
    return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_seqs * num_heads * pm;
  pa::DecodeArgs a = {};
  a.ws_max = static_cast<float*>(workspace);
  a.ws_sum = a.ws_max + rows;
  a.ws_out = a.ws_sum + rows;
  int* part_start = reinterpret_cast<int*>(a.ws_out + rows * head_size);
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.partition_size = partition_size;
  a.max_partitions = (int)pm;
  a.split = 1;
  a.scale = scale;
  a.grp_offsets = group_offsets;
  a.grp_members = group_members;
  a.grp_blocks = group_blocks;
  a.num_groups = num_groups;
  int64_t gp = (int64_t)max_group_blocks * block_size / partition_size;
  a.grp_max_parts = (int)(gp < pm ? gp : pm);
  a.grp_max_members = (int)(tiles * per_tile);
  a.q_tiles = (int)(tiles > 0 ? tiles : 1);
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  st = hip_status(pa::launch_prefix_marks(a, block_size, part_start, stream));
  if (st != PA_OK) return st;
  if (num_groups > 0 && tiles > 0 && a.grp_max_parts > 0) {
    dim3 pg(num_kv_heads, (unsigned)(num_groups * tiles), (unsigned)a.grp_max_parts);
    st = hip_status(pa::launch_prefix(a, head_size, block_size, g, pg,
                                      whole_line, stream));
    if (st != PA_OK) return st;
  }
  a.part_start = part_start;
  dim3 grid(num_kv_heads, num_seqs, (unsigned)pm);
  st = hip_status(pa::launch_decode(a, head_size, block_size, g, grid, stream));
  if (st != PA_OK) return st;
  pa::ReduceArgs r = {};
  r.out = static_cast<_Float16*>(out);
  r.ws_max = a.ws_max;
  r.ws_sum = a.ws_sum;
  r.ws_out = a.ws_out;
  r.context_lens = context_lens;
  r.num_heads = num_heads;
  r.max_partitions = (int)pm;
  r.partition_size = partition_size;
  r.max_tokens = max_blocks_per_seq * block_size;
  return hip_status(pa::launch_reduce(r, head_size, num_seqs, stream));
}

size_t pa_multi_workspace_size(int32_t num_q_tokens, int32_t num_heads,
                               int32_t head_size, int32_t max_blocks_per_seq,
                               int32_t block_size, int32_t partition_size) {
  return pa_splitk_workspace_size(num_q_tokens, num_heads, head_size,
                                  max_blocks_per_seq, block_size,
                                  partition_size);
}

pa_status pa_decode_multi(void* out, const void* query, const void* key_cache,
                          const void* value_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                          int32_t max_q_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_size,
                          int32_t block_size, int32_t num_blocks, float scale,
                          int32_t partition_size, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (num_q_tokens < 0 || max_q_per_seq <= 0 || num_heads > 65535 ||
      partition_size <= 0 || partition_size % block_size != 0)
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_q_tokens == 0) return PA_OK;
  const int32_t g = num_heads / num_kv_heads;
  // the narrow form of the matrix-core body (split_columns/g query tokens
  // per tile) when it needs no more tiles, i.e. no more K/V passes, than the
  // 16-column form
  const int64_t per16 = 16 / g;
  const int64_t perw = pa::split_columns(head_size, g) / g;
  const int64_t tiles16 = (max_q_per_seq + per16 - 1) / per16;
  const int64_t tilesw = perw > 0 ? (max_q_per_seq + perw - 1) / perw : tiles16 + 1;
  const bool whole_line = tilesw <= tiles16;
  const int64_t tiles = whole_line ? tilesw : tiles16;
  const int64_t pm = max_partitions(max_blocks_per_seq, block_size, partition_size);
  if (pm > 65535 || (int64_t)num_seqs * tiles > 65535 || num_q_tokens > 65535)
    return PA_ERR_SHAPE;                      // grid.z, grid.y
  if (!out || !cu_seqlens_q || !workspace) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(workspace, 16) || !aligned(cu_seqlens_q, 4))
    return PA_ERR_ALIGN;
  if (workspace_bytes < pa_multi_workspace_size(num_q_tokens, num_heads,
                                                head_size, max_blocks_per_seq,
                                                block_size, partition_size))
    return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)num_q_tokens * num_heads * pm;
  pa::DecodeArgs a = {};
  a.ws_max = static_cast<float*>(workspace);
  a.ws_sum = a.ws_max + rows;
  a.ws_out = a.ws_sum + rows;
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.partition_size = partition_size;
  a.max_partitions = (int)pm;
  a.split = 1;
  a.scale = scale;
  a.cu_seqlens_q = cu_seqlens_q;
  a.q_tiles = (int)tiles;
  a.num_q_tokens = num_q_tokens;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  // more than 16 rows x heads per sequence: the matrix-core prefill body,
  // 128 of them per pass over a partition's keys, states in the same layout
  const int64_t ptiles = ((int64_t)max_q_per_seq * g + pa::kPrefillRows - 1) /
                         pa::kPrefillRows;
  if ((int64_t)max_q_per_seq * g > 16 && (int64_t)num_seqs * pm <= 65535 &&
      (int64_t)num_q_tokens * num_heads * head_size < (1ll << 31)) {
    pa::PrefillArgs p = {};
    p.query = a.query;
    p.key_cache = a.key_cache;
    p.value_cache = a.value_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.cu_seqlens_q = cu_seqlens_q;
    p.num_q_tokens = num_q_tokens;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.num_heads = num_heads;
    p.num_kv_heads = num_kv_heads;
    p.num_blocks = num_blocks;
    p.scale = scale;
    p.ws_max = a.ws_max;
    p.ws_sum = a.ws_sum;
    p.ws_out = a.ws_out;
    p.partition_size = partition_size;
    p.max_partitions = (int)pm;
    p.num_seqs = num_seqs;
    p.max_tokens = max_blocks_per_seq * block_size;
    p.out = static_cast<_Float16*>(out);
    dim3 pgrid(num_kv_heads, (unsigned)ptiles, (unsigned)(num_seqs * pm));
    st = hip_status(pa::launch_prefill(p, head_size, block_size, g, pgrid, true, stream));
    if (st != PA_OK) return st;
    return hip_status(pa::launch_prefill_fold(p, head_size, stream));
  } else {
    dim3 grid(num_kv_heads, (unsigned)(num_seqs * tiles), (unsigned)pm);
    st = hip_status(pa::launch_multi(a, head_size, block_size, g, grid,
                                     whole_line, stream));
  }
  if (st != PA_OK) return st;
  pa::ReduceArgs r = {};
  r.out = static_cast<_Float16*>(out);
  r.ws_max = a.ws_max;
  r.ws_sum = a.ws_sum;
  r.ws_out = a.ws_out;
  r.context_lens = context_lens;
  r.num_heads = num_heads;
  r.max_partitions = (int)pm;
  r.partition_size = partition_size;
  r.max_tokens = max_blocks_per_seq * block_size;
  r.cu_seqlens_q = cu_seqlens_q;
  r.num_seqs = num_seqs;
  return hip_status(pa::launch_multi_reduce(r, head_size, num_q_tokens, stream));
}

pa_status pa_prefill(void* out, const void* query, const void* key_cache,
                     const void* value_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                     int32_t num_q_tokens, int32_t max_q_per_seq,
                     const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size, int32_t num_blocks, float scale,
                     hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (num_q_tokens < 0 || max_q_per_seq <= 0) return PA_ERR_SHAPE;
  const int32_t g = num_heads / num_kv_heads;
  const int64_t tiles = ((int64_t)max_q_per_seq * g + pa::kPrefillRows - 1) /
                        pa::kPrefillRows;
  if (tiles > 65535) return PA_ERR_SHAPE;             // grid.y
  // row offsets of query and out are 32-bit in the kernel
  if ((int64_t)num_q_tokens * num_heads * head_size >= (1ll << 31)) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_q_tokens == 0) return PA_OK;
  if (!out || !cu_seqlens_q) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(cu_seqlens_q, 4)) return PA_ERR_ALIGN;
  pa::PrefillArgs a = {};
  a.out = static_cast<_Float16*>(out);
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_q_tokens = num_q_tokens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.scale = scale;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  dim3 grid(num_kv_heads, (unsigned)tiles, num_seqs);
  return hip_status(pa::launch_prefill(a, head_size, block_size, g, grid, false, stream));
}

// the narrow form of the matrix-core body when a sequence's rows x heads
// fit its columns, else the 16-column form
static bool multi_whole_line(int32_t head_size, int32_t g, int32_t max_q) {
  return (int64_t)max_q * g <= pa::split_columns(head_size, g);
}

// column tiles per (sequence, kv head) of the balanced multi-token kernel:
// one for the narrow form, ceil(max_q * g / 16) for the 16-column form
static int64_t multi_tiles(int32_t head_size, int32_t g, int32_t max_q) {
  if (multi_whole_line(head_size, g, max_q)) return 1;
  return ((int64_t)max_q * g + 15) / 16;
}

int32_t pa_multi_balanced_grid(int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size,
                               int32_t max_q_per_seq) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !supported_head(head_size) || !supported_block(block_size) ||
      !supported_group(num_heads / num_kv_heads) || max_q_per_seq <= 0 ||
      max_q_per_seq > 65535)
    return 0;
  const int32_t g = num_heads / num_kv_heads;
  const bool narrow = multi_whole_line(head_size, g, max_q_per_seq);
  const int32_t grid = pa::multi_balanced_grid(head_size, block_size, g, narrow);
  // The narrow form's 4-column body fits four workgroups per CU; two run
  // faster (half the slices, half the cut pairs).  Measured on MI355X,
  // grid 1024 / 768 / 512: 4-token verify of the Llama-2-13B layer 121.0 /
  // 118.9 / 111.6 us, one query row per sequence on GQA-4 67.5 / 65.7 /
  // 61.0.  The 8-column body fits three and stays there (2-token GQA-4
  // verify 77.5 at 768, 78.4 at 512).
  if (narrow && grid > 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) ==
            hipSuccess &&
        cus > 0 && grid >= 4 * cus)
      return 2 * cus;
  }
  return grid;
}

// the fixed counter header, then max, sum (fp32 [rows]) and out (fp32
// [rows, D]) with rows = (grid + S*H_kv) * 16.
size_t pa_multi_balanced_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t head_size, int32_t grid) {
  if (num_seqs < 0 || num_kv_heads <= 0 || head_size <= 0 || grid <= 0 ||
      !counters_fit(num_seqs, num_kv_heads))
    return 0;
  const uint64_t rows = balanced_rows(num_seqs, num_kv_heads, grid, 16);
  return kCounterBytes + (size_t)(rows * 8 + rows * head_size * 4);
}

// the same layout with a counter and a state row group per (sequence, kv
// head, column tile)
size_t pa_multi_balanced_workspace_size_tiles(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads,
                                              int32_t head_size, int32_t grid,
                                              int32_t max_q_per_seq) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 ||
      num_heads % num_kv_heads != 0 || head_size <= 0 || grid <= 0 ||
      max_q_per_seq <= 0 || max_q_per_seq > 65535)
    return 0;
  const int64_t tl = multi_tiles(head_size, num_heads / num_kv_heads, max_q_per_seq);
  if ((uint64_t)num_seqs * num_kv_heads * tl > kCounterSlots) return 0;
  const uint64_t rows = ((uint64_t)grid + (uint64_t)num_seqs * num_kv_heads * tl) * 16;
  return kCounterBytes + (size_t)(rows * 8 + rows * head_size * 4);
}

pa_status pa_decode_multi_balanced(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, int32_t num_q_tokens, int32_t max_q_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t grid, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (num_q_tokens < 0 || max_q_per_seq <= 0 || max_q_per_seq > 65535 ||
      grid <= 0 || grid > (1 << 20))
    return PA_ERR_SHAPE;
  const int32_t g = num_heads / num_kv_heads;
  const int64_t tl = multi_tiles(head_size, g, max_q_per_seq);
  if ((uint64_t)num_seqs * num_kv_heads * tl > kCounterSlots) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_q_tokens == 0) return PA_OK;
  if (!out || !cu_seqlens_q || !workspace) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(workspace, 16) || !aligned(cu_seqlens_q, 4))
    return PA_ERR_ALIGN;
  if (workspace_bytes <
      pa_multi_balanced_workspace_size_tiles(num_seqs, num_heads, num_kv_heads,
                                             head_size, grid, max_q_per_seq))
    return PA_ERR_WORKSPACE;
  const size_t rows = ((size_t)grid + (size_t)num_seqs * num_kv_heads * tl) * 16;
  char* ws = static_cast<char*>(workspace);
  float* fmax = reinterpret_cast<float*>(ws + kCounterBytes);
  pa::DecodeArgs a = {};
  a.out = static_cast<_Float16*>(out);
  a.ws_max = fmax;
  a.ws_sum = fmax + rows;
  a.ws_out = fmax + 2 * rows;
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  set_balanced(a, ws);
  a.split = 1;
  a.scale = scale;
  a.cu_seqlens_q = cu_seqlens_q;
  a.num_q_tokens = num_q_tokens;
  a.q_tiles = (int)tl;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, false, stream);
  if (st != PA_OK) return st;
  return hip_status(pa::launch_multi_balanced(
      a, head_size, block_size, g, grid,
      multi_whole_line(head_size, g, max_q_per_seq), stream));
}

pa_status pa_decode_reduce(void* out, const void* workspace,
                           size_t workspace_bytes,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_size,
                           int32_t max_blocks_per_seq, int32_t block_size,
                           int32_t partition_size, hipStream_t stream) {
  if (num_seqs < 0 || num_heads <= 0 || max_blocks_per_seq <= 0 ||
      num_seqs > 65535 || num_heads > 65535 || block_size <= 0 ||
      partition_size <= 0 || partition_size % block_size != 0 ||
      (int64_t)max_blocks_per_seq * block_size >= (1ll << 31))
    return PA_ERR_SHAPE;
  if (!supported_head(head_size) || !supported_block(block_size))
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !workspace || !context_lens) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(workspace, 16) || !aligned(context_lens, 4))
    return PA_ERR_ALIGN;
  if (workspace_bytes < pa_splitk_workspace_size(num_seqs, num_heads, head_size,
                                                 max_blocks_per_seq, block_size,
                                                 partition_size))
    return PA_ERR_WORKSPACE;
  const int64_t pm = max_partitions(max_blocks_per_seq, block_size, partition_size);
  const size_t rows = (size_t)num_seqs * num_heads * pm;
  pa::ReduceArgs a = {};
  a.out = static_cast<_Float16*>(out);
  a.ws_max = static_cast<const float*>(workspace);
  a.ws_sum = a.ws_max + rows;
  a.ws_out = a.ws_sum + rows;
  a.context_lens = context_lens;
  a.num_heads = num_heads;
  a.max_partitions = (int)pm;
  a.partition_size = partition_size;
  a.max_tokens = max_blocks_per_seq * block_size;
  return hip_status(pa::launch_reduce(a, head_size, num_seqs, stream));
}

int32_t pa_balanced_grid(int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !supported_head(head_size) || !supported_block(block_size) ||
      !supported_group(num_heads / num_kv_heads))
    return 0;
  return pa::balanced_grid(head_size, block_size, num_heads / num_kv_heads);
}

int32_t pa_balanced_grid_fp8(int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size) {
  if (num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads != 0 ||
      !supported_head(head_size) || !supported_block(block_size) ||
      !supported_group(num_heads / num_kv_heads))
    return 0;
  return pa::balanced_grid(head_size, block_size, num_heads / num_kv_heads, 1);
}


size_t pa_balanced_workspace_size(int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size,
                                  int32_t grid) {
  if (num_seqs < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_size <= 0 ||
      grid <= 0 || num_heads % num_kv_heads != 0 ||
      !counters_fit(num_seqs, num_kv_heads))
    return 0;
  const uint64_t rows = balanced_rows(num_seqs, num_kv_heads, grid,
                                      num_heads / num_kv_heads);
  return kCounterBytes + (size_t)(rows * 8 + rows * head_size * 4);
}

}  // extern "C"

namespace pa {

// The balanced decode (with the fused append when key/value are given)
// whose range counters (counter_slots int32, zero between calls) and
// partial states (state_bytes) live at caller-given device addresses.
pa_status balanced_run(void* out, const void* query, void* key_cache,
                       void* value_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t num_blocks,
                       float scale, int32_t grid, int* counters,
                       size_t counter_slots, float* states, size_t state_bytes,
                       const void* key, const void* value, int32_t* slot_mapping,
                       hipStream_t stream, int elem_bytes, float k_scale,
                       float v_scale, bool launch) {
  pa_status st = check_decode(query, key_cache, value_cache, block_tables,
                              max_blocks_per_seq, context_lens, num_seqs,
                              num_heads, num_kv_heads, head_size, block_size,
                              num_blocks, scale);
  if (st != PA_OK) return st;
  if (grid <= 0 || grid > (1 << 20) || !counters_fit(num_seqs, num_kv_heads))
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  if (!out || (launch && (!counters || !states))) return PA_ERR_NULL;
  if (!aligned(out, 16) || !aligned(states, 16) || !aligned(counters, 4) ||
      (key && (!aligned(key, 16) || !aligned(value, 16))) ||
      (slot_mapping && !aligned(slot_mapping, 4)))
    return PA_ERR_ALIGN;
  const int32_t g = num_heads / num_kv_heads;
  const size_t rows = balanced_rows(num_seqs, num_kv_heads, grid, g);
  if ((uint64_t)num_seqs * num_kv_heads > counter_slots ||
      state_bytes < rows * 8 + rows * (size_t)head_size * 4)
    return PA_ERR_WORKSPACE;
  if (!launch) return PA_OK;
  st = checked_tables(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                      num_blocks, block_size, key != nullptr, stream);
  if (st != PA_OK) return st;
  pa::DecodeArgs a = {};
  a.out = static_cast<_Float16*>(out);
  a.ws_max = states;
  a.ws_sum = states + rows;
  a.ws_out = states + 2 * rows;
  a.query = static_cast<const _Float16*>(query);
  a.key_cache = static_cast<const char*>(key_cache);
  a.value_cache = static_cast<const char*>(value_cache);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.num_blocks = num_blocks;
  a.num_seqs = num_seqs;
  a.bal_count = counters;
  a.new_key = static_cast<const _Float16*>(key);
  a.new_value = static_cast<const _Float16*>(value);
  a.slot_out = slot_mapping;
  a.split = 1;
  a.scale = scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.inv_k_scale = 1.f / k_scale;
  a.inv_v_scale = 1.f / v_scale;
  return hip_status(pa::launch_balanced(a, head_size, block_size, g, grid,
                                        stream, elem_bytes));
}

}  // namespace pa

extern "C" {

static pa_status balanced_impl(void* out, const void* query, void* key_cache,
                               void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size,
                               int32_t num_blocks, float scale, int32_t grid,
                               void* workspace, size_t workspace_bytes,
                               const void* key, const void* value,
                               int32_t* slot_mapping, hipStream_t stream,
                               int elem_bytes = 2, float k_scale = 1.f,
                               float v_scale = 1.f) {
  // the workspace: the fixed counter header, then the states
  char* ws = static_cast<char*>(workspace);
  return pa::balanced_run(
      out, query, key_cache, value_cache, block_tables, max_blocks_per_seq,
      context_lens, num_seqs, num_heads, num_kv_heads, head_size, block_size,
      num_blocks, scale, grid, reinterpret_cast<int*>(ws), kCounterSlots,
      ws ? reinterpret_cast<float*>(ws + kCounterBytes) : nullptr,
      workspace_bytes >= kCounterBytes ? workspace_bytes - kCounterBytes : 0, key,
      value, slot_mapping, stream, elem_bytes, k_scale, v_scale, true);
}

pa_status pa_decode_balanced(void* out, const void* query, const void* key_cache,
                             const void* value_cache,
                             const int32_t* block_tables,
                             int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size,
                             int32_t num_blocks, float scale, int32_t grid,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  return balanced_impl(out, query, const_cast<void*>(key_cache),
                       const_cast<void*>(value_cache), block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_size, block_size, num_blocks, scale,
                       grid, workspace, workspace_bytes, nullptr, nullptr,
                       nullptr, stream);
}

pa_status pa_decode_balanced_fp8(void* out, const void* query,
                                 const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables,
                                 int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size,
                                 int32_t num_blocks, float scale, float k_scale,
                                 float v_scale, int32_t grid, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (!(isfinite(k_scale) && k_scale > 0.f) ||
      !(isfinite(v_scale) && v_scale > 0.f))
    return PA_ERR_SHAPE;
  return balanced_impl(out, query, const_cast<void*>(key_cache),
                       const_cast<void*>(value_cache), block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_size, block_size, num_blocks, scale,
                       grid, workspace, workspace_bytes, nullptr, nullptr,
                       nullptr, stream, 1, k_scale, v_scale);
}

pa_status pa_decode_step_fp8(void* out, const void* query, const void* key,
                             const void* value, void* key_cache,
                             void* value_cache, int32_t* slot_mapping,
                             const int32_t* block_tables,
                             int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size,
                             int32_t num_blocks, float scale, float k_scale,
                             float v_scale, int32_t grid, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!(isfinite(k_scale) && k_scale > 0.f) ||
      !(isfinite(v_scale) && v_scale > 0.f))
    return PA_ERR_SHAPE;
  if (num_seqs > 0 && (!key || !value)) return PA_ERR_NULL;
  return balanced_impl(out, query, key_cache, value_cache, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_size, block_size, num_blocks, scale,
                       grid, workspace, workspace_bytes, key, value,
                       slot_mapping, stream, 1, k_scale, v_scale);
}

pa_status pa_decode_step(void* out, const void* query, const void* key,
                         const void* value, void* key_cache, void* value_cache,
                         int32_t* slot_mapping, const int32_t* block_tables,
                         int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size,
                         int32_t num_blocks, float scale, int32_t grid,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (num_seqs > 0 && (!key || !value)) return PA_ERR_NULL;
  return balanced_impl(out, query, key_cache, value_cache, block_tables,
                       max_blocks_per_seq, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_size, block_size, num_blocks, scale,
                       grid, workspace, workspace_bytes, key, value,
                       slot_mapping, stream);
}

}  // extern "C"
