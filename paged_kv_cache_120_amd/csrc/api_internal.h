// Internal entry shared by the C ABI's balanced decode calls (not part of
// the ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// The balanced decode (with the fused append when key/value are given)
// whose range counters (counter_slots int32 words, zero between calls) and
// partial states (state_bytes, 16-byte aligned) live at device addresses
// the caller provides.  Validates every argument before launching;
// PA_ERR_WORKSPACE when the shape needs more counters or state bytes than
// given.  launch = false: validation only (counters and states may then be
// null; nothing touches the device).
pa_status balanced_run(void* out, const void* query, void* key_cache,
                       void* value_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_size, int32_t block_size, int32_t num_blocks,
                       float scale, int32_t grid, int* counters,
                       size_t counter_slots, float* states, size_t state_bytes,
                       const void* key, const void* value, int32_t* slot_mapping,
                       hipStream_t stream, int elem_bytes, float k_scale,
                       float v_scale, bool launch);

// PA_CHECK=1 in the environment (read at every call)
bool check_mode();

// The validation pass of PA_CHECK=1, run on `stream` and waited for: for
// the num_seqs sequences (when block_tables is given) context length <=
// M * block_size and every table entry a decode reads in [0, num_blocks);
// for the slots -- the explicit list `slots` [num_slots], or (derived_slots)
// the slot a fused step writes for each sequence -- in range and pairwise
// distinct.  PA_ERR_CHECK if any check fails (pa_last_check() says which).
pa_status device_check(const int32_t* block_tables, int32_t M,
                       const int32_t* context_lens, int32_t num_seqs,
                       int32_t num_blocks, int32_t block_size, bool derived_slots,
                       const int32_t* slots, int32_t num_slots, hipStream_t stream);

}  // namespace pa
