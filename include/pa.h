/*
 * pa.h -- C ABI of the MI355X (gfx950) paged KV-cache decode library.
 *
 * What is computed comes from these pages (cited by title and section):
 *   [BOOK] vLLM book ch.4 "PagedAttention：虚拟内存的启示" (yangyitao.com)
 *   [GUST] "PagedAttention：KV Cache的虚拟内存" (thegustafson.com "Paged
 *          Attention", bittide translation)
 *   [P5]   "PagedAttention原理（下）" (5688vip, vLLM推理框架全解析 04)
 *   [CSDN] CSDN PageAttention tutorial (nanhubrain.csdn.net)
 *
 * Conventions shared by every entry point
 *   - Every pointer is a device pointer unless stated otherwise.  The caller
 *     owns all memory; the library never allocates, frees or keeps a pointer
 *     after a call returns.  Work is enqueued on `stream` (0 = null stream)
 *     and the call returns without synchronising.
 *   - Errors are returned, never thrown.  Host-checkable arguments are
 *     validated before anything is enqueued; a failed launch returns
 *     PA_ERR_HIP.  Device-side preconditions are listed per call; where a
 *     kernel can still check one cheaply it skips the offending element
 *     instead of faulting (stated per call).
 *   - fp16 buffers are IEEE binary16 and must be 16-byte aligned; int32
 *     buffers 4-byte aligned.  All tensors are dense row-major.
 *   - Layout of one layer's pool ([BOOK] §4.3.1): a (2, num_blocks,
 *     block_size, num_kv_heads, head_size) fp16 tensor; index 0 of the first
 *     axis is K, index 1 is V.  key_cache / value_cache below are the two
 *     halves, each [num_blocks, block_size, num_kv_heads, head_size].  A
 *     "slot" is a row index into a half seen as [num_blocks*block_size,
 *     num_kv_heads, head_size], so slot = block * block_size + offset.
 *   - Supported shapes: head_size 64 or 128; block_size 16, 32 or 64;
 *     num_heads / num_kv_heads (the GQA group) 1, 2, 4 or 8.  Other shapes
 *     return PA_ERR_UNSUPPORTED.
 */
#ifndef PAGED_KV_PA_H
#define PAGED_KV_PA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int pa_status;

#define PA_OK 0
#define PA_ERR_NULL 1          /* a required pointer is NULL */
#define PA_ERR_SHAPE 2         /* a size is out of range or inconsistent */
#define PA_ERR_UNSUPPORTED 3   /* head_size / block_size / group not built */
#define PA_ERR_ALIGN 4         /* a pointer is not aligned as required */
#define PA_ERR_WORKSPACE 5     /* split-KV workspace too small */
#define PA_ERR_HIP 6           /* the HIP runtime reported an error */
#define PA_ERR_CHECK 7         /* PA_CHECK=1 only: a device-side precondition fails */

/*
 * Validation mode.  With the environment variable PA_CHECK set to 1 (read
 * at every call), the decode calls (pa_decode, pa_decode_splitk,
 * pa_decode_balanced, pa_decode_step, their fp8 forms, pa_decode_multi,
 * pa_decode_multi_balanced, pa_decode_shared_prefix,
 * pa_decode_step_noalloc) and the cache writes first run a validation pass
 * on the device, wait for it on `stream` (the one case where a call
 * synchronises; so not under graph capture), and return PA_ERR_CHECK with
 * nothing else enqueued if it finds a violated precondition:
 *   PA_CHECK_CONTEXT         context_lens[i] > max_blocks_per_seq * block_size
 *   PA_CHECK_TABLE           a table entry a decode reads (logical blocks
 *                            below ceil(context_lens[i] / block_size)) is
 *                            outside [0, num_blocks)
 *   PA_CHECK_SLOT_RANGE      a cache-write slot >= num_blocks * block_size
 *   PA_CHECK_DUPLICATE_SLOT  two tokens write the same slot (the cache
 *                            write's slot_mapping, or the slots a fused
 *                            step derives: two sequences whose last token
 *                            falls in one shared block position)
 * pa_last_check() returns these bits for the last pass on the calling host
 * thread.  The shared-prefix groups and cu_seqlens_q are not checked.
 * [P5] §4.1 recounts a block table shared by all requests whose concurrent
 * updates scrambled the logical-to-physical mapping; this mode catches the
 * marks such a bug leaves in the inputs: ids outside the pool and two tokens
 * writing one slot.
 */
#define PA_CHECK_CONTEXT 1u
#define PA_CHECK_TABLE 2u
#define PA_CHECK_SLOT_RANGE 4u
#define PA_CHECK_DUPLICATE_SLOT 8u
uint32_t pa_last_check(void);

/* Balanced-split workspaces (pa_decode_balanced, pa_decode_step, their fp8
 * forms and pa_decode_multi_balanced) start with a fixed header of range
 * counters: at most PA_BALANCED_MAX_PAIRS (sequence, kv head) pairs per
 * call (more: PA_ERR_SHAPE). */
#define PA_BALANCED_MAX_PAIRS (1 << 18)
#define PA_BALANCED_COUNTER_BYTES (4 * PA_BALANCED_MAX_PAIRS)

/* Human-readable name of a status code (static string, never NULL). */
const char* pa_status_str(pa_status status);

/* Shape of one layer's pool: writes (2, num_blocks, block_size, num_kv_heads,
 * head_size) to out_shape[0..4] (host memory) ([BOOK] §4.3.1). */
void pa_kv_cache_shape(int32_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_size,
                       int64_t out_shape[5]);

/*
 * pa_slot_mapping -- physical slot of each token to be written ([BOOK] §4.4.3).
 *   For token j with table row r = seq_idx[j] and logical position
 *   p = positions[j]:  slot_mapping[j] = block_tables[r, p / block_size] *
 *   block_size + p % block_size.
 *   block_tables  int32 [num_rows, max_blocks_per_seq]
 *   seq_idx       int32 [num_tokens], positions int32 [num_tokens]
 *   slot_mapping  int32 [num_tokens] (output)
 *   A token whose row is outside [0, num_rows) or whose position is outside
 *   [0, max_blocks_per_seq * block_size) gets slot -1 (no write).
 *   num_tokens == 0 is a no-op.
 */
pa_status pa_slot_mapping(int32_t* slot_mapping, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, int32_t num_rows,
                          const int32_t* seq_idx, const int32_t* positions,
                          int32_t num_tokens, int32_t block_size,
                          hipStream_t stream);

/*
 * pa_cache_write -- write new tokens' K and V into their slots ([BOOK] §4.3.2,
 * §4.5 (1): reshape_and_cache with slot_mapping).
 *   key, value    fp16 [num_tokens, num_kv_heads, head_size]
 *   key_cache, value_cache  fp16 [num_blocks, block_size, num_kv_heads,
 *                 head_size] (written in place)
 *   slot_mapping  int32 [num_tokens]; slot < 0 or >= num_blocks*block_size
 *                 means "skip this token".
 *   A bit-exact copy (no arithmetic).  Precondition: the non-negative slots
 *   are distinct (otherwise which token lands last is unspecified).
 *   num_tokens == 0 is a no-op.
 */
pa_status pa_cache_write(const void* key, const void* value, void* key_cache,
                         void* value_cache, const int32_t* slot_mapping,
                         int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, hipStream_t stream);

/*
 * pa_copy_blocks -- copy-on-write block copies ([GUST] copy-on-write
 * paragraph; [P5] §4.3 steps): for each pair k, physical block src[k] of both
 * key_cache and value_cache is copied bit-exactly into block dst[k].
 *   src, dst      int32 [num_pairs]; a pair with an id outside
 *                 [0, num_blocks) is skipped.
 *   Precondition: no dst is also a src or another pair's dst.
 */
pa_status pa_copy_blocks(void* key_cache, void* value_cache,
                         const int32_t* src, const int32_t* dst,
                         int32_t num_pairs, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads,
                         int32_t head_size, hipStream_t stream);

/*
 * pa_swap_blocks -- batched block moves between two pools ([P5] §4.4: the
 * physical blocks of a paused request are moved out to CPU memory to free
 * device memory, and back before it resumes).  For each pair k, physical
 * block src_ids[k] of (src_key_cache, src_value_cache) is copied
 * bit-exactly to block dst_ids[k] of (dst_key_cache, dst_value_cache).
 *   Pools       fp16 [num_blocks, block_size, num_kv_heads, head_size] each
 *               (the two halves of a (2, nb, ...) pool); either pool may be
 *               device memory or pinned host memory mapped for the device
 *               (hipHostMalloc / torch pin_memory), so one call swaps out
 *               (device -> host) or in (host -> device).
 *   src_ids, dst_ids  int32 [num_pairs], device-accessible; a pair with an
 *               id outside [0, src_num_blocks) or [0, dst_num_blocks) is
 *               skipped.
 *   One kernel on `stream` moves all pairs; the host must not touch the
 *   host pool until the stream has passed the call.
 *   Precondition: the dst blocks are distinct and do not overlap the src
 *   blocks being read.
 */
pa_status pa_swap_blocks(const void* src_key_cache, const void* src_value_cache,
                         int32_t src_num_blocks, void* dst_key_cache,
                         void* dst_value_cache, int32_t dst_num_blocks,
                         const int32_t* src_ids, const int32_t* dst_ids,
                         int32_t num_pairs, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_size,
                         hipStream_t stream);

/*
 * pa_decode -- single-pass paged decode attention ([BOOK] §4.5, §4.6).
 *   For sequence i and query head h (kv head h / (num_heads/num_kv_heads)):
 *     out[i,h,:] = sum_t softmax_t(scale * <query[i,h,:], K_t>) * V_t
 *   over exactly t = 0 .. context_lens[i]-1, where token t lives at offset
 *   t % block_size of physical block block_tables[i, t / block_size].
 *   Statistics and accumulation in fp32 (online softmax, [BOOK] §4.6); out
 *   is rounded to fp16 (nearest even).
 *   out, query    fp16 [num_seqs, num_heads, head_size]
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; entries at or past
 *                 ceil(context_lens[i]/block_size) are never read.
 *   context_lens  int32 [num_seqs]; values above max_blocks_per_seq *
 *                 block_size are clamped to it; a value <= 0 gives zeros.
 *   Slots past context_lens[i] in the last block are never read, so they
 *   may hold anything (Inf/NaN included).
 *   Precondition: the table entries that are read are in [0, num_blocks);
 *   a block outside that range is read as all-zero instead of faulting.
 *   One workgroup walks one (sequence, kv head) end to end: use
 *   pa_decode_splitk for long contexts.  num_seqs == 0 is a no-op.
 */
pa_status pa_decode(void* out, const void* query, const void* key_cache,
                    const void* value_cache, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                    int32_t head_size, int32_t block_size, int32_t num_blocks,
                    float scale, hipStream_t stream);

/*
 * Split-KV workspace.  The three partial-state arrays of the split form --
 * per partition its maximum, its sum of exponentials and its unnormalised
 * output, the (m, s, O) state that [BOOK] §4.6 merges blockwise -- travel as
 * ONE caller-owned buffer instead of three pointers, so that a caller sizes,
 * allocates and passes a single object and the pair of calls cannot be
 * handed mismatched arrays.  With Pmax = ceil(max_blocks_per_seq *
 * block_size / partition_size) (256 for 128K-token contexts split into
 * 512-token partitions), it holds, in this order and back to back:
 *   max_logits fp32 [num_seqs, num_heads, Pmax]
 *   exp_sums   fp32 [num_seqs, num_heads, Pmax]
 *   tmp_out    fp32 [num_seqs, num_heads, Pmax, head_size]
 * The caller owns it; the library neither keeps nor frees it, and reads or
 * writes only the entries of non-empty partitions.
 * pa_splitk_workspace_size returns its size in bytes (0 on bad arguments).
 */
size_t pa_splitk_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t head_size, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t partition_size);

/*
 * pa_decode_splitk -- per-partition softmax state for split-KV decode.
 *   Partition p of sequence i is tokens [p*P, min((p+1)*P, n_i)) with
 *   P = partition_size (a multiple of block_size; Pmax below must not
 *   exceed 65535).  For each
 *   non-empty (i, h, p) it stores, with x_t = scale * <query[i,h], K_t>:
 *     max_logits[i,h,p] = m = max_t x_t
 *     exp_sums[i,h,p]   = sum_t exp(x_t - m)
 *     tmp_out[i,h,p,:]  = sum_t exp(x_t - m) * V_t      (not normalised)
 *   Empty partitions (p*P >= n_i) are not written.  Arguments otherwise as
 *   pa_decode; `workspace` is device memory of workspace_bytes >=
 *   pa_splitk_workspace_size(...), 16-byte aligned.
 */
pa_status pa_decode_splitk(const void* query, const void* key_cache,
                           const void* value_cache,
                           const int32_t* block_tables,
                           int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_size, int32_t block_size,
                           int32_t num_blocks, float scale,
                           int32_t partition_size, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_reduce -- merge the partitions written by pa_decode_splitk with
 * the online-softmax recurrence of [BOOK] §4.6:
 *   M = max_p m_p,  S = sum_p s_p exp(m_p - M),
 *   out[i,h,:] = sum_p exp(m_p - M) O_p / S     (fp16, nearest even)
 * over the non-empty partitions p < ceil(n_i / P) only.  Same workspace,
 * sizes and partition_size as the pa_decode_splitk call it follows (on the
 * same stream).  A sequence with context_lens[i] <= 0 gets zeros.
 */
pa_status pa_decode_reduce(void* out, const void* workspace,
                           size_t workspace_bytes,
                           const int32_t* context_lens, int32_t num_seqs,
                           int32_t num_heads, int32_t head_size,
                           int32_t max_blocks_per_seq, int32_t block_size,
                           int32_t partition_size, hipStream_t stream);

/*
 * Balanced split-KV decode: the same result as pa_decode (within the same
 * tolerance; the summation order differs), with the work divided evenly
 * instead of by sequence or fixed partition, in ONE kernel.  The KV work of
 * all (sequence, kv head) pairs is laid end to end -- sequence-major, then
 * kv head, then token, each sequence padded to a multiple of 16 tokens --
 * and cut into `grid` equal slices, one per workgroup.  A pair inside one
 * slice is finished there; a pair cut across k slices leaves k partial
 * softmax states (max, sum, unnormalised output: the form of [BOOK] §4.6),
 * and whichever of its workgroups finishes last merges them with the §4.6
 * recurrence.  Slice boundaries and the merge order depend only on the
 * shape, so repeated calls give bit-identical outputs.  With `grid` =
 * pa_balanced_grid(...) every workgroup is resident from the start, so
 * none waits on another.
 *
 * pa_balanced_grid: workgroups of the balanced kernel that the current
 *   device holds at once for this shape (0 if unsupported or unknown).
 * pa_balanced_workspace_size: bytes of device workspace for `grid`
 *   workgroups (0 on bad arguments, or when num_seqs * num_kv_heads
 *   exceeds PA_BALANCED_MAX_PAIRS).  Layout: a fixed header of
 *   PA_BALANCED_COUNTER_BYTES holding int32 range counters (pair
 *   i * num_kv_heads + kv head uses counter i * num_kv_heads + kv head),
 *   then fp32 max [rows], sum [rows], out [rows, head_size] with rows =
 *   (grid + num_seqs * num_kv_heads) * group.
 *   Zero-fill the workspace once before its first call; every completed
 *   call leaves all counters zero, and since the header does not depend on
 *   the call's shape, the same workspace then serves any later call, of
 *   any shape, whose size requirement it meets (a serving loop can size it
 *   for its largest batch and reuse it for every batch).  Calls that share
 *   a workspace must not overlap.
 * pa_decode_balanced: arguments as pa_decode plus grid (> 0) and the
 *   workspace (16-byte aligned, >= pa_balanced_workspace_size).  Same
 *   preconditions and guards as pa_decode.
 */
int32_t pa_balanced_grid(int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size);
size_t pa_balanced_workspace_size(int32_t num_seqs, int32_t num_heads,
                                  int32_t num_kv_heads, int32_t head_size,
                                  int32_t grid);
pa_status pa_decode_balanced(void* out, const void* query,
                             const void* key_cache, const void* value_cache,
                             const int32_t* block_tables,
                             int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size,
                             int32_t num_blocks, float scale, int32_t grid,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Multi-token queries over the same block tables (speculative verify,
 * chunked prefill): [BOOK] §4.5 (2) has the attention backend take the
 * query tokens of every request delimited by cu_seqlens_q together with the
 * per-request key counts and the block table; §4.5 (1) writes the new
 * tokens' K/V into the cache first.  Sequence i owns query rows
 * cu_seqlens_q[i] .. cu_seqlens_q[i+1]-1, the last T_i of its
 * context_lens[i] = n_i tokens (already in the cache); row cu_seqlens_q[i]
 * + j sits at position p = n_i - T_i + j and attends to keys 0 .. p only
 * (causal).  Tolerance as pa_decode.
 *   query, out     fp16 [num_q_tokens, num_heads, head_size], 16-byte
 *                  aligned; out is written for every row of a sequence
 *                  with T_i > 0 (zeros where context_lens[i] <= 0 or the
 *                  row has no key, T_i > n_i)
 *   cu_seqlens_q   int32 [num_seqs + 1], device, non-decreasing, from 0 to
 *                  num_q_tokens (precondition, not checked)
 *   max_q_per_seq  >= every T_i (host value sizing the launch; rows past
 *                  it are not computed)
 *   partition_size keys per partition, a multiple of block_size; the rows
 *                  of a sequence are computed per partition of its keys in
 *                  one kernel and a second kernel folds the partitions with
 *                  the [BOOK] §4.6 recurrence.  Up to 16 rows x heads per
 *                  sequence share a pass over a partition's keys on the
 *                  decode bodies (4-8 on the narrow form); beyond 16
 *                  (chunked prefill) 128 of them do, on pa_prefill's
 *                  matrix-core body (when num_seqs * Pmax <= 65535 and
 *                  num_q_tokens * num_heads * head_size < 2^31, else the
 *                  16-column decode body in tiles)
 *   workspace      device, 16-byte aligned, >= pa_multi_workspace_size
 *                  bytes: fp32 max and sum [num_q_tokens, num_heads,
 *                  Pmax] and out [.., head_size] (Pmax as for
 *                  pa_decode_splitk); no zero-fill needed
 * Other arguments, preconditions and errors as pa_decode; additionally
 * PA_ERR_SHAPE when num_q_tokens, num_seqs x tiles or Pmax exceeds 65535.
 * num_q_tokens == 0 or num_seqs == 0 enqueues nothing.
 */
size_t pa_multi_workspace_size(int32_t num_q_tokens, int32_t num_heads,
                               int32_t head_size, int32_t max_blocks_per_seq,
                               int32_t block_size, int32_t partition_size);
pa_status pa_decode_multi(void* out, const void* query, const void* key_cache,
                          const void* value_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq,
                          const int32_t* cu_seqlens_q, int32_t num_q_tokens,
                          int32_t max_q_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_size,
                          int32_t block_size, int32_t num_blocks, float scale,
                          int32_t partition_size, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Chunked prefill: pa_decode_multi's result (same rows, causal limits,
 * zeros and tolerance; no workspace) for chunks of many query rows per
 * sequence.  Each workgroup takes 128 of a sequence's rows x heads of one
 * kv head and walks the keys they see once, in tiles of 64 staged through
 * LDS, with the scores and the weighted sum of values on the matrix cores;
 * a key is read from memory once per 128 rows x heads instead of once per
 * 16 (pa_decode_multi's column tile).  Launch: num_kv_heads x
 * ceil(max_q_per_seq * g / 128) x num_seqs workgroups; workgroups past a
 * sequence's own rows exit at once.  Arguments, preconditions and errors
 * as pa_decode_multi without partition_size and the workspace;
 * PA_ERR_SHAPE when ceil(max_q_per_seq * g / 128) exceeds 65535 or
 * num_q_tokens * num_heads * head_size reaches 2^31.  Row j of
 * a T-row chunk sees keys 0 .. n - T + j; the rows need not be more than
 * one ([BOOK] §4.5 (1)-(2); the running-max recurrence of §4.6 per row).
 */
pa_status pa_prefill(void* out, const void* query, const void* key_cache,
                     const void* value_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                     int32_t num_q_tokens, int32_t max_q_per_seq,
                     const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_heads, int32_t num_kv_heads, int32_t head_size,
                     int32_t block_size, int32_t num_blocks, float scale,
                     hipStream_t stream);

/*
 * Multi-token queries on the balanced split: pa_decode_multi's result
 * (same rows, causal limits and tolerance) in ONE kernel, with the work of
 * every (sequence, kv head) pair cut into equal slices as for
 * pa_decode_balanced and cut pairs merged in-kernel.  Up to 16 of a
 * sequence's query rows x g heads share one pass over its keys (a column
 * tile); with max_q_per_seq * g > 16 (chunked prefill) each (sequence, kv
 * head) carries ceil(max_q_per_seq * g / 16) tiles, laid end to end in the
 * balanced split, and a sequence with T rows uses ceil(T * g / 16) of
 * them.  Rows of a sequence with context_lens <= 0, and rows placed before
 * the first key (T > n), get zeros.  Precondition: no sequence has more
 * than max_q_per_seq rows (rows past it are not computed).  Each tile reads
 * the pair's keys again; from two tiles up the two-kernel pa_decode_multi,
 * whose partitions the hardware dispatcher balances, measured faster.
 * pa_multi_balanced_grid: resident workgroups of this kernel for this
 *   max_q_per_seq, at most two per CU for the 4-column body (0 if
 *   unsupported or unknown); pass the same
 *   max_q_per_seq to pa_decode_multi_balanced, which picks the matrix-core
 *   body with 4 or 8 columns when max_q_per_seq * g fits them and its
 *   16-column form otherwise.
 * pa_multi_balanced_workspace_size: the same fixed counter header as
 *   pa_balanced_workspace_size, then fp32 max/sum [rows] and out [rows,
 *   head_size], rows = (grid + num_seqs * num_kv_heads) * 16 (0 when
 *   num_seqs * num_kv_heads exceeds PA_BALANCED_MAX_PAIRS).  Zero-fill once
 *   before the first call; each completed call leaves the counters zero, so
 *   the workspace serves later calls of any shape it is large enough for
 *   (a decode workspace of the same size may be shared with it); calls
 *   sharing a workspace must not overlap.  Sized for one column tile per
 *   (sequence, kv head), i.e. max_q_per_seq * g <= 16.
 * pa_multi_balanced_workspace_size_tiles: the same for any max_q_per_seq:
 *   rows = (grid + num_seqs * num_kv_heads * tiles) * 16 with tiles = 1
 *   when max_q_per_seq * g fits the 4 or 8 columns, else
 *   ceil(max_q_per_seq * g / 16); 0 when num_seqs * num_kv_heads * tiles
 *   exceeds PA_BALANCED_MAX_PAIRS.  pa_decode_multi_balanced requires this
 *   size (equal to pa_multi_balanced_workspace_size for one tile).
 * Other arguments as pa_decode_multi ([BOOK] §4.5 (2)).
 */
int32_t pa_multi_balanced_grid(int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_size, int32_t block_size,
                               int32_t max_q_per_seq);
size_t pa_multi_balanced_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                        int32_t head_size, int32_t grid);
size_t pa_multi_balanced_workspace_size_tiles(int32_t num_seqs, int32_t num_heads,
                                              int32_t num_kv_heads,
                                              int32_t head_size, int32_t grid,
                                              int32_t max_q_per_seq);
pa_status pa_decode_multi_balanced(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* cu_seqlens_q, int32_t num_q_tokens, int32_t max_q_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t grid, void* workspace,
    size_t workspace_bytes, hipStream_t stream);

/*
 * Shared-prefix decode: the same result as pa_decode_splitk +
 * pa_decode_reduce (same partitions, same reduce; within pa_decode's
 * tolerance of the exact attention), but a partition that lies inside the
 * full blocks a group of sequences shares is read once for the whole group.
 * [GUST] copy-on-write paragraph: many requests start with the same system
 * prompt or sampled continuations of one prompt, so their tables point at
 * the same physical blocks until one of them writes; [BOOK] §4.7.1 (the
 * samples of one prompt reference its blocks) and §4.7.2-4.7.3 (prefix caching
 * reuses full blocks only).
 *   group_offsets  int32 [num_groups + 1]: members of group j are
 *                  group_members[group_offsets[j] .. group_offsets[j+1]-1]
 *   group_members  int32: sequence indices (each sequence in at most one
 *                  group; indices outside [0, num_seqs) are ignored)
 *   group_blocks   int32 [num_groups]: leading logical blocks that every
 *                  member's block_tables row holds with the same physical
 *                  ids (precondition; the first member's row is read)
 *   max_group_size >= every group's member count, and max_group_blocks >=
 *                  every group_blocks entry (host values sizing the launch;
 *                  members or blocks beyond them are simply not shared)
 *   The shared partitions of group j are the first
 *   min(group_blocks[j], max_group_blocks) * block_size / partition_size
 *   (whole partitions only); every other partition is computed per
 *   sequence.  A member whose context ends inside a shared partition gets
 *   its own key limit.  Other arguments as pa_decode_splitk; out as
 *   pa_decode_reduce.  num_groups == 0 is plain split-K decode.
 * pa_prefix_workspace_size: bytes of workspace (16-byte aligned): the
 *   split-K workspace followed by int32 [num_seqs].  No zero-fill needed.
 */
size_t pa_prefix_workspace_size(int32_t num_seqs, int32_t num_heads,
                                int32_t head_size, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t partition_size);
pa_status pa_decode_shared_prefix(
    void* out, const void* query, const void* key_cache, const void* value_cache,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t partition_size,
    const int32_t* group_offsets, const int32_t* group_members,
    const int32_t* group_blocks, int32_t num_groups, int32_t max_group_size,
    int32_t max_group_blocks, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * FP8 KV cache: a pool that stores one byte per element instead of two
 * ([BOOK] §4.8 names a lower-precision KV cache as a way to fit more
 * concurrent tokens in the same memory; [CSDN] part 3 (2), the KVBlock
 * field table, lists FP16/FP8 block storage).  Layout as the fp16 pool
 * with 1-byte elements: each half is [num_blocks, block_size, num_kv_heads,
 * head_size] uint8, 16-byte aligned.  Each byte is an OCP FP8 E4M3 code
 * (e4m3fn: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, 0x7f / 0xff NaN, largest finite 448).  The stored value of a
 * code c is decode(c) * k_scale for K and decode(c) * v_scale for V, with
 * one scale per tensor (per layer) chosen by the caller.  pa_copy_blocks and
 * pa_swap_blocks move bytes, so they serve an fp8 pool given as an fp16 one
 * with head_size / 2 (head_size / 2 must be a multiple of 8).
 *
 * pa_cache_write_fp8: as pa_cache_write, into an fp8 pool.  Element x
 *   becomes the code nearest (ties to even) to clamp(float(x) * (1 / s),
 *   -448, 448) where s = k_scale or v_scale and 1 / s is rounded to fp32
 *   once on the host; NaN inputs give a NaN code.  Scales must be finite
 *   and > 0 (else PA_ERR_SHAPE).
 * pa_balanced_grid_fp8 / pa_decode_balanced_fp8: as pa_balanced_grid /
 *   pa_decode_balanced over an fp8 pool (same workspace size and rules,
 *   query and output fp16).  The result is attention over the dequantised
 *   K and V (codes times their scales), within the fp16 path's tolerance
 *   of that.  Scales as above.
 * pa_decode_step_fp8: pa_decode_step over an fp8 pool: each sequence's new
 *   K/V row (fp16) is quantised exactly as pa_cache_write_fp8 does, stored
 *   into its slot, and attended to in that quantised form, in one kernel;
 *   the same as pa_slot_mapping + pa_cache_write_fp8 +
 *   pa_decode_balanced_fp8.  Grid from pa_balanced_grid_fp8.
 */
pa_status pa_cache_write_fp8(const void* key, const void* value,
                             void* key_cache, void* value_cache,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             int32_t num_blocks, int32_t block_size,
                             int32_t num_kv_heads, int32_t head_size,
                             float k_scale, float v_scale, hipStream_t stream);
int32_t pa_balanced_grid_fp8(int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_size, int32_t block_size);
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
                             size_t workspace_bytes, hipStream_t stream);
pa_status pa_decode_balanced_fp8(void* out, const void* query,
                                 const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables,
                                 int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_size, int32_t block_size,
                                 int32_t num_blocks, float scale, float k_scale,
                                 float v_scale, int32_t grid, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode_step -- one whole decode step in one kernel: for every
 * sequence i the token at position p = context_lens[i] - 1 is appended and
 * then attended to, exactly as pa_slot_mapping + pa_cache_write +
 * pa_decode_balanced would ([BOOK] §4.5: write this step's K/V by slot,
 * then read the history by block table).
 *   key, value    fp16 [num_seqs, num_kv_heads, head_size]: this step's
 *                 K/V rows, copied bit-exactly to slot
 *                 block_tables[i, p / block_size] * block_size +
 *                 p % block_size of key_cache / value_cache (skipped if that
 *                 block id is outside [0, num_blocks)).
 *   slot_mapping  int32 [num_seqs] output, or NULL: the slot written per
 *                 sequence (-1 where skipped or context_lens[i] <= 0).
 *   Other arguments as pa_decode_balanced (same workspace rules).
 *   Preconditions of pa_decode and pa_cache_write; sequences with
 *   context_lens[i] <= 0 append nothing and get zeros.
 */
pa_status pa_decode_step(void* out, const void* query, const void* key,
                         const void* value, void* key_cache, void* value_cache,
                         int32_t* slot_mapping, const int32_t* block_tables,
                         int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_size, int32_t block_size,
                         int32_t num_blocks, float scale, int32_t grid,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * pa_decode_step_noalloc -- pa_decode_step for callers that cannot allocate
 *   device memory: code under HIP graph capture, tight serving loops and
 *   harnesses that forbid hipMalloc.  The same arguments and result as
 *   pa_decode_step (same kernel, same grid from pa_balanced_grid), without
 *   the workspace: the range counters and partial states live in a static
 *   device array of PA_NOALLOC_SCRATCH_BYTES that the library holds on each
 *   device it runs on until the process ends.  The call allocates nothing
 *   (no hipMalloc, no library allocation); the caller still passes inputs
 *   and outputs.
 *   Limits: at most PA_NOALLOC_MAX_PAIRS (sequence, kv head) pairs, and
 *   (grid + num_seqs * num_kv_heads) * group * (head_size + 2) * 4 bytes of
 *   partial states at most PA_NOALLOC_SCRATCH_BYTES - 4 *
 *   PA_NOALLOC_MAX_PAIRS; larger shapes return PA_ERR_WORKSPACE before
 *   anything is enqueued.  fp16 pools only.
 *   The first call on a device clears the array's counters and waits for
 *   that on `stream`, so it must not be made during graph capture; later
 *   calls only enqueue.  Every call on a device shares that device's array
 *   and leaves its counters zero: calls that overlap on one device (other
 *   streams, other host threads) race and give wrong results.
 */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
#define PA_NOALLOC_MAX_PAIRS (1 << 16)
pa_status pa_decode_step_noalloc(
    void* out, const void* query, const void* key, const void* value,
    void* key_cache, void* value_cache, int32_t* slot_mapping,
    const int32_t* block_tables, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
    int32_t num_kv_heads, int32_t head_size, int32_t block_size,
    int32_t num_blocks, float scale, int32_t grid, hipStream_t stream);

/*
 * pa_stream_read -- measurement probe, not part of the method: one plain
 *   sequential read of `bytes` bytes at `buf` with 16-byte non-temporal
 *   loads.  Its rate is the device's streaming-read ceiling, against which a
 *   decode's KV read rate is compared beside the nominal HBM peak (a
 *   bandwidth-bound path such as [BOOK] §4.1.2 describes).
 *   buf   device, 16-byte aligned, bytes > 0 and a multiple of 16; read only
 *   sink  device uint32 [grid * 4]: each wave stores the xor of what it read
 *         (so the loads cannot be elided); contents otherwise meaningless
 *   grid  workgroups of 256 threads, 1 .. 65535 (a few per CU saturates HBM)
 *   Errors: PA_ERR_NULL, PA_ERR_SHAPE (bytes 0 or grid out of range),
 *   PA_ERR_ALIGN, PA_ERR_HIP.
 */
pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                         int32_t grid, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PA_H */
