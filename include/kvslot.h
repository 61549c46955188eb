/*
 * kvslot.h - C ABI of the Block KV decode hot path for AMD Instinct MI355X
 * (gfx950): slot mapping, the paged KV-cache write, GQA paged decode
 * attention and per-step context-length bucket selection.
 *
 * Pages cited (by title):
 *   [BKV] "Padding and Batching with Block KV" (AWS Neuron vllm-neuron docs)
 *   [BT]  "Block table: logical token -> physical KV block" (vLLM v0.25.1 notes)
 *   [CLB] "Decode Context-Length Bucketing" (AWS Neuron vllm-neuron docs)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Cache layout ([BKV] "Block Structure"): each of k_cache and v_cache is a
 *   dense row-major array [total_blocks][block_size][num_kv_heads][head_dim]
 *   of the cache element type. A slot s = block * block_size + offset names
 *   one [num_kv_heads][head_dim] row.
 * - Block table ([BKV] "Block Table"): int32 [rows][table_stride], row =
 *   request, column j = physical block of logical block j. An entry <= 0 is
 *   inactive: 0 is the null block, -1 the sentinel ([BKV] "Block ID 0 vs.
 *   Sentinel -1"); both behave identically in every entry point.
 * - Pointers of the GPU entry points are device pointers; each of those
 *   entry points only enqueues kernels on `stream` (a hipStream_t; NULL is
 *   the null stream) and returns. No entry point synchronises, reads device
 *   memory on the host, or allocates or frees memory. The caller owns every
 *   buffer.
 * - Alignment: arrays of cache elements and of fp32 results (q, k_cache,
 *   v_cache, k_new, v_new, out, outs and the decode workspace) must be
 *   16-byte aligned, int32 and int64 arrays naturally aligned; otherwise
 *   the entry point returns KVS_EINVAL. (Rows of the supported shapes are
 *   multiples of 16 bytes, so whole-row offsets keep the alignment.)
 * - Only scalar arguments and pointers are checked. A bad value inside a
 *   device array (a block id, a slot, a length) is a caller error: the
 *   kernels clamp their reads to the given sizes and skip what is out of
 *   range, so such a value never faults, but the result is unspecified.
 * - Return values: KVS_OK (0) or a negative KVS_E* status; nothing is
 *   enqueued when the status is not KVS_OK, except for KVS_EHIP, which
 *   reports a failed launch.
 */
#ifndef KVSLOT_H
#define KVSLOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVS_OK 0
#define KVS_EINVAL (-1)       /* null or misaligned pointer, bad size/scalar  */
#define KVS_EUNSUPPORTED (-2) /* dtype, head_dim, block_size or shape          */
#define KVS_EBUCKET (-3)      /* bucket list fails the [CLB] validation rules  */
#define KVS_ERANGE (-4)       /* needed_seq beyond max_model_len               */
#define KVS_ENOSPACE (-5)     /* workspace smaller than required               */
#define KVS_EHIP (-6)         /* a kernel launch failed (hipGetLastError)      */

/* Element type of caches, new K/V rows and q. The two range markers are not
 * dtypes: they make every int32 value a valid value of the type in C and C++
 * alike, so a caller passing some other number gets KVS_EUNSUPPORTED rather
 * than undefined behaviour. */
typedef enum {
  KVS_F32 = 0,
  KVS_BF16 = 1,
  KVS_DTYPE_RANGE_LO_ = -0x7fffffff - 1,
  KVS_DTYPE_RANGE_HI_ = 0x7fffffff
} kvs_dtype;

/* paged_decode_attention flag: walk every one of the first walk_blocks table
 * columns of every row, as a fixed-shape kernel does; inactive entries read
 * null block 0. The output is identical to the default context walk, which
 * reads only the blocks that cover each request's context. This mode exists
 * to measure the traffic of a fixed-shape step ([CLB] "Problem"). */
#define KVS_WALK_TABLE 0x1u

/* Short English text for a status code (static storage). */
const char* kvs_status_string(int status);

/*
 * kv_slot_mapping - slot of every token ([BKV] "The Core Formula" and "Slot
 * Mapping Computation"; tail padding as in the [BT] data-flow listing).
 *
 * For t < num_tokens, with r = req_indices[t] and p = positions[t]:
 *   slot_mapping[t] = block_table[r * table_stride + p / block_size]
 *                     * block_size + p % block_size
 * and slot_mapping[t] = -1 instead when r < 0 (a padding token, [BKV] "Slot
 * Mapping for Padded Tokens"), r >= table_rows, p < 0, p / block_size >=
 * table_stride, or the table entry is <= 0 (null block or sentinel). For
 * num_tokens <= t < max_num_tokens, slot_mapping[t] = -1.
 *
 *   req_indices   int32 [num_tokens], device
 *   positions     int64 [num_tokens], device
 *   block_table   int32 [table_rows][table_stride], device
 *   slot_mapping  int64 [max_num_tokens], device, written
 * Errors: KVS_EINVAL for null pointers (when the matching size is > 0),
 * num_tokens < 0, max_num_tokens < num_tokens, table_rows < 0,
 * table_stride < 1 or block_size < 1.
 */
int kv_slot_mapping(const int32_t* req_indices, const int64_t* positions, int64_t num_tokens,
                    int64_t max_num_tokens, const int32_t* block_table, int32_t table_rows,
                    int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                    void* stream);

/*
 * kv_cache_write - scatter new K/V rows into the paged caches ([BKV] "Slot
 * ID -1: Padding Tokens": the write to K_cache[slot_ids] skips
 * out-of-bounds slots).
 *
 * For every t < num_tokens with 0 <= s = slot_mapping[t] < total_blocks *
 * block_size, copies row t of k_new (num_kv_heads * head_dim elements) to
 * slot s of k_cache, and the same for v_new / v_cache. Other tokens write
 * nothing. The copy is of raw elements, so the cache receives the exact
 * bytes of k_new / v_new.
 *
 *   k_new, v_new      [num_tokens][num_kv_heads][head_dim] of dtype, device
 *   slot_mapping      int64 [num_tokens], device
 *   k_cache, v_cache  cache layout above, device, updated in place
 * Two tokens with one slot is a caller error (which row lands is
 * unspecified). k_new / v_new must not overlap the caches.
 * Errors: KVS_EINVAL (null pointers, negative sizes, num_kv_heads < 1,
 * block_size < 1, total_blocks < 1); KVS_EUNSUPPORTED when a row is not a
 * multiple of 16 bytes or dtype is unknown.
 */
int kv_cache_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   int64_t num_tokens, void* k_cache, void* v_cache, int64_t total_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim, kvs_dtype dtype,
                   void* stream);

/*
 * kv_slot_mapping_cache_write - kv_slot_mapping and kv_cache_write in one
 * launch ([BKV] "The Core Formula" and "Slot ID -1: Padding Tokens": the
 * cache write consumes the slot ids as they are computed).
 *
 * Writes slot_mapping exactly as kv_slot_mapping does with the same first
 * nine arguments, and updates the caches exactly as kv_cache_write does
 * with those slots, k_new, v_new, total_blocks, block_size, num_kv_heads,
 * head_dim and dtype: the same bytes land in the same places, and
 * slot_mapping is also the caller's for later use.
 *
 *   req_indices, positions, block_table, slot_mapping   as kv_slot_mapping
 *   k_new, v_new      [num_tokens][num_kv_heads][head_dim] of dtype, device
 *   k_cache, v_cache  cache layout above, device, updated in place
 * Two tokens with one slot is a caller error (which row lands is
 * unspecified). k_new / v_new must not overlap the caches or slot_mapping.
 * Errors: KVS_EINVAL for null pointers (when the matching size is > 0) and
 * every size kv_slot_mapping or kv_cache_write rejects; KVS_EUNSUPPORTED
 * when a row is not a multiple of 16 bytes or dtype is unknown.
 */
int kv_slot_mapping_cache_write(const int32_t* req_indices, const int64_t* positions,
                                int64_t num_tokens, int64_t max_num_tokens,
                                const int32_t* block_table, int32_t table_rows,
                                int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, int64_t total_blocks, int32_t num_kv_heads,
                                int32_t head_dim, kvs_dtype dtype, void* stream);

/*
 * select_ctx_bucket - per-step decode context bucket ([CLB] "Per-step
 * bucket selection", "Validation", "Block-table head-trim vs. SWA
 * tail-trim", "Backwards compatibility"). Host only; pointers are host
 * pointers; no GPU work.
 *
 * buckets == NULL means the feature is off: returns max_model_len and
 * ceil(max_model_len / block_size). Otherwise the list must be non-empty,
 * positive, strictly ascending, each value below max_model_len and
 * divisible by 128 (else KVS_EBUCKET); needed_seq = max_num_computed_tokens
 * + 1 + num_speculative_tokens must not exceed max_model_len (else
 * KVS_ERANGE); the result is the smallest bucket >= needed_seq among the
 * list and max_model_len, and walk_blocks = ceil(bucket / block_size), the
 * table columns a head-trimmed step keeps.
 * Errors: KVS_EINVAL for null outputs, num_buckets < 0, negative
 * max_num_computed_tokens or num_speculative_tokens, max_model_len < 1 or
 * block_size < 1.
 */
int select_ctx_bucket(int64_t max_num_computed_tokens, int32_t num_speculative_tokens,
                      const int32_t* buckets, int32_t num_buckets, int32_t max_model_len,
                      int32_t block_size, int32_t* bucket_len_out, int32_t* walk_blocks_out);

/*
 * kv_map_to_kernel_blocks - expand a block table from manager blocks to
 * kernel blocks ([BT] design motivation: one manager block becomes
 * manager_block_size / kernel_block_size kernel blocks; a kernel size that
 * does not divide the manager size is rejected). Host only.
 *
 * With k = manager_block_size / kernel_block_size, entry m of column c
 * becomes entries m * k + i at columns c * k + i (i < k) when m > 0; an
 * inactive entry (<= 0) is copied to all k columns. This is the layout a
 * [N][manager_bs][H][D] pool has when viewed as [N * k][kernel_bs][H][D].
 *
 *   src  int32 [rows][src_stride], host
 *   dst  int32 [rows][dst_stride], host, dst_stride >= src_stride * k
 * Errors: KVS_EINVAL (null pointers, rows < 0, bad strides or sizes,
 * kernel_block_size not dividing manager_block_size, or an expanded id that
 * does not fit int32).
 */
int kv_map_to_kernel_blocks(const int32_t* src, int32_t rows, int32_t src_stride,
                            int32_t manager_block_size, int32_t kernel_block_size, int32_t* dst,
                            int32_t dst_stride);

/*
 * select_batch_bucket - padded batch size of a decode step ([BKV] "Decode
 * Batch Padding": the scheduler takes the smallest configured
 * num_seqs_buckets entry that fits the active requests; the rows past them
 * are dummy requests: request index -1 and position 0 for their tokens, so
 * their slots are -1 and nothing is written, and seq_len 0 with null-block
 * table rows, so decode attention reads nothing for them and writes zeros).
 * Host only; pointers are host pointers.
 *
 * Writes the smallest buckets[i] >= num_active.
 * Errors: KVS_EINVAL for a null padded_out or negative counts; KVS_EBUCKET
 * for an empty, non-positive or not strictly ascending list; KVS_ERANGE
 * when num_active exceeds the largest bucket.
 */
int select_batch_bucket(int32_t num_active, const int32_t* buckets, int32_t num_buckets,
                        int32_t* padded_out);

/*
 * paged_decode_attention_workspace_bytes - bytes of device workspace a
 * paged_decode_attention call with these sizes needs. Depends on these
 * arguments only (not on context lengths or walk_blocks), so one workspace
 * serves every bucket. Returns 0 for invalid sizes.
 */
size_t paged_decode_attention_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim);

/*
 * paged_decode_attention - GQA decode attention over the paged cache
 * ([BKV] "Cache Masking", "Block ID 0 vs. Sentinel -1", "Multi-Token
 * Decode"; [CLB] "Problem" and "Block-table head-trim vs. SWA tail-trim").
 *
 * Request r has context length L = seq_lens[r], which counts the q_len
 * tokens of this step (already written to the cache). Query token j of
 * request r sits at position L - q_len + j; q head h reads KV head
 * h / (num_q_heads / num_kv_heads). It attends to every position p with
 * p <= its own position and p < walk_blocks * block_size whose table entry
 * block_table[r * table_stride + p / block_size] is active (> 0 and <
 * total_blocks): key K = k_cache[block][p % block_size][kv_head], value
 * likewise, score = scale * <q, K>, output = softmax-weighted sum of the
 * values, accumulated in fp32. A request with L <= 0 (a padded row) and a
 * query that sees no key produce zeros.
 *
 *   q            [num_seqs][q_len][num_q_heads][head_dim] of dtype, device
 *   k_cache, v_cache   cache layout above, dtype, device
 *   block_table  int32 [num_seqs][table_stride], device; walk_blocks <=
 *                table_stride columns of it are read (the head trim)
 *   seq_lens     int32 [num_seqs], device
 *   out          float [num_seqs][q_len][num_q_heads][head_dim], device
 *   workspace    device memory of at least
 *                paged_decode_attention_workspace_bytes(...) bytes, scratch
 *                for the split-K partials; no initial contents are needed.
 *                Calls that run concurrently must not share a workspace.
 *   flags        0 (context walk: only blocks covering each request's
 *                context are read) or KVS_WALK_TABLE.
 * By default only the blocks covering min(L, walk_blocks * block_size)
 * positions are read. Results do not depend on walk_blocks beyond that
 * trim, on the flags, on the physical block ids, or on whether unused
 * entries hold 0 or -1: on one device they are bitwise identical across
 * those. (How the batch is split over the device's compute units follows
 * from the context lengths and the device's unit count, and the split
 * decides the fp32 summation order.)
 * Supported: head_dim 64 or 128; block_size 16, 32, 64, 128 or 256;
 * (num_q_heads / num_kv_heads) * q_len <= 64; num_seqs <= 8192;
 * num_seqs * (walk_blocks * block_size / 16 + 1) <= 2^30 - 1.
 * Errors: KVS_EINVAL (null pointers, non-positive sizes, num_q_heads not a
 * multiple of num_kv_heads, walk_blocks outside [0, table_stride]),
 * KVS_EUNSUPPORTED (outside the supported set), KVS_ENOSPACE (workspace
 * too small), KVS_EHIP.
 */
int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int32_t table_stride, int32_t walk_blocks,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t q_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t total_blocks, float scale,
                           kvs_dtype dtype, uint32_t flags, void* workspace,
                           size_t workspace_bytes, float* out, void* stream);

/*
 * paged_decode_attention_noalloc - paged_decode_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same arguments and results
 * without the workspace: the split-K partials go to a device array the
 * library owns, KVS_NOALLOC_WORKSPACE_BYTES on each GPU it runs on, held
 * from the loading of the library's code object until the process ends.
 * The call allocates and frees nothing; its first call on a device looks
 * the array's address up (hipGetSymbolAddress) with that device current.
 *
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's contents (no call needs it cleared). Calls that overlap on
 * one GPU (two streams, two threads) race on it and their results are
 * unspecified: the caller orders them, e.g. on one stream.
 *
 * On one device the output is bitwise that of paged_decode_attention with
 * the same arguments (the same kernels and launch). The call needs
 * 256-rounded 8 * num_seqs bytes plus (S + num_seqs) partial slots of
 * num_q_heads * q_len * (head_dim + 4) * 4 bytes, S being the number of
 * slices the launch cuts the batch into (at most the device's resident
 * pass-1 workgroups per head group: 64 on MI355X at 8 KV heads of bf16, two
 * heads per workgroup); a call that needs more than
 * KVS_NOALLOC_WORKSPACE_BYTES returns KVS_ENOSPACE before anything is
 * enqueued (the 256-request, 64-query-head batch needs about 11 MB).
 * Errors: those of paged_decode_attention, KVS_ENOSPACE as above, KVS_EHIP
 * when the array's address cannot be obtained.
 */
#define KVS_NOALLOC_WORKSPACE_BYTES ((size_t)64 << 20)

int paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t table_stride,
                                   int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t total_blocks,
                                   float scale, kvs_dtype dtype, uint32_t flags, float* out,
                                   void* stream);

/*
 * paged_decode_attention_append - the step's cache write and the decode
 * attention in one call: the result is that of kv_slot_mapping_cache_write
 * (with table_rows = num_seqs: the step's tokens index the batch's rows)
 * followed by paged_decode_attention with the same arguments, for the
 * callers that hold both ([BKV] "Slot Mapping Computation" and "Slot ID -1"
 * for the write, the passages cited above for the attention).
 *
 * Step tokens, as in kv_slot_mapping_cache_write: req_indices, positions
 * [num_tokens]; slot_mapping [max_num_tokens] (written, -1 tail); k_new,
 * v_new [num_tokens][num_kv_heads][head_dim] of dtype. Attention arguments
 * as in paged_decode_attention; k_cache and v_cache are written and read.
 *
 * When max_num_tokens <= 64 * NW, NW the largest of 8, 4, 2 and 1 that
 * divides num_kv_heads (the KV heads one workgroup holds: 512 tokens at 8
 * KV heads), and flags is 0, the decode launch writes the rows itself: each
 * row is written by the workgroup that reads it, so one launch fewer. This needs what a decode step guarantees: a written
 * slot lies in a block that no other request of the batch reads in this
 * call (the request's own tail block); otherwise the result is
 * unspecified. Larger steps, and the fixed-shape walk, take the fused
 * slot-map + write launch first; the result is the same.
 * Errors: those of both calls.
 */
int paged_decode_attention_append(const int32_t* req_indices, const int64_t* positions,
                                  int64_t num_tokens, int64_t max_num_tokens,
                                  int64_t* slot_mapping, const void* k_new, const void* v_new,
                                  const void* q, void* k_cache, void* v_cache,
                                  const int32_t* block_table, int32_t table_stride,
                                  int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t total_blocks,
                                  float scale, kvs_dtype dtype, uint32_t flags, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream);


/*
 * paged_decode_attention_swa - decode attention for a sliding-window layer
 * over a tail-trimmed block table ([KVC] "Attention Type": a sliding-window
 * layer keeps only the recent tokens within its window; [CLB] "Block-table
 * head-trim vs. SWA tail-trim": the trimmed table keeps a request's last
 * blocks and swa_kv_pos_offset gives the position of its first one, so
 * positions stay absolute).
 *
 * As paged_decode_attention (flags 0), except that:
 *   - column c of request r's table row holds the block of absolute
 *     positions kv_pos_offset[r] + c * block_size onward, and only positions
 *     kv_pos_offset[r] .. kv_pos_offset[r] + walk_blocks * block_size - 1
 *     are visible;
 *   - with sliding_window > 0, the query at position qpos sees only keys at
 *     positions qpos - sliding_window + 1 .. qpos (the window counts the
 *     query's own position); 0 means no window.
 * Only the blocks those keys sit in are read.
 *
 *   kv_pos_offset  int32 [num_seqs], device, each >= 0 and a multiple of
 *                  block_size (kv_swa_tail_trim writes them); NULL means 0
 *                  for every request (a whole table with a window)
 * On one device the output does not depend on whether the table is whole
 * (offsets 0) or trimmed, as long as the trim keeps every block a window of
 * the step touches: the two are bitwise identical.
 * Errors: as paged_decode_attention, and KVS_EINVAL for sliding_window < 0.
 */
int paged_decode_attention_swa(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t table_stride,
                               int32_t walk_blocks, const int32_t* seq_lens,
                               const int32_t* kv_pos_offset, int32_t sliding_window,
                               int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t total_blocks, float scale, kvs_dtype dtype,
                               void* workspace, size_t workspace_bytes, float* out,
                               void* stream);

/*
 * kv_swa_tail_trim - tail-trim a block table for a sliding-window layer
 * ([CLB] "Block-table head-trim vs. SWA tail-trim"). Host only; every
 * pointer is a host pointer; no GPU work.
 *
 * width = min(src_stride, ceil((sliding_window + q_len - 1) / block_size)
 * + 1): the blocks the windows of a step's q_len queries can touch at any
 * alignment (the page's window / block_size assumes one query and an
 * aligned window). Row r keeps the width columns ending at its last
 * context block (seq_lens[r] - 1) / block_size, starting no earlier than
 * column 0: dst[r][c] = src[r][first + c], -1 past the source width, and
 * kv_pos_offset[r] = first * block_size. A row with seq_lens[r] <= 0 keeps
 * columns from 0.
 *
 *   src            int32 [rows][src_stride]
 *   seq_lens       int32 [rows]
 *   dst            int32 [rows][dst_stride], dst_stride >= width, written
 *   kv_pos_offset  int32 [rows], written
 *   width_out      written with width (also on KVS_EINVAL for a short dst)
 * Errors: KVS_EINVAL for null pointers, rows < 0, src_stride < 1,
 * q_len < 1, sliding_window < 1, block_size < 1, dst_stride < width, or an
 * offset beyond int32.
 */
int kv_swa_tail_trim(const int32_t* src, int32_t rows, int32_t src_stride,
                     const int32_t* seq_lens, int32_t q_len, int32_t sliding_window,
                     int32_t block_size, int32_t* dst, int32_t dst_stride, int32_t* kv_pos_offset,
                     int32_t* width_out);

/*
 * Decode context parallelism, one rank's part ("Block table: logical token
 * -> physical KV block", design motivation: with TOTAL_CP_WORLD_SIZE,
 * TOTAL_CP_RANK and CP_KV_CACHE_INTERLEAVE_SIZE the slot kernel writes a
 * real slot only for the tokens its rank stores and PAD_ID for the others).
 * The page prints no formula; the reading here: runs of cp_interleave
 * consecutive positions go round-robin to the cp_world_size ranks (rank of
 * position p: (p / cp_interleave) % cp_world_size), and each rank packs
 * its runs densely, so position p lives in its rank's cache at local
 * position lp = (p / (cp_world_size * cp_interleave)) * cp_interleave +
 * p % cp_interleave. lp / block_size = p / (cp_world_size * block_size): the
 * ranks share one table row, a column standing for cp_world_size *
 * block_size consecutive positions of which each rank stores block_size.
 * cp_interleave is a power of two dividing block_size.
 */

/*
 * kv_slot_mapping_dcp - kv_slot_mapping on rank cp_rank: a token this rank
 * stores gets table[r][lp / block_size] * block_size + lp % block_size
 * (with every -1 rule of kv_slot_mapping), every other token -1, and the
 * tail of the buffer -1. The cache write is then kv_cache_write.
 * Errors: as kv_slot_mapping; KVS_EINVAL also for cp_world_size < 1,
 * cp_rank outside [0, cp_world_size), a block_size that is not a power of
 * two, or a cp_interleave that is not a power of two dividing block_size.
 */
int kv_slot_mapping_dcp(const int32_t* req_indices, const int64_t* positions, int64_t num_tokens,
                        int64_t max_num_tokens, const int32_t* block_table, int32_t table_rows,
                        int32_t table_stride, int32_t block_size, int32_t cp_world_size,
                        int32_t cp_rank, int32_t cp_interleave, int64_t* slot_mapping,
                        void* stream);

/*
 * paged_decode_attention_dcp - one rank's decode attention over the keys it
 * stores: the positions p < seq_lens[r] (and below walk_blocks *
 * cp_world_size * block_size) that rank cp_rank owns, read from this
 * rank's caches at their local positions. Queries keep their global
 * positions (L - q_len + j) and the causal rule. Writes out, normalised
 * over this rank's keys, and lse[r][j][h], the natural-log sum of
 * exp(scale * <q, k>) over them (-inf, with zero output, for a row that
 * sees none of this rank's keys): the partial state the ranks exchange and
 * decode_lse_merge combines.
 *
 *   lse  float [num_seqs][q_len][num_q_heads], device, written
 * Other arguments, the workspace contract and the supported shapes: as
 * paged_decode_attention (context walk).
 * Errors: as paged_decode_attention; KVS_EINVAL also for a null lse and
 * the cp_* rules of kv_slot_mapping_dcp.
 */
int paged_decode_attention_dcp(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t table_stride,
                               int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t total_blocks,
                               float scale, kvs_dtype dtype, int32_t cp_world_size,
                               int32_t cp_rank, int32_t cp_interleave, void* workspace,
                               size_t workspace_bytes, float* out, float* lse, void* stream);

/*
 * decode_lse_merge - combine the ranks' (out, lse) partial states into the
 * attention over all their keys: out = sum_k exp(lse_k - lse) out_k with
 * lse = log sum_k exp(lse_k); ranks with lse_k = -inf contribute nothing; a
 * row no rank saw stays zero with lse -inf.
 *
 *   outs  float [world][rows][head_dim], device (rows = requests * q_len * heads)
 *   lses  float [world][rows], device
 *   out   float [rows][head_dim], device, written
 *   lse   float [rows], device, written; may be NULL
 * Errors: KVS_EINVAL for world < 1, rows < 0, head_dim not a positive
 * multiple of 4, or null pointers when rows > 0.
 */
int decode_lse_merge(const float* outs, const float* lses, int32_t world, int64_t rows,
                     int32_t head_dim, float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSLOT_H */
