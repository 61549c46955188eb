// Internal launch interface between the C-ABI layer (abi.cpp) and the HIP
// kernels. Not installed; the public interface is include/kvslot.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

hipError_t launch_slot_mapping(const int32_t* req_indices, const int64_t* positions,
                               int64_t num_tokens, int64_t max_num_tokens,
                               const int32_t* block_table, int32_t table_rows,
                               int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                               hipStream_t stream);

hipError_t launch_cache_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                              int64_t num_tokens, void* k_cache, void* v_cache,
                              int64_t total_slots, int32_t row_bytes, hipStream_t stream);

hipError_t launch_slot_mapping_dcp(const int32_t* req_indices, const int64_t* positions,
                                   int64_t num_tokens, int64_t max_num_tokens,
                                   const int32_t* block_table, int32_t table_rows,
                                   int32_t table_stride, int32_t block_size, int32_t world,
                                   int32_t rank, int32_t interleave, int64_t* slot_mapping,
                                   hipStream_t stream);

hipError_t launch_lse_merge(const float* outs, const float* lses, int32_t world, int64_t rows,
                            int32_t head_dim, float* out, float* lse, hipStream_t stream);

hipError_t launch_slot_write(const int32_t* req_indices, const int64_t* positions,
                             int64_t num_tokens, int64_t max_num_tokens,
                             const int32_t* block_table, int32_t table_rows,
                             int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             int64_t total_slots, int32_t row_bytes, hipStream_t stream);

// Everything the decode kernel needs; filled and checked by abi.cpp.
struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* kv_pos_offset;  // per request, position of table column 0; null: 0
  float* out;
  float* lse_out;  // optional [num_seqs][q_len][num_q_heads]: natural-log sum of exp(scores)
  float* partials;      // [slots][num_kv_heads][rows][head_dim + 4]
  int32_t* chunk_meta;  // [num_seqs][2]: first partial slot and partial count
  int64_t total_blocks;
  int32_t table_stride;
  int32_t walk_blocks;
  int32_t num_seqs;
  int32_t q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t window;  // sliding window in positions; 0: none
  int32_t cp_world, cp_rank, cp_ishift;  // context parallelism (1, 0, 0: none)
  int32_t max_slices;  // partial storage bound on the slices (per head group)
  int32_t slices;      // set by the launcher: slices the batch's tiles are cut into
  int32_t min_tiles;   // never cut a slice shorter than this many 16-token tiles
  int32_t start_tiles;  // units a request start counts for when cutting slices
  // The step's new tokens, written by pass 1 itself (paged_decode_attention
  // with an append): as kv_slot_mapping_cache_write with table_rows =
  // num_seqs. app_max_tokens = 0: no append.
  const int32_t* app_req;
  const int64_t* app_pos;
  const void* app_k;
  const void* app_v;
  void* app_k_cache;
  void* app_v_cache;
  int64_t* app_slots;
  int64_t app_tokens, app_max_tokens;
  float scale_log2;          // softmax scale times log2(e)
  uint32_t flags;
  int is_bf16;
};

// Largest batch the decode kernels take (their LDS holds one int per request).
constexpr int32_t kDecodeMaxSeqs = 8192;

// Workspace layout shared by the size query and the launch:
// [chunk_meta, rounded up to 256 bytes][partials].
size_t decode_meta_bytes(int32_t num_seqs);
int32_t decode_max_slices(int32_t num_kv_heads);
size_t decode_partial_bytes(int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim);
// Bytes of one partial slot (every KV head's rows of one (slice, request)).
size_t decode_partial_slot_bytes(int32_t q_len, int32_t num_q_heads, int32_t head_dim);
// Dynamic LDS of the pass-1 kernel: the batch's tile prefix.
size_t decode_lds_bytes(int32_t num_seqs);
// Slices a launch with these parameters cuts the batch into on the current
// device (the launch uses partial slots below slices + num_seqs).
hipError_t decode_slices(const DecodeParams& p, int* slices);

hipError_t launch_paged_decode(const DecodeParams& p, hipStream_t stream);

// The library's own device workspace for the entry point that allocates
// nothing: kNoallocScratchBytes on each device, shared by every such call
// on that device. Returns its address on the current device.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace kvs
