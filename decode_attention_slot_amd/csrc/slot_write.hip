// Slot mapping and paged KV-cache write in one launch.
//
// "Padding and Batching with Block KV", sections "The Core Formula" and "Slot
// ID -1: Padding Tokens": the write scatters each new K (V) row to the slot
// the slot formula gives and skips pad and out-of-bounds slots. The NKI
// write consumes the slot ids as they are computed; here too each thread
// computes its token's slot in registers, one thread per token stores it to
// slot_mapping, and every thread copies one 16-byte piece of the token's K
// row and of its V row to that slot. The result is, bit for bit, that of
// kv_slot_mapping followed by kv_cache_write, with one launch instead of two
// and no re-read of the slots.
#include "kvslot_internal.h"
#include "slot_formula.h"

namespace kvs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
slot_write_kernel(const int32_t* __restrict__ req_indices, const int64_t* __restrict__ positions,
                  int64_t num_tokens, int64_t max_num_tokens,
                  const int32_t* __restrict__ block_table, int32_t table_rows,
                  int32_t table_stride, int32_t block_size, int32_t block_shift,
                  int64_t* __restrict__ slot_mapping, const u32x4* __restrict__ k_new,
                  const u32x4* __restrict__ v_new, u32x4* __restrict__ k_cache,
                  u32x4* __restrict__ v_cache, int64_t total_slots, uint32_t pieces_per_row) {
  const int64_t copies = num_tokens * (int64_t)pieces_per_row;
  const int64_t n = copies + (max_num_tokens - num_tokens);  // then the -1 tail
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (i >= copies) {
      slot_mapping[num_tokens + (i - copies)] = -1;
      continue;
    }
    const int64_t t = i / pieces_per_row;
    const int64_t piece = i - t * pieces_per_row;
    const int64_t s = token_slot(req_indices[t], positions[t], block_table, table_rows,
                                 table_stride, block_size, block_shift);
    if (piece == 0) slot_mapping[t] = s;
    if (s < 0 || s >= total_slots) continue;  // pad slot or out of bounds: skip
    const int64_t dst = s * pieces_per_row + piece;
    const u32x4 kv = __builtin_nontemporal_load(&k_new[i]);
    const u32x4 vv = __builtin_nontemporal_load(&v_new[i]);
    // Streaming stores: the rows go on to memory now rather than staying
    // dirty in cache, where their later eviction slowed the next launch's
    // reads (a decode pass over 2.2 GB ran about 20 us longer after an
    // 8448-row write with plain stores, within 1 us with these).
    __builtin_nontemporal_store(kv, &k_cache[dst]);
    __builtin_nontemporal_store(vv, &v_cache[dst]);
  }
}

}  // namespace

hipError_t launch_slot_write(const int32_t* req_indices, const int64_t* positions,
                             int64_t num_tokens, int64_t max_num_tokens,
                             const int32_t* block_table, int32_t table_rows,
                             int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                             const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                             int64_t total_slots, int32_t row_bytes, hipStream_t stream) {
  const uint32_t pieces = (uint32_t)(row_bytes / 16);
  const int64_t n = num_tokens * (int64_t)pieces + (max_num_tokens - num_tokens);
  if (n == 0) return hipSuccess;
  const int shift =
      (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  slot_write_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows, table_stride,
      block_size, shift, slot_mapping, (const u32x4*)k_new, (const u32x4*)v_new,
      (u32x4*)k_cache, (u32x4*)v_cache, total_slots, pieces);
  return hipGetLastError();
}

}  // namespace kvs
