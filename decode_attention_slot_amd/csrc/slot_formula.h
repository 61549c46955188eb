// The slot of one token, shared by the slot-mapping kernels.
//
// "Padding and Batching with Block KV", sections "The Core Formula", "Slot
// ID -1: Padding Tokens" and "Block ID 0 vs. Sentinel -1": the token at
// position p of request r sits in slot block_table[r][p / block_size] *
// block_size + p % block_size. A padding token (r < 0), a row or column
// outside the table, a negative position and an inactive entry (null block
// 0, sentinel -1) give the pad slot -1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

// block_shift >= 0 when block_size is a power of two (then p >> block_shift
// replaces the division).
__device__ __forceinline__ int64_t token_slot(int32_t r, int64_t p,
                                              const int32_t* __restrict__ block_table,
                                              int32_t table_rows, int32_t table_stride,
                                              int32_t block_size, int32_t block_shift) {
  if (r < 0 || r >= table_rows || p < 0) return -1;
  const int64_t logical_block = block_shift >= 0 ? (p >> block_shift) : p / block_size;
  if (logical_block >= table_stride) return -1;
  const int32_t block = block_table[(int64_t)r * table_stride + logical_block];
  if (block <= 0) return -1;
  return (int64_t)block * block_size + (p - logical_block * block_size);
}

// Decode context parallelism ("Block table: logical token -> physical KV
// block", design motivation: under DCP the slot kernel writes a real slot
// only for the tokens its own rank stores, PAD otherwise). Runs of
// 2^interleave_shift consecutive positions go round-robin to the ranks; a
// rank packs its runs densely, so the position inside its own cache is
// (p / (world * I)) * I + p % I, whose block index is p / (world *
// block_size): every rank shares the table row. The interleave divides the
// block size.
__device__ __forceinline__ int64_t token_slot_dcp(int32_t r, int64_t p,
                                                  const int32_t* __restrict__ block_table,
                                                  int32_t table_rows, int32_t table_stride,
                                                  int32_t block_size, int32_t block_shift,
                                                  int32_t world, int32_t rank,
                                                  int32_t interleave_shift) {
  if (p < 0) return -1;
  const int64_t run = p >> interleave_shift;
  if (run % world != rank) return -1;
  const int64_t mask = ((int64_t)1 << interleave_shift) - 1;
  const int64_t local = ((run / world) << interleave_shift) + (p & mask);
  return token_slot(r, local, block_table, table_rows, table_stride, block_size, block_shift);
}

}  // namespace kvs
