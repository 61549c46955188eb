// Slot mapping: the physical cache slot of every token of a step.
//
// "Padding and Batching with Block KV", sections "The Core Formula" and
// "Slot Mapping Computation": the slot of a token at position p of request r
// is block_table[r][p / block_size] * block_size + p % block_size. Padding
// tokens (request index -1) and inactive table entries (null block 0, the -1
// sentinel) give the pad slot -1 (sections "Slot ID -1" and "Block ID 0 vs.
// Sentinel -1"), and the tail of a fixed-size slot buffer is padded with -1
// (the vLLM block-table notes, data-flow listing).
//
// One thread per output entry, or per four consecutive entries when the
// three arrays are 16-byte aligned (one 16-byte load of request indices, two
// of positions and two 16-byte stores: a step's tokens come in runs of one
// request, so most of a launch's bytes are these streams, not the table).
// The streams are touched once, so they are read and written with the
// nontemporal hint; the table reads, which neighbouring tokens share, are
// plain loads.
// The vLLM kernel runs one program per request; a flat grid over tokens keeps
// every lane busy whatever the length mix.
#include "kvslot_internal.h"
#include "slot_formula.h"

namespace kvs {
namespace {

__global__ void __launch_bounds__(256)
slot_mapping_kernel(const int32_t* __restrict__ req_indices, const int64_t* __restrict__ positions,
                    int64_t num_tokens, int64_t max_num_tokens,
                    const int32_t* __restrict__ block_table, int32_t table_rows,
                    int32_t table_stride, int32_t block_size, int32_t block_shift,
                    int64_t* __restrict__ slot_mapping) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < max_num_tokens; t += stride) {
    slot_mapping[t] = t < num_tokens ? token_slot(req_indices[t], positions[t], block_table,
                                                  table_rows, table_stride, block_size,
                                                  block_shift)
                                     : -1;
  }
}

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int64_t i64x2 __attribute__((ext_vector_type(2)));

__global__ void __launch_bounds__(256)
slot_mapping_x4_kernel(const int32_t* __restrict__ req_indices,
                       const int64_t* __restrict__ positions, int64_t num_tokens,
                       int64_t max_num_tokens, const int32_t* __restrict__ block_table,
                       int32_t table_rows, int32_t table_stride, int32_t block_size,
                       int32_t block_shift, int64_t* __restrict__ slot_mapping) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t quads = (max_num_tokens + 3) / 4;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < quads; q += stride) {
    const int64_t t = 4 * q;
    if (t + 4 <= num_tokens) {
      const i32x4 r = __builtin_nontemporal_load((const i32x4*)(req_indices + t));
      const i64x2 p01 = __builtin_nontemporal_load((const i64x2*)(positions + t));
      const i64x2 p23 = __builtin_nontemporal_load((const i64x2*)(positions + t + 2));
      const i64x2 s01 = {token_slot(r[0], p01[0], block_table, table_rows, table_stride,
                                    block_size, block_shift),
                         token_slot(r[1], p01[1], block_table, table_rows, table_stride,
                                    block_size, block_shift)};
      const i64x2 s23 = {token_slot(r[2], p23[0], block_table, table_rows, table_stride,
                                    block_size, block_shift),
                         token_slot(r[3], p23[1], block_table, table_rows, table_stride,
                                    block_size, block_shift)};
      __builtin_nontemporal_store(s01, (i64x2*)(slot_mapping + t));
      __builtin_nontemporal_store(s23, (i64x2*)(slot_mapping + t + 2));
    } else {
      // the quad holding the step's last tokens, or only padding
      for (int64_t u = t; u < t + 4 && u < max_num_tokens; ++u)
        slot_mapping[u] = u < num_tokens ? token_slot(req_indices[u], positions[u], block_table,
                                                      table_rows, table_stride, block_size,
                                                      block_shift)
                                         : -1;
    }
  }
}

__global__ void __launch_bounds__(256)
slot_mapping_dcp_kernel(const int32_t* __restrict__ req_indices,
                        const int64_t* __restrict__ positions, int64_t num_tokens,
                        int64_t max_num_tokens, const int32_t* __restrict__ block_table,
                        int32_t table_rows, int32_t table_stride, int32_t block_size,
                        int32_t block_shift, int32_t world, int32_t rank, int32_t interleave_shift,
                        int64_t* __restrict__ slot_mapping) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < max_num_tokens; t += stride) {
    slot_mapping[t] = t < num_tokens
                          ? token_slot_dcp(req_indices[t], positions[t], block_table, table_rows,
                                           table_stride, block_size, block_shift, world, rank,
                                           interleave_shift)
                          : -1;
  }
}

}  // namespace

hipError_t launch_slot_mapping_dcp(const int32_t* req_indices, const int64_t* positions,
                                   int64_t num_tokens, int64_t max_num_tokens,
                                   const int32_t* block_table, int32_t table_rows,
                                   int32_t table_stride, int32_t block_size, int32_t world,
                                   int32_t rank, int32_t interleave, int64_t* slot_mapping,
                                   hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  int64_t blocks = (max_num_tokens + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  slot_mapping_dcp_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows, table_stride,
      block_size, __builtin_ctz((unsigned)block_size), world, rank,
      __builtin_ctz((unsigned)interleave), slot_mapping);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* req_indices, const int64_t* positions,
                               int64_t num_tokens, int64_t max_num_tokens,
                               const int32_t* block_table, int32_t table_rows,
                               int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                               hipStream_t stream) {
  if (max_num_tokens == 0) return hipSuccess;
  const int shift =
      (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  const bool x4 = (((uintptr_t)req_indices | (uintptr_t)positions | (uintptr_t)slot_mapping) &
                   15) == 0;
  const int64_t units = x4 ? (max_num_tokens + 3) / 4 : max_num_tokens;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (x4)
    slot_mapping_x4_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows,
        table_stride, block_size, shift, slot_mapping);
  else
    slot_mapping_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
        req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows,
        table_stride, block_size, shift, slot_mapping);
  return hipGetLastError();
}

}  // namespace kvs
