// Merge of per-rank decode attention partial states (context parallelism).
//
// Each rank of a context-parallel group attends over the keys it stores
// and returns its normalised output and the natural-log sum of exp(scores)
// of each row ("Block table: logical token -> physical KV block", DCP / PCP
// interleave: ranks hold disjoint slots). Softmax over the union of the
// ranks' disjoint key sets is the ranks' outputs weighted by
// exp(lse_rank - lse_total). After the ranks' partials are gathered this
// kernel produces the attention output, and the total lse.
//
// One thread per (row, 4 dimensions): it reads the world lse values of its
// row (cache hits after the first thread of the row) and the world float4s.
#include <math.h>

#include "kvslot_internal.h"

namespace kvs {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
lse_merge_kernel(const f32x4* __restrict__ outs, const float* __restrict__ lses, int32_t world,
                 int64_t rows, int32_t f4_per_row, f32x4* __restrict__ out,
                 float* __restrict__ lse) {
  const int64_t n = rows * f4_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t row = i / f4_per_row;
    float mx = -INFINITY;
    for (int k = 0; k < world; ++k) mx = fmaxf(mx, lses[(int64_t)k * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.0f;
    if (mx != -INFINITY) {
      for (int k = 0; k < world; ++k) {
        const float lk = lses[(int64_t)k * rows + row];
        if (lk == -INFINITY) continue;  // this rank saw no key of the row
        const float wk = expf(lk - mx);
        acc += outs[(int64_t)k * n + i] * wk;
        tot += wk;
      }
    }
    out[i] = tot > 0.0f ? acc * (1.0f / tot) : acc;
    if (lse && i == row * f4_per_row) lse[row] = tot > 0.0f ? mx + logf(tot) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_lse_merge(const float* outs, const float* lses, int32_t world, int64_t rows,
                            int32_t head_dim, float* out, float* lse, hipStream_t stream) {
  const int32_t f4 = head_dim / 4;
  const int64_t n = rows * f4;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  lse_merge_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      (const f32x4*)outs, lses, world, rows, f4, (f32x4*)out, lse);
  return hipGetLastError();
}

}  // namespace kvs
