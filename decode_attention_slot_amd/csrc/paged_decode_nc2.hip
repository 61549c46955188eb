// Pass 1 of the decode attention at 17-32 query rows per KV head (2 column
// tiles of 16 rows per wave), in a translation unit of its own so that the
// library's sources compile side by side. The kernel is in paged_decode.h.
#include "paged_decode.h"

namespace kvs {

hipError_t decode_pass1_nc2(const DecodeParams& p, hipStream_t stream) {
  return pass1_for<2, 1>(p, stream);
}

hipError_t decode_slices_nc2(const DecodeParams& p, int* slices) {
  return slices_for<2, 1>(p, slices);
}

}  // namespace kvs
