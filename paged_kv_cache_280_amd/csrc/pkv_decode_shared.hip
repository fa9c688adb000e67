// Launches of shared-prefix decode over bf16 pools: the prefix pass (one or two
// 16-column tiles of (group member, head) rows per wave) and the tail pass.
// Kernels in pkv_decode_kernels.h.

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_shared_prefix(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                                int merge_groups, hipStream_t stream) {
  if (d.R <= 16) return dispatch<1, true, false, false, 1>(b, d, D, B, merge_groups, stream);
  if (d.R <= kMaxRows) return dispatch<2, true, false, false, 1>(b, d, D, B, merge_groups, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_shared_tail(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                              int merge_groups, hipStream_t stream) {
  return dispatch<1, false, false, false, 2>(b, d, D, B, merge_groups, stream);
}

}  // namespace pkv
