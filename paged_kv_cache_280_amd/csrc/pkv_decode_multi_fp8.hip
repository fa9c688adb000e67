// Launch of multi-token (causal) paged attention over fp8 pools (kernels in
// pkv_decode_kernels.h).

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_multi_fp8(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                            int merge_groups, hipStream_t stream) {
  if (d.R <= 16) return dispatch<1, true, true>(b, d, D, B, merge_groups, stream);
  if (d.R <= kMaxRows) return dispatch<2, true, true>(b, d, D, B, merge_groups, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
