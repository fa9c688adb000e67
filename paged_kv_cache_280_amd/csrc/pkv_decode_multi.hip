// Launch of multi-token (causal) paged attention over bf16 pools, one or two
// 16-column tiles of (query token, head) rows per wave; fp8 pools go to
// launch_multi_fp8 (pkv_decode_multi_fp8.hip).  Kernels in pkv_decode_kernels.h.

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_multi(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                        int merge_groups, hipStream_t stream, bool fp8) {
  if (fp8) return launch_multi_fp8(b, d, D, B, merge_groups, stream);
  if (d.R <= 16) return dispatch<1, true, false>(b, d, D, B, merge_groups, stream);
  if (d.R <= kMaxRows) return dispatch<2, true, false>(b, d, D, B, merge_groups, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
