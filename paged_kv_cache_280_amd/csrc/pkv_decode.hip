// Launch of paged decode attention over bf16 pools: the decode kernel and the merge
// of split pairs (kernels in pkv_decode_kernels.h).  The kernel instances are spread
// over several translation units so that they compile in parallel.

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_decode(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                         int merge_groups, hipStream_t stream) {
  return dispatch<1, false, false>(b, d, D, B, merge_groups, stream);
}

}  // namespace pkv
