// Launch of paged decode attention over fp8 (E4M3FN) pools (kernels in
// pkv_decode_kernels.h).

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_decode_fp8(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                             int merge_groups, hipStream_t stream) {
  return dispatch<1, false, true>(b, d, D, B, merge_groups, stream);
}

}  // namespace pkv
