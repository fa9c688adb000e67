// Launch of one decode step with its KV append over bf16 pools (kernels in
// pkv_decode_kernels.h).

#include "pkv_decode_kernels.h"

namespace pkv {

hipError_t launch_decode_append(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                                int merge_groups, hipStream_t stream) {
  return dispatch<1, false, false, true>(b, d, D, B, merge_groups, stream);
}

}  // namespace pkv
