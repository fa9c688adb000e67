// Launches of shared-prefix decode over bf16 pools: both passes in one launch
// (the prefix pass with one or two 16-column tiles of (group member, head) rows
// per wave, the tail pass with one) and the tail merge, or the tail pass alone.
// Kernels in pkv_decode_kernels.h.

#include "pkv_decode_kernels.h"

namespace pkv {

namespace {

template <int NCp>
hipError_t shared_for(const DecodeBuffers& bp, const DecodeDims& a, const DecodeBuffers& bt,
                      const DecodeDims& d, int D, int B, int32_t* gmap, int mgt, hipStream_t s) {
  if (D == 128) {
    if (B == 16) return launch_shared_t<128, 16, NCp>(bp, a, bt, d, gmap, mgt, s);
    if (B == 32) return launch_shared_t<128, 32, NCp>(bp, a, bt, d, gmap, mgt, s);
    if (B == 8) return launch_shared_t<128, 8, NCp>(bp, a, bt, d, gmap, mgt, s);
  } else if (D == 64) {
    if (B == 16) return launch_shared_t<64, 16, NCp>(bp, a, bt, d, gmap, mgt, s);
    if (B == 32) return launch_shared_t<64, 32, NCp>(bp, a, bt, d, gmap, mgt, s);
    if (B == 8) return launch_shared_t<64, 8, NCp>(bp, a, bt, d, gmap, mgt, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_shared(const DecodeBuffers& bp, const DecodeDims& a, const DecodeBuffers& bt,
                         const DecodeDims& d, int D, int B, int32_t* gmap, int merge_groups_tail,
                         hipStream_t stream) {
  if (a.R <= 16) return shared_for<1>(bp, a, bt, d, D, B, gmap, merge_groups_tail, stream);
  if (a.R <= kMaxRows) return shared_for<2>(bp, a, bt, d, D, B, gmap, merge_groups_tail, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_shared_tail(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                              int merge_groups, hipStream_t stream) {
  return dispatch<1, false, false, false, 2>(b, d, D, B, merge_groups, stream);
}

}  // namespace pkv
