// E4M3FN encoding shared by the kernels that write fp8 pools ("KV cache,
// PagedAttention", aiwiki.vn, paragraph on cache quantisation): an element is
// stored as the code nearest to x / scale (ties to even), saturating at +-448;
// NaN is stored as 0x7F.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// y clamped to +-448: the hardware conversion (round to nearest even) then never
// leaves the finite range.
__device__ __forceinline__ float e4m3_ready(float y) { return fminf(fmaxf(y, -448.0f), 448.0f); }

// Four codes packed in one dword, first element in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const bool nan_a = __builtin_isnan(a), nan_b = __builtin_isnan(b);
  const bool nan_c = __builtin_isnan(c), nan_d = __builtin_isnan(d);
  uint32_t w = static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_ready(a), e4m3_ready(b), 0, false));
  w = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_ready(c), e4m3_ready(d),
                                                            static_cast<int>(w), true));
  if (nan_a) w = (w & 0xFFFFFF00u) | 0x7Fu;
  if (nan_b) w = (w & 0xFFFF00FFu) | 0x7F00u;
  if (nan_c) w = (w & 0xFF00FFFFu) | 0x7F0000u;
  if (nan_d) w = (w & 0x00FFFFFFu) | 0x7F000000u;
  return w;
}

// The two bf16 values of a dword as floats (first element in the low half).
__device__ __forceinline__ float lo_bf16(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t x) {
  return __builtin_bit_cast(float, x & 0xFFFF0000u);
}

}  // namespace pkv
