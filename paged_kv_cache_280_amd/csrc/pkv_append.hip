// KV append: the key and value rows of new tokens go into the slots their
// positions map to through the block table.  "PagedAttention (vLLM)"
// (troisinh.com), section "Cơ chế Block Table": position p of a sequence lives in
// logical block p / B at offset p % B, and the table gives the physical block;
// blocks are taken only when a token needs them, so the caller's block manager
// has already made room (and resolved copy-on-write) before this runs.
//
// One wave per (token, group of four KV heads).  K rows land as 16-byte chunks
// (the K pool keeps 8 consecutive dims together); V rows are dim-major in the pool,
// so each dim of a token is one 2-byte store.
//
// fp8 pools ("KV cache, PagedAttention", aiwiki.vn, paragraph on cache
// quantisation): each element is stored as the E4M3FN code nearest to x / scale
// (ties to even), saturating at +-448; NaN is stored as 0x7F.  K chunks of 16 dims
// are one 16-byte store; V codes are one byte each.

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAppendHeadsPerWave = 4;

template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  constexpr int kChunks = D / 8;                        // 16-byte K chunks per head row
  constexpr int kLanesPerHead = kWave / kAppendHeadsPerWave;  // 16
  const int lane = __lane_id();
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + threadIdx.x / kWave;
  const int32_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  if (item >= static_cast<int64_t>(a.T) * head_groups) return;
  const int32_t t = static_cast<int32_t>(item / head_groups);
  const int32_t g = static_cast<int32_t>(item % head_groups) * kAppendHeadsPerWave +
                    lane / kLanesPerHead;
  if (g >= a.Hkv) return;
  const int32_t s = token_seq[t];
  const int32_t p = token_pos[t];
  if (s < 0 || s >= a.S || p < 0 || p >= a.M * a.B) return;  // not a slot of this pool
  const int32_t b = tables[static_cast<int64_t>(s) * a.M + p / a.B];
  if (b < 0 || b >= a.NB) return;                            // never write outside the pool
  const int32_t o = p % a.B;
  const int64_t tile = (static_cast<int64_t>(b) * a.Hkv + g) * D * a.B;  // (block, head) tile
  const uint16_t* kr = k_new + (static_cast<int64_t>(t) * a.Hkv + g) * D;
  const uint16_t* vr = v_new + (static_cast<int64_t>(t) * a.Hkv + g) * D;
  const int sub = lane % kLanesPerHead;
  for (int c = sub; c < kChunks; c += kLanesPerHead)
    *reinterpret_cast<u32x4_t*>(k_cache + tile + (static_cast<int64_t>(c) * a.B + o) * 8) =
        *reinterpret_cast<const u32x4_t*>(kr + c * 8);
  for (int dd = sub; dd < D; dd += kLanesPerHead)
    v_cache[tile + static_cast<int64_t>(dd) * a.B + o] = vr[dd];
}

// E4M3FN code of y: NaN -> 0x7F; otherwise y clamped to +-448 and converted by
// the hardware (round to nearest even), which then never leaves the finite range.
__device__ __forceinline__ float e4m3_ready(float y) {
  return fminf(fmaxf(y, -448.0f), 448.0f);
}

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

__device__ __forceinline__ float widen_bf16(uint16_t x) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
}

template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_fp8_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  constexpr int kChunks = D / 16;                       // 16-byte K chunks per head row
  constexpr int kLanesPerHead = kWave / kAppendHeadsPerWave;  // 16
  const int lane = __lane_id();
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + threadIdx.x / kWave;
  const int32_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  if (item >= static_cast<int64_t>(a.T) * head_groups) return;
  const int32_t t = static_cast<int32_t>(item / head_groups);
  const int32_t g = static_cast<int32_t>(item % head_groups) * kAppendHeadsPerWave +
                    lane / kLanesPerHead;
  if (g >= a.Hkv) return;
  const int32_t s = token_seq[t];
  const int32_t p = token_pos[t];
  if (s < 0 || s >= a.S || p < 0 || p >= a.M * a.B) return;  // not a slot of this pool
  const int32_t b = tables[static_cast<int64_t>(s) * a.M + p / a.B];
  if (b < 0 || b >= a.NB) return;                            // never write outside the pool
  const int32_t o = p % a.B;
  const int64_t tile = (static_cast<int64_t>(b) * a.Hkv + g) * D * a.B;  // bytes
  const uint16_t* kr = k_new + (static_cast<int64_t>(t) * a.Hkv + g) * D;
  const uint16_t* vr = v_new + (static_cast<int64_t>(t) * a.Hkv + g) * D;
  const int sub = lane % kLanesPerHead;
  for (int c = sub; c < kChunks; c += kLanesPerHead) {
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = widen_bf16(kr[c * 16 + i]) / a.k_scale;
    const u32x4_t w = {e4m3x4(x[0], x[1], x[2], x[3]), e4m3x4(x[4], x[5], x[6], x[7]),
                       e4m3x4(x[8], x[9], x[10], x[11]), e4m3x4(x[12], x[13], x[14], x[15])};
    *reinterpret_cast<u32x4_t*>(k_cache + tile + (static_cast<int64_t>(c) * a.B + o) * 16) = w;
  }
  // V element (o, d) at [d%16][o/4][d/16][o%4] of the tile
  for (int dd = sub; dd < D; dd += kLanesPerHead) {
    const float y = widen_bf16(vr[dd]) / a.v_scale;
    const uint32_t code = e4m3x4(y, 0.f, 0.f, 0.f) & 0xFFu;
    v_cache[tile + ((static_cast<int64_t>(dd % 16) * (a.B / 4) + o / 4) * (D / 16) + dd / 16) * 4 +
            o % 4] = static_cast<uint8_t>(code);
  }
}

}  // namespace

hipError_t launch_append(const AppendBuffers& b, const AppendDims& a, int D, hipStream_t stream) {
  const int64_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  const int64_t waves = static_cast<int64_t>(a.T) * head_groups;
  const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  if (groups <= 0) return hipSuccess;
  if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
  if (D == 128)
    hipLaunchKernelGGL((append_kernel<128>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new,
                       static_cast<uint16_t*>(b.k_cache), static_cast<uint16_t*>(b.v_cache),
                       b.tables, b.token_seq, b.token_pos, a);
  else if (D == 64)
    hipLaunchKernelGGL((append_kernel<64>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new,
                       static_cast<uint16_t*>(b.k_cache), static_cast<uint16_t*>(b.v_cache),
                       b.tables, b.token_seq, b.token_pos, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_append_fp8(const AppendBuffers& b, const AppendDims& a, int D,
                             hipStream_t stream) {
  const int64_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  const int64_t waves = static_cast<int64_t>(a.T) * head_groups;
  const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  if (groups <= 0) return hipSuccess;
  if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
  uint8_t* kc = static_cast<uint8_t*>(b.k_cache);
  uint8_t* vc = static_cast<uint8_t*>(b.v_cache);
  if (D == 128)
    hipLaunchKernelGGL((append_fp8_kernel<128>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new, kc, vc, b.tables,
                       b.token_seq, b.token_pos, a);
  else if (D == 64)
    hipLaunchKernelGGL((append_fp8_kernel<64>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new, kc, vc, b.tables,
                       b.token_seq, b.token_pos, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
