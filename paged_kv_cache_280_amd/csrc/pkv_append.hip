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

}  // namespace

hipError_t launch_append(const AppendBuffers& b, const AppendDims& a, int D, hipStream_t stream) {
  const int64_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  const int64_t waves = static_cast<int64_t>(a.T) * head_groups;
  const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  if (groups <= 0) return hipSuccess;
  if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
  if (D == 128)
    hipLaunchKernelGGL((append_kernel<128>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new, b.k_cache,
                       b.v_cache, b.tables, b.token_seq, b.token_pos, a);
  else if (D == 64)
    hipLaunchKernelGGL((append_kernel<64>), dim3(static_cast<uint32_t>(groups)),
                       dim3(kWave * kWavesPerGroup), 0, stream, b.k_new, b.v_new, b.k_cache,
                       b.v_cache, b.tables, b.token_seq, b.token_pos, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
