// HBM read-stream probe (declared in include/pkv_stream.h): sequential reads and
// the decode kernel's paired gather of K/V units, with no arithmetic beyond an XOR
// that keeps every load live.  Every load carries the non-temporal hint, as the
// decode kernel's K/V loads do.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pkv.h"
#include "pkv_stream.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = kThreads / kWave;

// Work-group g reads the 16 KiB chunks g, g + G, g + 2G, ... (G work-groups); a
// thread takes four 16-byte elements 4 KiB apart, so one load instruction of a
// wave covers 1 KiB of contiguous memory.
__global__ __launch_bounds__(kThreads) void read_seq_kernel(const u32x4_t* __restrict__ src,
                                                            int64_t n16,
                                                            uint32_t* __restrict__ sink) {
  constexpr int64_t kChunk = kThreads * 4;  // 16-byte elements per chunk
  const int64_t chunks = n16 / kChunk;
  u32x4_t acc = {0, 0, 0, 0};
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const u32x4_t* p = src + c * kChunk + threadIdx.x;
    const u32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + kThreads),
                  d = __builtin_nontemporal_load(p + 2 * kThreads),
                  e = __builtin_nontemporal_load(p + 3 * kThreads);
    acc ^= a ^ b ^ d ^ e;
  }
  for (int64_t i = chunks * kChunk + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
       i < n16; i += static_cast<int64_t>(gridDim.x) * kThreads)
    acc ^= __builtin_nontemporal_load(src + i);
  sink[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// One unit of a pool in registers: kUnit bytes as kUnit/1024 16-byte lane loads (K)
// or kUnit/512 8-byte lane loads (V with 8-byte loads).
template <int kUnit, int kVBytes>
struct Unit {
  static constexpr int kK = kUnit / 1024;
  static constexpr int kV = kUnit / (kWave * kVBytes);
  using VLoad = typename std::conditional<kVBytes == 16, u32x4_t, u32x2_t>::type;
  u32x4_t k[kK];
  VLoad v[kV];

  __device__ __forceinline__ void load(const uint8_t* kp, const uint8_t* vp, int64_t off,
                                       int lane) {
#pragma unroll
    for (int c = 0; c < kK; ++c)
      k[c] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(kp + off + c * 1024 + lane * 16));
#pragma unroll
    for (int c = 0; c < kV; ++c)
      v[c] = __builtin_nontemporal_load(
          reinterpret_cast<const VLoad*>(vp + off + c * kWave * kVBytes + lane * kVBytes));
  }
  __device__ __forceinline__ uint32_t fold() const {
    uint32_t x = 0;
#pragma unroll
    for (int c = 0; c < kK; ++c) x ^= k[c].x ^ k[c].y ^ k[c].z ^ k[c].w;
#pragma unroll
    for (int c = 0; c < kV; ++c) {
      x ^= v[c].x ^ v[c].y;
      if constexpr (kVBytes == 16) x ^= v[c].z ^ v[c].w;
    }
    return x;
  }
};

template <int kUnit, int kVBytes, int kInFlight>
__global__ __launch_bounds__(kThreads) void read_pairs_kernel(const uint8_t* __restrict__ kp,
                                                              const uint8_t* __restrict__ vp,
                                                              int64_t pool_units,
                                                              const int32_t* __restrict__ ids,
                                                              int32_t n, int32_t waves,
                                                              uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % kWave;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup +
                    __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  if (w >= waves) return;
  const int64_t i0 = w * n / waves, i1 = (w + 1) * n / waves;
  Unit<kUnit, kVBytes> u[kInFlight];
  uint32_t acc = 0;
  auto off = [&](int64_t j) {
    const int64_t id = ids[j];
    return (id < 0 ? 0 : (id >= pool_units ? pool_units - 1 : id)) * kUnit;
  };
  int64_t i = i0;
  // whole groups of kInFlight units: all loads issued, then folded
  for (; i + kInFlight <= i1; i += kInFlight) {
#pragma unroll
    for (int j = 0; j < kInFlight; ++j)
      u[j].load(kp, vp, off(i + j), lane);
#pragma unroll
    for (int j = 0; j < kInFlight; ++j) acc ^= u[j].fold();
  }
  for (; i < i1; ++i) {
    u[0].load(kp, vp, off(i), lane);
    acc ^= u[0].fold();
  }
  sink[w * kWave + lane] = acc;
}

template <int kUnit, int kVBytes, int kInFlight>
hipError_t launch_depth(const void* k, const void* v, int64_t pool_units, const int32_t* ids,
                        int32_t n, int32_t waves, uint32_t* sink, hipStream_t s) {
  const int groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL((read_pairs_kernel<kUnit, kVBytes, kInFlight>), dim3(groups), dim3(kThreads), 0, s,
                     static_cast<const uint8_t*>(k), static_cast<const uint8_t*>(v), pool_units,
                     ids, n, waves, sink);
  return hipGetLastError();
}

// Units of each pool a wave keeps in flight: 3 (as the decode kernel's tile
// pipeline) or 6.
template <int kUnit, int kVBytes>
hipError_t launch_pairs(const void* k, const void* v, int64_t pool_units, const int32_t* ids,
                        int32_t n, int32_t waves, int32_t depth, uint32_t* sink, hipStream_t s) {
  return depth == 6 ? launch_depth<kUnit, kVBytes, 6>(k, v, pool_units, ids, n, waves, sink, s)
                    : launch_depth<kUnit, kVBytes, 3>(k, v, pool_units, ids, n, waves, sink, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int32_t pkv_stream_read(const void* src, size_t n_bytes, uint32_t* sink, int32_t groups,
                        void* stream) {
  if (n_bytes == 0 || n_bytes % 16 != 0 || groups <= 0) return PKV_ERR_SHAPE;
  if (!src || !sink) return PKV_ERR_NULL;
  if (!aligned16(src)) return PKV_ERR_ALIGNMENT;
  hipLaunchKernelGGL(read_seq_kernel, dim3(groups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src),
                     static_cast<int64_t>(n_bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

int32_t pkv_stream_read_pairs(const void* k_pool, const void* v_pool, int64_t pool_units,
                              const int32_t* ids, int32_t n_units, int32_t unit_bytes,
                              int32_t v_load_bytes, uint32_t* sink, int32_t waves,
                              int32_t depth, void* stream) {
  if (n_units < 0 || waves <= 0 || pool_units <= 0) return PKV_ERR_SHAPE;
  if (depth != 3 && depth != 6) return PKV_ERR_UNSUPPORTED;
  if (unit_bytes != 1024 && unit_bytes != 2048 && unit_bytes != 4096) return PKV_ERR_UNSUPPORTED;
  if (v_load_bytes != 8 && v_load_bytes != 16) return PKV_ERR_UNSUPPORTED;
  if (n_units == 0) return PKV_OK;
  if (!k_pool || !v_pool || !ids || !sink) return PKV_ERR_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool)) return PKV_ERR_ALIGNMENT;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (v_load_bytes == 16)
    e = unit_bytes == 4096   ? launch_pairs<4096, 16>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s)
        : unit_bytes == 2048 ? launch_pairs<2048, 16>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s)
                             : launch_pairs<1024, 16>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s);
  else
    e = unit_bytes == 4096   ? launch_pairs<4096, 8>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s)
        : unit_bytes == 2048 ? launch_pairs<2048, 8>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s)
                             : launch_pairs<1024, 8>(k_pool, v_pool, pool_units, ids, n_units, waves, depth, sink, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
