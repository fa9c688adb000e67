// KV append: the key and value rows of new tokens go into the slots their
// positions map to through the block table.  "PagedAttention (vLLM)"
// (troisinh.com), section "Cơ chế Block Table": position p of a sequence lives in
// logical block p / B at offset p % B, and the table gives the physical block;
// blocks are taken only when a token needs them, so the caller's block manager
// has already made room (and resolved copy-on-write) before this runs.
//
// One wave per (16 consecutive input tokens, group of four KV heads); lane
// (j, h) writes token t0 + j's row of head h.  K rows land as 16-byte chunks (the
// K pool keeps 8 consecutive dims together).  V rows are dim-major in the pool
// (each 16-position half of a block its own [D][16] run), so each dim of a token is
// one 2-byte store; when the 16 tokens are consecutive positions of one sequence (a
// prefill chunk), the stores of one dim from the 16 lanes of a head fall on
// consecutive slots and coalesce.
//
// Small appends (a decode step: one token per sequence, scattered over blocks) take
// the row kernels instead: one thread per (token, KV head, 8 dims), so that a few
// tokens still spread over many waves (with 16 tokens per wave a decode step of 8
// sequences ran as two waves, each lane converting 128 values in a row).
//
// fp8 pools ("KV cache, PagedAttention", aiwiki.vn, paragraph on cache
// quantisation): each element is stored as the E4M3FN code nearest to x / scale
// (ties to even), saturating at +-448; NaN is stored as 0x7F.  K chunks of 16 dims
// are one 16-byte store; V codes are one byte each.

#include "pkv_fp8.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kAppendHeadsPerWave = 4;
constexpr int kAppendTokensPerWave = kWave / kAppendHeadsPerWave;  // 16

// Slot of token t's row of head g: its (block, head) tile (elements of the pool
// before it) and offset o in the block.  False when the token names no slot of this
// pool: sequence or position out of range, or a table entry outside the pool.
template <int D>
__device__ __forceinline__ bool token_slot(int64_t t, int32_t g, const int32_t* __restrict__ tables,
                                           const int32_t* __restrict__ token_seq,
                                           const int32_t* __restrict__ token_pos,
                                           const AppendDims& a, int64_t& tile, int32_t& o) {
  if (t >= a.T || g >= a.Hkv) return false;
  const int32_t cap = a.M * a.B;
  const int32_t s = a.newest ? static_cast<int32_t>(t) : token_seq[t];
  const int32_t p = a.newest ? (token_pos[t] < 0 ? 0 : min(token_pos[t], cap)) - 1 : token_pos[t];
  if (s < 0 || s >= a.S || p < 0 || p >= cap) return false;
  const int32_t b = tables[static_cast<int64_t>(s) * a.M + p / a.B];
  if (b < 0 || b >= a.NB) return false;  // never write outside the pool
  tile = (static_cast<int64_t>(b) * a.Hkv + g) * D * a.B * tile_span(a.kv_mul);
  o = p % a.B;
  return true;
}

// Index of this lane's wave among all waves of the launch, and the wave's group
// of four KV heads and first token.
struct AppendWave {
  int32_t g0;   // first KV head of the group
  int64_t t0;   // first of the wave's 16 tokens
};

__device__ __forceinline__ AppendWave append_wave(const AppendDims& a) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + threadIdx.x / kWave;
  const int32_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  return {static_cast<int32_t>(item % head_groups) * kAppendHeadsPerWave,
          (item / head_groups) * kAppendTokensPerWave};
}

template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  const int lane = __lane_id();
  const AppendWave w = append_wave(a);
  const int64_t t = w.t0 + lane % kAppendTokensPerWave;
  const int32_t g = w.g0 + lane / kAppendTokensPerWave;
  int64_t tile;
  int32_t o;
  if (!token_slot<D>(t, g, tables, token_seq, token_pos, a, tile, o)) return;
  const uint16_t* kr = k_new + (t * a.Hkv + g) * D;
  const uint16_t* vr = v_new + (t * a.Hkv + g) * D;
#pragma unroll
  for (int c = 0; c < D / 8; ++c)
    *reinterpret_cast<u32x4_t*>(k_cache + tile + (static_cast<int64_t>(c) * a.B + o) * 8) =
        *reinterpret_cast<const u32x4_t*>(kr + c * 8);
  const int32_t bt = a.B < 16 ? a.B : 16;  // positions of one V run
  uint16_t* vrun = v_cache + tile + static_cast<int64_t>(o / bt) * D * bt + o % bt;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(vr + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vrun[static_cast<int64_t>(c * 8 + i) * bt] = static_cast<uint16_t>(x[i / 2] >> (16 * (i % 2)));
  }
}

// Codes of 8 consecutive bf16 values (one 16-byte load) divided by scale.
__device__ __forceinline__ void e4m3x8(const uint16_t* src, float scale, uint32_t& lo,
                                       uint32_t& hi) {
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(src);
  lo = e4m3x4(lo_bf16(x[0]) / scale, hi_bf16(x[0]) / scale, lo_bf16(x[1]) / scale,
              hi_bf16(x[1]) / scale);
  hi = e4m3x4(lo_bf16(x[2]) / scale, hi_bf16(x[2]) / scale, lo_bf16(x[3]) / scale,
              hi_bf16(x[3]) / scale);
}

// Appends of fewer tokens than this take the row kernels.
constexpr int32_t kRowAppendTokens = 1024;

// Thread (t, g, c) of a row kernel: token t's row of KV head g, dims 8c .. 8c + 7.
struct RowItem {
  int64_t t;
  int32_t g, c;
};

template <int D>
__device__ __forceinline__ bool row_item(const AppendDims& a, RowItem& r) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_token = static_cast<int64_t>(a.Hkv) * (D / 8);
  r.t = i / per_token;
  const int32_t rem = static_cast<int32_t>(i - r.t * per_token);
  r.g = rem / (D / 8);
  r.c = rem - r.g * (D / 8);
  return r.t < a.T;
}

template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_rows_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  RowItem r;
  if (!row_item<D>(a, r)) return;
  int64_t tile;
  int32_t o;
  if (!token_slot<D>(r.t, r.g, tables, token_seq, token_pos, a, tile, o)) return;
  const int64_t row = (r.t * a.Hkv + r.g) * D + r.c * 8;
  *reinterpret_cast<u32x4_t*>(k_cache + tile + (static_cast<int64_t>(r.c) * a.B + o) * 8) =
      *reinterpret_cast<const u32x4_t*>(k_new + row);
  const int32_t bt = a.B < 16 ? a.B : 16;  // positions of one V run
  uint16_t* vrun = v_cache + tile + static_cast<int64_t>(o / bt) * D * bt + o % bt;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(v_new + row);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    vrun[static_cast<int64_t>(r.c * 8 + i) * bt] = static_cast<uint16_t>(x[i / 2] >> (16 * (i % 2)));
}

template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_fp8_rows_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  RowItem r;
  if (!row_item<D>(a, r)) return;
  int64_t tile;
  int32_t o;
  if (!token_slot<D>(r.t, r.g, tables, token_seq, token_pos, a, tile, o)) return;
  const int64_t row = (r.t * a.Hkv + r.g) * D + r.c * 8;
  uint32_t k0, k1, v0, v1;
  e4m3x8(k_new + row, a.k_scale, k0, k1);
  e4m3x8(v_new + row, a.v_scale, v0, v1);
  // K: dims of one 16-dim group are 16 consecutive bytes of token o
  *reinterpret_cast<u32x2_t*>(k_cache + tile + (static_cast<int64_t>(r.c / 2) * a.B + o) * 16 +
                              (r.c % 2) * 8) = u32x2_t{k0, k1};
  // V element (o, d) at [d%16][o/4][d/16][o%4] of the tile
  const int64_t row_bytes = (D / 16) * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = r.c * 8 + i;
    const uint32_t code = ((i < 4 ? v0 : v1) >> (8 * (i % 4))) & 0xFFu;
    v_cache[tile + (static_cast<int64_t>(d % 16) * (a.B / 4) + o / 4) * row_bytes + (d / 16) * 4 +
            o % 4] = static_cast<uint8_t>(code);
  }
}

// fp8: lane (j, k) of a head's 16 lanes takes tokens t0 + 4j .. t0 + 4j + 3 and
// dims k*D/4 .. (k+1)*D/4 - 1.  The V pool keeps the codes of 4 consecutive
// positions of one dim in one dword, so when the lane's 4 tokens are such a
// position quad (same block, offsets 4m .. 4m+3: a prefill chunk in order) each
// dim is one dword store; otherwise each token's codes are byte stores.
template <int D>
__global__ __launch_bounds__(kWave* kWavesPerGroup) void append_fp8_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ token_seq,
    const int32_t* __restrict__ token_pos, AppendDims a) {
  constexpr int kDims = D / 4;  // dims per lane: 32 or 16
  const int lane = __lane_id();
  const AppendWave w = append_wave(a);
  const int32_t g = w.g0 + lane / kAppendTokensPerWave;
  const int64_t t0 = w.t0 + (lane % kAppendTokensPerWave) / 4 * 4;
  const int d0 = (lane % 4) * kDims;
  int64_t tile[4];  // in bytes for fp8 pools
  int32_t o[4];
  bool ok[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    ok[u] = token_slot<D>(t0 + u, g, tables, token_seq, token_pos, a, tile[u], o[u]);
  bool quad = ok[0] && ok[1] && ok[2] && ok[3] && o[0] % 4 == 0;
#pragma unroll
  for (int u = 1; u < 4; ++u) quad = quad && tile[u] == tile[0] && o[u] == o[0] + u;

  uint32_t cv[4][kDims / 4];  // V codes, dword i of token u = dims d0 + 4i .. 4i+3
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (!ok[u]) continue;
    const int64_t row = ((t0 + u) * a.Hkv + g) * D + d0;
#pragma unroll
    for (int c = 0; c < kDims / 16; ++c) {  // one 16-byte K chunk per 16 dims
      uint32_t k0, k1, k2, k3;
      e4m3x8(k_new + row + c * 16, a.k_scale, k0, k1);
      e4m3x8(k_new + row + c * 16 + 8, a.k_scale, k2, k3);
      *reinterpret_cast<u32x4_t*>(
          k_cache + tile[u] + (static_cast<int64_t>(d0 / 16 + c) * a.B + o[u]) * 16) =
          u32x4_t{k0, k1, k2, k3};
    }
#pragma unroll
    for (int c = 0; c < kDims / 8; ++c) e4m3x8(v_new + row + c * 8, a.v_scale, cv[u][2 * c],
                                               cv[u][2 * c + 1]);
  }
  // V element (o, d) at [d%16][o/4][d/16][o%4] of the tile
  const int64_t row_bytes = (D / 16) * 4;  // one [d%16][o/4] row
  if (quad) {
#pragma unroll
    for (int i = 0; i < kDims; ++i) {
      const int d = d0 + i;
      const int sh = 8 * (i % 4);
      const uint32_t word = ((cv[0][i / 4] >> sh) & 0xFFu) | (((cv[1][i / 4] >> sh) & 0xFFu) << 8) |
                            (((cv[2][i / 4] >> sh) & 0xFFu) << 16) |
                            (((cv[3][i / 4] >> sh) & 0xFFu) << 24);
      *reinterpret_cast<uint32_t*>(
          v_cache + tile[0] + (static_cast<int64_t>(d % 16) * (a.B / 4) + o[0] / 4) * row_bytes +
          (d / 16) * 4) = word;
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int i = 0; i < kDims; ++i) {
        const int d = d0 + i;
        v_cache[tile[u] + (static_cast<int64_t>(d % 16) * (a.B / 4) + o[u] / 4) * row_bytes +
                (d / 16) * 4 + o[u] % 4] = static_cast<uint8_t>(cv[u][i / 4] >> (8 * (i % 4)));
      }
    }
  }
}

}  // namespace

// Row-kernel launch: one thread per (token, KV head, 8 dims).
template <typename KernelT, typename Elem>
hipError_t launch_rows(KernelT kernel, const AppendBuffers& b, const AppendDims& a, int D,
                       Elem* kc, Elem* vc, hipStream_t stream) {
  const int64_t threads = static_cast<int64_t>(a.T) * a.Hkv * (D / 8);
  const int64_t groups = (threads + kWave * kWavesPerGroup - 1) / (kWave * kWavesPerGroup);
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL(kernel, dim3(static_cast<uint32_t>(groups)), dim3(kWave * kWavesPerGroup), 0,
                     stream, b.k_new, b.v_new, kc, vc, b.tables, b.token_seq, b.token_pos, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendBuffers& b, const AppendDims& a, int D, hipStream_t stream) {
  if (a.T < kRowAppendTokens) {
    uint16_t* kc = static_cast<uint16_t*>(b.k_cache);
    uint16_t* vc = static_cast<uint16_t*>(b.v_cache);
    if (D == 128) return launch_rows(append_rows_kernel<128>, b, a, D, kc, vc, stream);
    if (D == 64) return launch_rows(append_rows_kernel<64>, b, a, D, kc, vc, stream);
    return hipErrorInvalidValue;
  }
  const int64_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  const int64_t waves =
      (static_cast<int64_t>(a.T) + kAppendTokensPerWave - 1) / kAppendTokensPerWave * head_groups;
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
  if (a.T < kRowAppendTokens) {
    uint8_t* kc = static_cast<uint8_t*>(b.k_cache);
    uint8_t* vc = static_cast<uint8_t*>(b.v_cache);
    if (D == 128) return launch_rows(append_fp8_rows_kernel<128>, b, a, D, kc, vc, stream);
    if (D == 64) return launch_rows(append_fp8_rows_kernel<64>, b, a, D, kc, vc, stream);
    return hipErrorInvalidValue;
  }
  const int64_t head_groups = (a.Hkv + kAppendHeadsPerWave - 1) / kAppendHeadsPerWave;
  const int64_t waves =
      (static_cast<int64_t>(a.T) + kAppendTokensPerWave - 1) / kAppendTokensPerWave * head_groups;
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
