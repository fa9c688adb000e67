// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Tokens per compute tile: the M (or K) extent of one 16x16 MFMA.
constexpr int kTile = 16;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kMaxGroup = 16;   // query heads per KV head served by one MFMA column tile
constexpr int kMaxLayers = 128; // copy_blocks pool pointers travel as kernel arguments

// Buffers of one decode call.  The kernels take them as separate __restrict__
// parameters so that reads of the block table and lengths become scalar loads.
struct DecodeBuffers {
  const uint16_t* q;        // bf16 [S][Hq][D]
  const uint16_t* k;        // K pool
  const uint16_t* v;        // V pool
  const int32_t* tables;    // int32 [S][M]
  const int32_t* lens;      // int32 [S]
  uint16_t* out;            // bf16 [S][Hq][D]
  float* ws;                // workspace: partial records, then per-worker descriptors
};

// Sizes of one decode call (passed by value).
struct DecodeDims {
  int32_t S, Hq, Hkv, G, M;
  int32_t n_workers;        // workers launched; the kernels use min(n_workers, units)
  int64_t NB;
  float c;                  // scale * log2(e): scores are kept in the log2 domain
};

// Floats in one partial record: O[G][D], then m[G], then l[G], padded to a
// multiple of four floats so every record starts 16-byte aligned.
__host__ __device__ inline int64_t record_floats(int G, int D) {
  return static_cast<int64_t>(G) * D + ((2 * G + 3) / 4) * 4;
}

// Workspace of a decode call: partial records ([n_workers][2][record_floats]),
// then one 16-byte descriptor per worker.
__host__ __device__ inline int64_t records_bytes(int64_t workers, int G, int D) {
  return workers * 2 * record_floats(G, D) * static_cast<int64_t>(sizeof(float));
}
inline int64_t workspace_bytes_for(int64_t workers, int G, int D) {
  return records_bytes(workers, G, D) + workers * 16;
}

// Launches the decode kernel and the merge kernel (pkv_decode.hip).  Returns a
// hipError_t.
hipError_t launch_decode(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                         int merge_groups, hipStream_t stream);

// KV append (pkv_append.hip).
struct AppendBuffers {
  const uint16_t* k_new;      // bf16 [T][Hkv][D]
  const uint16_t* v_new;      // bf16 [T][Hkv][D]
  uint16_t* k_cache;          // K pool
  uint16_t* v_cache;          // V pool
  const int32_t* tables;      // int32 [S][M]
  const int32_t* token_seq;   // int32 [T]
  const int32_t* token_pos;   // int32 [T]
};

struct AppendDims {
  int32_t T, S, Hkv, B, M;
  int64_t NB;
};

hipError_t launch_append(const AppendBuffers& b, const AppendDims& a, int D, hipStream_t stream);

// Launcher (pkv_copy.hip).
hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                              int32_t num_pairs, hipStream_t stream);

}  // namespace pkv
