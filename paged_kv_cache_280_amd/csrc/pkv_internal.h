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
// Positions one block-table row may address (max_blocks_per_seq * block_size): the
// work plan sums a row's work units in 32-bit lane scans.
constexpr int64_t kMaxRowPositions = int64_t(1) << 26;

// Buffers of one decode call.  The kernels take them as separate __restrict__
// parameters so that reads of the block table and lengths become scalar loads.
struct DecodeBuffers {
  const uint16_t* q;        // bf16 [S][Qmax][Hq][D], offset to the launch's first query token
  const void* k;            // K pool (bf16, or fp8 codes)
  const void* v;            // V pool
  const int32_t* tables;    // int32 [S][M]
  const int32_t* lens;      // int32 [S]
  const int32_t* qlens;     // int32 [S] query tokens per sequence (multi-token launches only)
  uint16_t* out;            // bf16, same layout and offset as q
  float* ws;                // workspace: partial records, then per-worker descriptors
  // decode-with-append launches only: each sequence's newest position, written into
  // its slot and attended to in the same launch
  const uint16_t* k_new;    // bf16 [S][Hkv][D]
  const uint16_t* v_new;    // bf16 [S][Hkv][D]
  void* kw;                 // the K pool (written: the new rows)
  void* vw;                 // the V pool
  // shared-prefix launches only: the prefix softmax states ([S][record_floats(Hq, D)])
  float* state;
};

// Sizes of one launch (passed by value).  A decode launch has one query token
// per sequence (Qmax = Qc = 1, q_off = 0, R = G).  A multi-token launch covers
// query tokens [q_off, q_off + Qc) of every sequence; each (sequence, KV head)
// pair then has R = G * Qc rows, row n being query token n / G of head n % G.
struct DecodeDims {
  int32_t S, Hq, Hkv, G, M;
  int32_t n_workers;        // workers launched; the kernels use min(n_workers, units)
  int64_t NB;
  float c;                  // scale * log2(e): scores are kept in the log2 domain
  int32_t Qmax;             // query-token stride of q and out
  int32_t Qc;               // query tokens of this launch
  int32_t q_off;            // first query token of this launch
  int32_t R;                // rows of a (sequence, KV head) pair: G * Qc
  float v_scale;            // multiplies the outputs (fp8 V pools; 1 for bf16)
  int32_t pair_mode;        // 1: worker w takes (sequence, KV head) pair w whole (no split,
                            // no records, no merge); n_workers = S * Hkv
  int32_t unit;             // work units of one tile (1, or 4 when pairs are weighted)
  int32_t hdr;              // work units of a pair's query and output rows
  int32_t len_off;          // 1 in decode-with-append launches: the tiles cover the first
                            // context_lens[s] - 1 positions, the newest comes from k_new/v_new
  float k_scale;            // fp8 decode-with-append: new K rows are stored as E4M3(x / k_scale)
  // shared-prefix launches: prefix lengths are used clamped into [0, min(M*B, pre_cap)]
  // and rounded down to a multiple of pre_align (max(16, B): whole tiles and blocks);
  // seqs is the batch's sequence count (the prefix pass runs over groups)
  int32_t pre_align, pre_cap, seqs;
  // Multi-token launches whose rows exceed one wave's column tiles: nch waves of a
  // work-group (2 or 4; 0 or 1: one) share each planned range of tiles, wave
  // `chunk` taking query tokens q_off + chunk*Qc .. + Qc - 1, so a K/V tile is read
  // from memory once for all of them.  n_workers counts the ranges (slots).
  int32_t nch, chunk;
  // Pool form: 1 for separate K and V pools; 2 when both are the halves of one pool
  // whose (block, head) entries hold the K tile and then the V tile (v = k + one
  // tile), so blocks and heads step over two tiles.
  int32_t kv_mul;
};

// Floats in one partial record: O[R][D], then m[R], then l[R], padded to a
// multiple of four floats so every record starts 16-byte aligned.
// Tiles one (block, head) entry of the pools spans: 2 in the paired form, else 1.
__host__ __device__ inline int64_t tile_span(int32_t kv_mul) { return kv_mul == 2 ? 2 : 1; }

__host__ __device__ inline int64_t record_floats(int R, int D) {
  return static_cast<int64_t>(R) * D + ((2 * R + 3) / 4) * 4;
}

// Workspace of a launch: partial records ([n_workers][2][record_floats]), then
// one 16-byte descriptor per worker.
__host__ __device__ inline int64_t records_bytes(int64_t workers, int R, int D) {
  return workers * 2 * record_floats(R, D) * static_cast<int64_t>(sizeof(float));
}

// Libraries built with PKV_TIMELINE (a measurement build, never the default) also
// leave one WorkerStamp per decode worker after the descriptors: when the worker
// entered the kernel, finished its plan, computed its first tile and finished, on
// the 100 MHz s_memrealtime clock, and where it ran.
struct WorkerStamp {
  uint64_t t_entry;
  uint32_t d_plan, d_first, d_end;  // ticks after t_entry (0xFFFFFFFF: no tile)
  uint32_t xcc;                     // XCC (chiplet) the wave ran on
  uint32_t tiles;                   // tiles of the worker's range
  uint32_t group;                   // work-group index
};
#ifdef PKV_TIMELINE
constexpr int64_t kStampBytes = sizeof(WorkerStamp);
#else
constexpr int64_t kStampBytes = 0;
#endif

inline int64_t workspace_bytes_for(int64_t workers, int R, int D) {
  return records_bytes(workers, R, D) + workers * (16 + kStampBytes);
}

// Rows one multi-token launch can hold: two 16-column MFMA tiles per wave.
constexpr int kMaxRows = 32;

// Launch the decode kernel and the merge kernel (kernels in pkv_decode_kernels.h,
// launches in pkv_decode*.hip).  Return a hipError_t.  launch_multi takes a
// multi-token launch (d.R <= kMaxRows) over bf16 or fp8 pools (fp8: launch_multi_fp8).
hipError_t launch_decode(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                         int merge_groups, hipStream_t stream);
hipError_t launch_multi(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                        int merge_groups, hipStream_t stream, bool fp8);
hipError_t launch_multi_fp8(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                            int merge_groups, hipStream_t stream);
// Decode over fp8 (E4M3FN) pools: d.c carries scale * k_scale * log2(e), d.v_scale
// the V pool's scale.
hipError_t launch_decode_fp8(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                             int merge_groups, hipStream_t stream);
// Shared-prefix decode over bf16 pools (pkv_decode_shared.hip).  launch_shared:
// the prefix pass over the sharing groups (a.R = G * largest group <= kMaxRows;
// bp.lens = prefix lengths, bp.qlens = group offsets) and the tail pass (bt.qlens =
// prefix lengths) in one launch, then the tail merge; both with the same state
// buffer, and gmap (2 int32 per sequence) for the prefix pass's member map.
// launch_shared_tail: the tail pass alone (no prefix anywhere).
hipError_t launch_shared(const DecodeBuffers& bp, const DecodeDims& a, const DecodeBuffers& bt,
                         const DecodeDims& d, int D, int B, int32_t* gmap, int merge_groups_tail,
                         hipStream_t stream);
hipError_t launch_shared_tail(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                              int merge_groups, hipStream_t stream);
// Decode with append (d.len_off = 1; b.k_new, v_new, kw, vw set), bf16 pools.
hipError_t launch_decode_append(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                                int merge_groups, hipStream_t stream);

// KV append (pkv_append.hip).
struct AppendBuffers {
  const uint16_t* k_new;      // bf16 [T][Hkv][D]
  const uint16_t* v_new;      // bf16 [T][Hkv][D]
  void* k_cache;              // K pool (bf16, or fp8 codes)
  void* v_cache;              // V pool
  const int32_t* tables;      // int32 [S][M]
  const int32_t* token_seq;   // int32 [T]
  const int32_t* token_pos;   // int32 [T]
};

struct AppendDims {
  int32_t T, S, Hkv, B, M;
  int64_t NB;
  float k_scale, v_scale;     // fp8 pools: stored code = E4M3(x / scale)
  int32_t newest;             // 1: token t is sequence t's newest position, and token_pos
                              // holds the context lengths (position = length - 1)
  int32_t kv_mul;             // pool form, as in DecodeDims
};

hipError_t launch_append(const AppendBuffers& b, const AppendDims& a, int D, hipStream_t stream);
hipError_t launch_append_fp8(const AppendBuffers& b, const AppendDims& a, int D,
                             hipStream_t stream);

// Table-contract check (pkv_check.hip): S sequences, M entries per table row,
// block size B, NB pool blocks, Qmax query rows per sequence (multi-token).
struct CheckDims {
  int32_t S, M, B, Qmax;
  int64_t NB;
};

hipError_t launch_check(const int32_t* tables, const int32_t* lens, const int32_t* qlens,
                        int32_t* result, const CheckDims& c, hipStream_t stream);

// Launcher (pkv_copy.hip).
hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                              int32_t num_pairs, hipStream_t stream);

}  // namespace pkv
