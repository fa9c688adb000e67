// Paged decode attention for gfx950 (CDNA4): block-table walk, MFMA scores,
// online softmax, MFMA value accumulation, split-K across persistent workers and a
// deterministic merge of split (sequence, KV head) pairs.
//
// What is computed: "KV cache, PagedAttention" (aiwiki.vn), paragraph on query, key
// and value -- the query of the current position scores every cached key, and the
// softmax of the scores weights the cached values.  Where the K/V rows are: a
// per-sequence block table maps logical block j to a physical block of B tokens
// anywhere in the pool ("PagedAttention (vLLM)", troisinh.com, section "Cơ chế
// Block Table"); the kernel gathers the rows it needs by walking that table (same
// page, section "Tại sao nó hoạt động").
//
// Work decomposition.  Work is counted over the 16-token tiles of the (sequence,
// KV head) pairs, numbered sequence-major, then KV head, then tile, and the N
// workers (one wave each) take equal contiguous ranges of that count, so every
// worker streams about the same bytes whatever the mix of context lengths (batches
// of more than 64 sequences also count each pair's query and output rows).  A
// worker's range is cut into segments at (sequence, head) boundaries.
// A segment that covers a whole pair writes the output directly; a segment that
// covers part of a pair writes its softmax state (reference max m, sum l,
// unnormalised accumulator O; fp32) to the workspace; a second kernel merges the
// states of each split pair in worker order (deterministic result).
//
// Per tile (one wave, 16 tokens x D dims, up to 16 query heads of one KV head):
//   scores  S[token][head] = K_tile (16 x D) * q^T (D x 16)  -- D/32 MFMA 16x16x32 bf16
//   weights p = exp2(S*scale*log2e - m), m a per-head reference max shared by the
//           four lanes holding that head; m moves up (and O, l are rescaled) only
//           when a score exceeds it by more than 2^8, so p <= 256 and the
//           cross-lane max runs only on those rare tiles; p rounded to bf16
//   values  O^T[dim][head] += V_tile^T (D x 16) * P^T (16 x 16) -- D/16 MFMA 16x16x16
//   sum     l[head] += sum_t P[head][t] -- one more MFMA against a block of ones,
//           so l adds exactly the bf16 weights that O used
// The pool layouts put each lane's MFMA operand in 16 (K) or 8 (V) contiguous
// bytes, so tiles go from HBM straight into operand registers with coalesced
// loads, and the score MFMA's output registers are already the weight operand of
// the value MFMA (no shuffles, no LDS).  Loads run kPipe-1 tiles ahead of the
// arithmetic through the worker's whole range, across segment boundaries.
//
// Multi-token launches (a prefill chunk, or the draft tokens a speculative step
// verifies: "vLLM PagedAttention: Bước đột phá về thông lượng suy luận LLM",
// vi.news.hada.io, list of advanced features).  A sequence's query tokens are its
// last T positions; query token i sits at position L - T + i and sees positions
// 0 .. L - T + i.  The MFMA columns then hold (query token, head) rows of the
// pair, one or two 16-column tiles per wave, each column with its own position
// limit; every K/V tile is loaded once for all of them.  A pair's tiles stop at
// the last position its last query token sees.
//
// fp8 pools ("KV cache, PagedAttention", aiwiki.vn, paragraph on cache
// quantisation): one-byte E4M3FN codes, loaded 16 bytes per lane and widened
// exactly to bf16 for the same MFMAs; the K pool's scale folds into the score
// factor and the V pool's into the output, so nothing is scaled per element.
//
// Pair mode (short contexts): worker w takes pair w whole, so nothing is split and
// no merge runs.
//
// Decode with append: the tiles cover all but each sequence's newest position,
// which the worker holding the pair's last tile adds from the new rows and writes
// into its slot (one launch for the append and the attention over it).

#pragma once

#include <math.h>

#include <type_traits>

#include "pkv_fp8.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Tile buffers in registers (kPipe-1 loads in flight).  Two column tiles of
// 128-dim rows leave room for two buffers only.  fp8 tiles run best with two
// buffers too (measured: fewer registers, 200 VGPRs at D = 128, beat deeper
// pipelines on every workload).
template <int D, int NC, bool kFp8>
constexpr int pipe_depth() {
  return (kFp8 || (NC == 2 && D == 128)) ? 2 : 3;
}
constexpr float kRescaleThreshold = 8.0f;  // log2 units: weights stay below 2^8

__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int32_t tiles_of(int32_t L) { return (L + kTile - 1) / kTile; }

__device__ __forceinline__ int32_t clamp_block(int32_t b, int64_t nb) {
  return b < 0 ? 0 : (b >= nb ? static_cast<int32_t>(nb - 1) : b);
}

// K/V tile loads carry the non-temporal hint: every K/V byte of a call is read once,
// so its lines are not kept in L2 or the last-level cache in place of the records,
// tables and queries that are read again.  Measured against plain loads (same box,
// graph-replayed): long context 97.6-100.6 -> 90.6-91.5 us per call, mix 368-378 ->
// 345-356 us, chat 46.4 -> 42.9 us.
template <typename V, typename T>
__device__ __forceinline__ V stream_load(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS traffic):
// doubling shifts within each row of 16 lanes, then each row's running total
// broadcast into the rows after it (lane 15 into rows 1 and 3, lane 31 into rows
// 2 and 3).  Out-of-row sources of the shifts read 0.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xC, 0xF, false);
  return x;
}

// Context a launch processes for sequence s.  Decode: L = context_lens[s], one
// query token.  Multi-token launch: the sequence's query tokens are its last
// T = query_lens[s] positions (T clamped into [0, min(L, Qmax)]); the launch
// takes the Tc of them in [q_off, q_off + Qc), and its context ends at the
// position the last of those sees, so L_c = L - T + q_off + Tc (0 when Tc = 0).
//
// Shared-prefix launches (kShare != 0) run in two passes.  The prefix pass
// (kShare = 1, a multi-token launch) takes group v of sequences first ..
// first + T - 1 (first = qlens[v], T = qlens[v+1] - first clamped into [0, Qmax]:
// qlens holds the group offsets) as one set of rows: its context is the first
// P positions of the group's first sequence, P = prefix_positions(lens[first])
// (lens holds the per-sequence prefix lengths).  The tail pass (kShare = 2, a
// decode launch) takes sequence s from position P = prefix_positions(qlens[s])
// on (qlens holds the prefix lengths): L = context_lens[s] - P.  x is `first` in
// the prefix pass and P in the tail pass; in multi-token launches it is the
// position offset of the wave's query tokens (seq_len).
struct SeqLen {
  int32_t L, T, x;
};

// Positions of a shared prefix as the launches use them: clamped into
// [0, min(cap, d.pre_cap)] and rounded down to a whole number of tiles and blocks
// (d.pre_align).
__device__ __forceinline__ int32_t prefix_positions(int32_t p, const DecodeDims& d, int32_t cap) {
  const int32_t c = clamp_len(p, min(cap, d.pre_cap));
  return c - c % d.pre_align;
}

template <bool kCausal, int kShare = 0>
__device__ __forceinline__ SeqLen seq_len(const int32_t* __restrict__ lens,
                                          const int32_t* __restrict__ qlens, const DecodeDims& d,
                                          int32_t cap, int32_t s) {
  if constexpr (kShare == 1) {
    const int32_t first = min(max(qlens[s], 0), d.seqs - 1);
    const int32_t T = clamp_len(qlens[s + 1] - first, min(d.Qmax, d.seqs - first));
    return SeqLen{T > 0 ? prefix_positions(lens[first], d, cap) : 0, T, first};
  }
  // decode with append: the tiles cover all but the newest position
  const int32_t L = max(clamp_len(lens[s], cap) - d.len_off, 0);
  if constexpr (kShare == 2) {
    const int32_t P = prefix_positions(qlens[s], d, cap);
    return SeqLen{max(L - P, 0), 1, P};
  } else if constexpr (!kCausal) {
    return SeqLen{L, 1};
  } else {
    // every chunk of the launch plans over the context its last token sees,
    // L_c = L - T + hi; this wave's tokens start at qoc and x = hi - qoc, so its
    // token i (query token qoc + i, at position L - T + qoc + i) sees positions
    // up to L_c - x + i
    const int32_t T = clamp_len(qlens[s], min(L, d.Qmax));
    const int32_t qoc = d.q_off + d.chunk * d.Qc;
    const int32_t hi = min(T, d.q_off + max(d.nch, 1) * d.Qc);
    if (hi <= d.q_off) return SeqLen{0, 0, 0};
    return SeqLen{L - T + hi, clamp_len(T - qoc, d.Qc), hi - qoc};
  }
}

// Work units.  A tile of a (sequence, KV head) pair counts d.unit units and each
// pair d.hdr more (its query and output rows, with d.unit = 4 in quarters of a
// tile's K/V bytes, plus a fixed share for starting and closing a pair), so ranges
// of equal units carry about equal work however many pairs they hold.  The pairs of sequence s follow each other in head order:
// pair (s, g) spans units [start_s + g*P_s, start_s + (g+1)*P_s), P_s =
// unit*T_s + hdr, and its tile t sits at unit start_s + g*P_s + hdr + unit*t.
// Empty sequences hold no units.  A worker owns the tiles whose unit lies in its
// range.  Launches over at most 64 sequences use unit 1 and hdr 0 (units are
// tiles), which keeps the plan to one scan and one lookup.
__device__ __forceinline__ int32_t pair_units(int32_t T, const DecodeDims& d) {
  return T > 0 ? d.unit * T + d.hdr : 0;
}

// Range of worker w: units [w*U/N, (w+1)*U/N) (range_of below).  worker_of(u) is
// the largest w whose range starts at or before u.
__device__ __forceinline__ int64_t worker_of(int64_t u, int64_t U, int64_t N) {
  return ((u + 1) * N - 1) / U;
}

// Per-lane view of 64 consecutive sequences base + lane: their SeqLen (L, Tq),
// tiles T, pair units P, and inclusive scans of T and P (zeros past the batch).
struct Chunk {
  int32_t base, L, Tq, T, P, incT, incP;
};

template <bool kCausal, int kShare = 0>
__device__ __forceinline__ SeqLen lane_len(const int32_t* __restrict__ lens,
                                           const int32_t* __restrict__ qlens, const DecodeDims& d,
                                           int32_t cap, int32_t base, int lane) {
  return base + lane < d.S ? seq_len<kCausal, kShare>(lens, qlens, d, cap, base + lane)
                           : SeqLen{0, 0, 0};
}

// One shuffle scan: the unit scan follows from the tile scan and the count of
// non-empty sequences up to this lane.
__device__ __forceinline__ Chunk make_chunk(int32_t base, SeqLen sl, const DecodeDims& d,
                                            int lane) {
  Chunk c;
  c.base = base;
  c.L = sl.L;
  c.Tq = sl.T;
  const int32_t T = tiles_of(sl.L);
  c.T = T;
  c.P = pair_units(T, d);
  c.incT = wave_inclusive_scan(c.T);
  const uint64_t upto = lane == kWave - 1 ? ~0ull : ((1ull << (lane + 1)) - 1);
  c.incP = d.unit * c.incT + d.hdr * __builtin_popcountll(__ballot(T > 0) & upto);
  return c;
}

// Where unit x falls (x at or past the chunk's first unit acc_u): false when x
// lies past the chunk.  Otherwise the sequence s holding x, the first unit and
// the first tile (index over the whole batch) of s, the tiles of s, and the first
// tile of s at or after x as (g, t), g = Hkv when x lies past the last tile of s.
struct UnitLoc {
  int32_t s, g, t, T, P, L, Tq;
  int64_t start, tstart;
};

__device__ __forceinline__ bool locate_in(const Chunk& c, const DecodeDims& d, int64_t acc_u,
                                          int64_t acc_t, int64_t x, UnitLoc& r) {
  const int64_t chunk_u = static_cast<int64_t>(__builtin_amdgcn_readlane(c.incP, kWave - 1)) * d.Hkv;
  if (x >= acc_u + chunk_u) return false;
  const uint64_t hit = __ballot(acc_u + static_cast<int64_t>(c.incP) * d.Hkv > x);
  const int32_t i = uniform(__builtin_ctzll(hit));
  r.s = c.base + i;
  r.L = __builtin_amdgcn_readlane(c.L, i);
  r.Tq = __builtin_amdgcn_readlane(c.Tq, i);
  r.T = __builtin_amdgcn_readlane(c.T, i);
  r.P = __builtin_amdgcn_readlane(c.P, i);
  r.start = acc_u + static_cast<int64_t>(__builtin_amdgcn_readlane(c.incP, i) - r.P) * d.Hkv;
  r.tstart = acc_t + static_cast<int64_t>(__builtin_amdgcn_readlane(c.incT, i) - r.T) * d.Hkv;
  const int64_t rel = x - r.start;
  r.g = rel < (int64_t(1) << 31) ? static_cast<int32_t>(rel) / r.P : static_cast<int32_t>(rel / r.P);
  const int32_t off = static_cast<int32_t>(rel - static_cast<int64_t>(r.g) * r.P);
  r.t = off <= d.hdr ? 0 : (off - d.hdr + d.unit - 1) / d.unit;
  if (r.t >= r.T) {
    ++r.g;
    r.t = 0;
  }
  return true;
}

// Index over the whole batch of the first tile at or after the located unit.
__device__ __forceinline__ int64_t first_tile(const UnitLoc& r) {
  return r.tstart + static_cast<int64_t>(r.g) * r.T + r.t;
}

// A worker's share of the batch: total units U, active workers N, the first tile
// (s, g, t) of its range, the first unit `start` and the SeqLen (L, Tq) of s, and
// its tile count n.
struct WorkerPlan {
  int64_t U, N, start;
  int32_t s, g, t, n, L, Tq;
};

// Chunks of the batch's sequences held in registers (the rest are read again on
// every pass): one read of the lengths and one scan serve every pass up to 256
// sequences.
constexpr int kPlanChunks = 4;

// Passes over the chunks in order: f(chunk, acc_u, acc_t) returns true to stop.
template <bool kCausal, int kShare = 0, typename F>
__device__ __forceinline__ void for_chunks(const int32_t* __restrict__ lens,
                                           const int32_t* __restrict__ qlens,
                                           const DecodeDims& d, int32_t cap,
                                           const Chunk (&ch)[kPlanChunks], int lane, F&& f) {
  int64_t acc_u = 0, acc_t = 0;
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k) {
    if (k * kWave >= d.S) return;
    const Chunk& c = ch[k];
    if (f(c, acc_u, acc_t)) return;
    acc_u += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incP, kWave - 1)) * d.Hkv;
    acc_t += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incT, kWave - 1)) * d.Hkv;
  }
  for (int32_t base = kPlanChunks * kWave; base < d.S; base += kWave) {
    const Chunk c =
        make_chunk(base, lane_len<kCausal, kShare>(lens, qlens, d, cap, base, lane), d, lane);
    if (f(c, acc_u, acc_t)) return;
    acc_u += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incP, kWave - 1)) * d.Hkv;
    acc_t += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incT, kWave - 1)) * d.Hkv;
  }
}

// Ends of worker w's range, [w*U/N, (w+1)*U/N), with 32-bit divisions whenever
// the operands fit (U = q*N + r, so w*U/N = w*q + r*w/N).
__device__ __forceinline__ void range_of(int64_t w, int64_t U, int64_t N, int64_t& u, int64_t& ue) {
  const bool small = U < (int64_t(1) << 32) && N < (int64_t(1) << 16);
  const int64_t q = small ? static_cast<uint32_t>(U) / static_cast<uint32_t>(N) : U / N;
  const int64_t r = U - q * N;  // < N
  if (small) {
    u = w * q + static_cast<uint32_t>(r * w) / static_cast<uint32_t>(N);
    ue = (w + 1) * q + static_cast<uint32_t>(r * (w + 1)) / static_cast<uint32_t>(N);
  } else {
    u = w * q + r * w / N;
    ue = (w + 1) * q + r * (w + 1) / N;
  }
}

// Returns false when worker w has no tile.
template <bool kCausal, int kShare = 0>
__device__ bool plan_worker(const int32_t* __restrict__ lens, const int32_t* __restrict__ qlens,
                            const DecodeDims& d, int32_t cap, int64_t w, int lane, WorkerPlan& p) {
  if (d.S <= kWave) {  // units are tiles: one scan, one lookup
    const SeqLen sl = lane_len<kCausal, kShare>(lens, qlens, d, cap, 0, lane);
    const int32_t T = tiles_of(sl.L);
    const int32_t incl = wave_inclusive_scan(T);
    p.U = static_cast<int64_t>(__builtin_amdgcn_readlane(incl, kWave - 1)) * d.Hkv;
    p.N = min(static_cast<int64_t>(d.n_workers), p.U);
    if (w >= p.N) return false;
    int64_t u, ue;
    range_of(w, p.U, p.N, u, ue);
    const uint64_t hit = __ballot(static_cast<int64_t>(incl) * d.Hkv > u);
    const int32_t i = uniform(__builtin_ctzll(hit));
    p.s = i;
    p.L = __builtin_amdgcn_readlane(sl.L, i);
    p.Tq = __builtin_amdgcn_readlane(sl.T, i);
    const int32_t Ts = __builtin_amdgcn_readlane(T, i);
    p.start = static_cast<int64_t>(__builtin_amdgcn_readlane(incl, i) - Ts) * d.Hkv;
    const int64_t rel = u - p.start;
    p.g = rel < (int64_t(1) << 31) ? static_cast<int32_t>(rel) / Ts : static_cast<int32_t>(rel / Ts);
    p.t = static_cast<int32_t>(rel - static_cast<int64_t>(p.g) * Ts);
    p.n = static_cast<int32_t>(ue - u);
    return true;
  }
  SeqLen T0[kPlanChunks];  // all lengths read first: one round trip
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k)
    T0[k] = lane_len<kCausal, kShare>(lens, qlens, d, cap, k * kWave, lane);
  Chunk Tc[kPlanChunks];
#pragma unroll
  for (int k = 0; k < kPlanChunks; ++k)
    if (k * kWave < d.S) Tc[k] = make_chunk(k * kWave, T0[k], d, lane);
  // pass 1: total units and tiles
  int64_t U = 0, tiles = 0;
  for_chunks<kCausal, kShare>(lens, qlens, d, cap, Tc, lane, [&](const Chunk& c, int64_t, int64_t) {
    U += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incP, kWave - 1)) * d.Hkv;
    tiles += static_cast<int64_t>(__builtin_amdgcn_readlane(c.incT, kWave - 1)) * d.Hkv;
    return false;
  });
  p.U = U;
  p.N = min(static_cast<int64_t>(d.n_workers), tiles);  // every range >= d.unit units
  if (w >= p.N) return false;
  int64_t u, ue;
  range_of(w, p.U, p.N, u, ue);
  // pass 2: where the range starts and ends
  UnitLoc lu, le;
  bool found_u = false, found_e = ue >= U;
  int64_t first = 0, last = tiles;
  for_chunks<kCausal, kShare>(lens, qlens, d, cap, Tc, lane, [&](const Chunk& c, int64_t au, int64_t at) {
    if (!found_u && locate_in(c, d, au, at, u, lu)) {
      found_u = true;
      first = first_tile(lu);
    }
    if (!found_e && locate_in(c, d, au, at, ue, le)) {
      found_e = true;
      last = first_tile(le);
    }
    return found_u && found_e;
  });
  if (!found_u || last <= first) return false;
  p.n = static_cast<int32_t>(last - first);
  if (lu.g >= d.Hkv) {
    // u lies past the last tile of its sequence: the range starts at the next
    // sequence that holds units
    const int64_t next = lu.start + static_cast<int64_t>(lu.P) * d.Hkv;
    for_chunks<kCausal, kShare>(lens, qlens, d, cap, Tc, lane, [&](const Chunk& c, int64_t au, int64_t at) {
      return locate_in(c, d, au, at, next, lu);
    });
  }
  p.s = lu.s;
  p.g = lu.g;
  p.t = lu.t;
  p.L = lu.L;
  p.Tq = lu.Tq;
  p.start = lu.start;
  return true;
}

// Where one (sequence, KV head) pair's tiles come from (T: pool element type).
template <typename T>
struct PairCursor {
  const T* k;               // K pool
  const T* v;               // V pool
  const int32_t* trow;      // block-table row of the sequence
  int64_t head_off;         // g * (elements of one (block, head) tile)
  int64_t block_stride;     // elements of one block (all heads)
  int64_t nb;
  int32_t nblk;             // ceil(L / B)
};

// Pair mode: worker w takes (sequence w / Hkv, KV head w % Hkv) whole.  Returns
// false for workers past the pairs and for empty sequences.
template <bool kCausal, int kShare = 0>
__device__ bool plan_pair(const int32_t* __restrict__ lens, const int32_t* __restrict__ qlens,
                          const DecodeDims& d, int32_t cap, int64_t w, WorkerPlan& p) {
  if (w >= static_cast<int64_t>(d.S) * d.Hkv) return false;
  const int32_t s = static_cast<int32_t>(w / d.Hkv);
  const int32_t g = static_cast<int32_t>(w - static_cast<int64_t>(s) * d.Hkv);
  const SeqLen sl = seq_len<kCausal, kShare>(lens, qlens, d, cap, s);
  const int32_t T = tiles_of(sl.L);
  if (T == 0) return false;
  p.L = sl.L;
  p.Tq = sl.T;
  p.U = 1;  // only used to find the workers of split pairs, and none is split
  p.N = 1;
  p.start = 0;
  p.s = s;
  p.g = g;
  p.t = 0;
  p.n = T;
  return true;
}

// A tile of bf16 K/V in registers: every lane's MFMA operands, as loaded.
template <int D, int B>
struct Bf16Tile {
  using Elem = uint16_t;
  u32x4_t k[D / 32];  // score MFMA A operand: token lane%16, dims c*32 + (lane/16)*8 .. +7
  u32x2_t v[D / 16];  // value MFMA A operand: dim mt*16 + lane%16, tokens (lane/16)*4 .. +3

  // Issue the loads of tile t.
  __device__ __forceinline__ void load(const PairCursor<Elem>& pc, int32_t t, int lane) {
    const int32_t tok0 = t * kTile;
    if constexpr (B >= kTile) {
      const int32_t b = clamp_block(pc.trow[tok0 / B], pc.nb);
      const int32_t ob = tok0 % B;
      const int64_t base = static_cast<int64_t>(b) * pc.block_stride + pc.head_off;
      const uint16_t* kt = pc.k + base;
      // V keeps each 16-position half of a block as its own [D][16] run
      const uint16_t* vt = pc.v + base + (ob / kTile) * D * kTile;
      const uint32_t koff = static_cast<uint32_t>(((lane >> 4) * B + ob + (lane & 15)) * 8);
      const uint32_t voff = static_cast<uint32_t>((lane & 15) * kTile + (lane >> 4) * 4);
#pragma unroll
      for (int c = 0; c < D / 32; ++c) k[c] = stream_load<u32x4_t>(kt + koff + c * 4 * B * 8);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) v[mt] = stream_load<u32x2_t>(vt + voff + mt * 16 * kTile);
    } else {
      // B == 8: the tile spans logical blocks 2t and 2t+1 (the second clamped to
      // the sequence's last block; its lanes are masked when it lies past the
      // context).
      static_assert(B == 8, "block sizes below 16 other than 8 are not built");
      const int32_t j0 = tok0 / B;
      const int32_t j1 = j0 + 1 < pc.nblk ? j0 + 1 : pc.nblk - 1;
      const int64_t base0 = static_cast<int64_t>(clamp_block(pc.trow[j0], pc.nb)) * pc.block_stride;
      const int64_t base1 = static_cast<int64_t>(clamp_block(pc.trow[j1], pc.nb)) * pc.block_stride;
      const int64_t kb = ((lane & 15) < 8 ? base0 : base1) + pc.head_off;
      const int64_t vb = ((lane >> 4) < 2 ? base0 : base1) + pc.head_off;
      const uint16_t* kt = pc.k + kb + ((lane >> 4) * B + (lane & 7)) * 8;
      const uint16_t* vt = pc.v + vb + (lane & 15) * B + ((lane >> 4) & 1) * 4;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) k[c] = stream_load<u32x4_t>(kt + c * 4 * B * 8);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) v[mt] = stream_load<u32x2_t>(vt + mt * 16 * B);
    }
  }
  __device__ __forceinline__ bf16x8_t kop(int cc) const { return __builtin_bit_cast(bf16x8_t, k[cc]); }
  __device__ __forceinline__ u32x2_t vop(int mt) const { return v[mt]; }
  // Keep the first n of this lane's four tokens (the others lie past the context).
  __device__ __forceinline__ void mask_v(int32_t n) {
    const uint64_t keep = n >= 4 ? ~0ull : (n <= 0 ? 0ull : ((1ull << (16 * n)) - 1));
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      v[mt].x &= static_cast<uint32_t>(keep);
      v[mt].y &= static_cast<uint32_t>(keep >> 32);
    }
  }
};

// Two E4M3FN codes (word kHi of x) as two bf16 numbers, exactly: every E4M3
// value is a bf16 value, and the conversion's scale is 1.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, kHi));
}

// A tile of fp8 K/V in registers (one byte per element, 16-byte loads); the
// operands are widened to bf16 when the MFMAs need them.  The score MFMA's
// reduction runs over a permutation of the head dimension: MFMA cc at lane group
// gq = lane/16 takes dims (cc/2)*64 + gq*16 + (cc%2)*8 .. +7 (the query uses the
// same permutation).
template <int D, int B>
struct Fp8Tile {
  using Elem = uint8_t;
  u32x4_t k[D / 64];  // token lane%16, dims c*64 + (lane/16)*16 .. +15
  u32x4_t v[D / 64];  // dims (4i + jj)*16 + lane%16 (dword jj), tokens (lane/16)*4 .. +3

  __device__ __forceinline__ void load(const PairCursor<Elem>& pc, int32_t t, int lane) {
    const int32_t tok0 = t * kTile;
    const uint8_t* kt;
    const uint8_t* vt;
    if constexpr (B >= kTile) {
      const int32_t b = clamp_block(pc.trow[tok0 / B], pc.nb);
      const int32_t ob = tok0 % B;
      const int64_t base = static_cast<int64_t>(b) * pc.block_stride + pc.head_off;
      kt = pc.k + base + ((lane >> 4) * B + ob + (lane & 15)) * 16;
      vt = pc.v + base + ((lane & 15) * (B / 4) + ob / 4 + (lane >> 4)) * (D / 16) * 4;
    } else {
      static_assert(B == 8, "block sizes below 16 other than 8 are not built");
      const int32_t j0 = tok0 / B;
      const int32_t j1 = j0 + 1 < pc.nblk ? j0 + 1 : pc.nblk - 1;
      const int64_t base0 = static_cast<int64_t>(clamp_block(pc.trow[j0], pc.nb)) * pc.block_stride;
      const int64_t base1 = static_cast<int64_t>(clamp_block(pc.trow[j1], pc.nb)) * pc.block_stride;
      const int64_t kb = ((lane & 15) < 8 ? base0 : base1) + pc.head_off;
      const int64_t vb = ((lane >> 4) < 2 ? base0 : base1) + pc.head_off;
      kt = pc.k + kb + ((lane >> 4) * B + (lane & 7)) * 16;
      vt = pc.v + vb + ((lane & 15) * (B / 4) + ((lane >> 4) & 1)) * (D / 16) * 4;
    }
#pragma unroll
    for (int c = 0; c < D / 64; ++c) k[c] = stream_load<u32x4_t>(kt + c * 4 * B * 16);
#pragma unroll
    for (int i = 0; i < D / 64; ++i) v[i] = stream_load<u32x4_t>(vt + i * 16);
  }
  __device__ __forceinline__ bf16x8_t kop(int cc) const {
    const u32x4_t w = k[cc / 2];
    const uint32_t a = (cc & 1) ? w.z : w.x;
    const uint32_t b = (cc & 1) ? w.w : w.y;
    const u32x4_t r = {e4m3x2_to_bf16x2<false>(a), e4m3x2_to_bf16x2<true>(a),
                       e4m3x2_to_bf16x2<false>(b), e4m3x2_to_bf16x2<true>(b)};
    return __builtin_bit_cast(bf16x8_t, r);
  }
  __device__ __forceinline__ u32x2_t vop(int mt) const {
    const uint32_t w = v[mt / 4][mt % 4];
    return u32x2_t{e4m3x2_to_bf16x2<false>(w), e4m3x2_to_bf16x2<true>(w)};
  }
  // Keep the first n of this lane's four tokens: code 0 is +0.
  __device__ __forceinline__ void mask_v(int32_t n) {
    const uint32_t keep = n >= 4 ? ~0u : (n <= 0 ? 0u : ((1u << (8 * n)) - 1));
#pragma unroll
    for (int i = 0; i < D / 64; ++i) v[i] &= keep;
  }
};

template <int D, int B, bool kFp8>
using TileOf = typename std::conditional<kFp8, Fp8Tile<D, B>, Bf16Tile<D, B>>::type;

// Softmax state of one wave's column tile over one segment.
template <int D>
struct SegState {
  f32x4_t o[D / 16];  // O^T[dim mt*16 + (lane/16)*4 + i][column lane%16]
  f32x4_t l;          // every entry: sum of the bf16 weights of column lane%16
  float m;            // reference max of column lane%16 (log2 domain)
};

// Column n = j*16 + lane%16 of column tile j is row n of a (sequence, KV head)
// pair: query token qi = n / G of head n % G.  `row` is the offset of its q and
// out row from the pair's first row (qi*Hq + n % G), or -1 when n >= R.
template <int NC>
struct Cols {
  int32_t qi[NC];
  int32_t row[NC];
};

template <int NC, bool kCausal>
__device__ __forceinline__ Cols<NC> make_cols(const DecodeDims& d, int lane) {
  Cols<NC> cl;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int32_t n = j * 16 + (lane & 15);
    if constexpr (kCausal) {
      const int32_t qi = n / d.G;
      cl.qi[j] = qi;
      cl.row[j] = n < d.R ? qi * d.Hq + (n - qi * d.G) : -1;
    } else {  // one query token: R = G
      cl.qi[j] = 0;
      cl.row[j] = n < d.G ? n : -1;
    }
  }
  return cl;
}

// One tile for NC column tiles: scores, softmax weights, value and sum
// accumulation.  `valid` is the number of tokens of the tile inside the context
// (16 except in the last tile).  Multi-token launches also mask by position:
// column j of this lane sees the tile's tokens 0 .. lim[j], and lim_lo is the
// smallest lim of the wave (nothing is masked by position when lim_lo >= 15).
template <int D, int NC, bool kCausal, typename Tile>
__device__ __forceinline__ void compute_tile(Tile& r, const bf16x8_t (&qop)[NC][D / 32],
                                             SegState<D> (&st)[NC], float c, int32_t valid,
                                             int32_t lim_lo, const int32_t (&lim)[NC], int lane) {
  f32x4_t sc[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    sc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < D / 32; ++cc)
      sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.kop(cc), qop[j][cc], sc[j], 0, 0, 0);
  }
  const int32_t tq = (lane >> 4) * 4;  // first of the four tokens this lane scores
  float x[NC][4];
#pragma unroll
  for (int j = 0; j < NC; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[j][i] = fmaf(sc[j][i], c, -st[j].m);
  if constexpr (kCausal) {
    if (lim_lo < kTile - 1) {
#pragma unroll
      for (int j = 0; j < NC; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tq + i > lim[j]) x[j][i] = -INFINITY;
    }
  } else {
    if (valid < kTile) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tq + i >= valid) x[0][i] = -INFINITY;
    }
  }
  // V rows past the context are zeroed: their slots may hold anything
  if (valid < kTile) r.mask_v(valid - tq);
  bool over = false;
#pragma unroll
  for (int j = 0; j < NC; ++j)
    over = over || x[j][0] > kRescaleThreshold || x[j][1] > kRescaleThreshold ||
           x[j][2] > kRescaleThreshold || x[j][3] > kRescaleThreshold;
  if (__ballot(over)) {
    // Move the reference max of every column up to its max over everything seen
    // so far (always taken on a segment's first tile, where m = -inf and x = +inf).
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool masked = kCausal ? tq + i > lim[j] : (valid < kTile && tq + i >= valid);
        sv[i] = masked ? -INFINITY : sc[j][i] * c;
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(st[j].m, mx);
      // a column that has seen no position yet keeps m = -inf and weights 0
      const float m_ref = (kCausal && m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(st[j].m - m_ref);
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) st[j].o[mt] *= alpha;
      st[j].l *= alpha;
      st[j].m = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[j][i] = sv[i] - m_ref;
    }
  }
  const bf16x4_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                         static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    bf16x4_t pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) pb[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(x[j][i]));
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      st[j].o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          __builtin_bit_cast(bf16x4_t, r.vop(mt)), pb, st[j].o[mt], 0, 0, 0);
    st[j].l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, st[j].l, 0, 0, 0);
  }
}

template <typename T>
struct Ctx {
  const uint16_t* __restrict__ q;
  const T* __restrict__ k;
  const T* __restrict__ v;
  const int32_t* __restrict__ tables;
  const int32_t* __restrict__ lens;
  const int32_t* __restrict__ qlens;
  uint16_t* __restrict__ out;
  float* __restrict__ ws;
  const uint16_t* __restrict__ k_new;  // decode with append: the newest rows, bf16 [S][Hkv][D]
  const uint16_t* __restrict__ v_new;
  T* kw;                               // the pools, written (the newest rows)
  T* vw;
  float* __restrict__ state;           // shared-prefix launches: prefix softmax states
  int4* desc;                          // descriptors (shared-prefix passes add pair descriptors)
  int32_t* gmap;                       // prefix pass: per sequence, its group and member index
};

// Position in a worker's stream of tiles: tile t of (sequence s, KV head g); L
// and T are the context and tile count of s in this launch, Tq its query tokens,
// `start` the first unit of s.
struct Cursor {
  int64_t start;
  int32_t s, g, t, T, L, Tq;
  int32_t x;  // shared-prefix launches: SeqLen::x of s
};

template <bool kCausal, int kShare = 0, typename Cx>
__device__ __forceinline__ void advance(Cursor& c, const Cx& cx, const DecodeDims& d,
                                        int32_t cap) {
  if (++c.t < c.T) return;
  c.t = 0;
  if (++c.g < d.Hkv) return;
  c.g = 0;
  c.start += static_cast<int64_t>(d.Hkv) * pair_units(c.T, d);
  do {
    ++c.s;
    if (c.s < d.S) {
      const SeqLen sl = seq_len<kCausal, kShare>(cx.lens, cx.qlens, d, cap, c.s);
      c.L = sl.L;
      c.Tq = sl.T;
      if constexpr (kShare != 0 || kCausal) c.x = sl.x;
    } else {
      c.L = 1;  // past the batch only at the very end
      c.Tq = 1;
    }
  } while (c.L == 0);
  c.T = tiles_of(c.L);
}

// Block-table entries of a pair's tiles: row s; the prefix pass reads the row of
// the group's first sequence, the tail pass skips the prefix's blocks.
template <int B, int kShare>
__device__ __forceinline__ int64_t table_offset(const DecodeDims& d, const Cursor& c) {
  if constexpr (kShare == 1) return static_cast<int64_t>(c.x) * d.M;
  if constexpr (kShare == 2) return static_cast<int64_t>(c.s) * d.M + c.x / B;
  return static_cast<int64_t>(c.s) * d.M;
}

template <int D, int B, int kShare = 0, typename Tile, typename Cx>
__device__ __forceinline__ void load_at(Tile& r, const Cx& cx, const DecodeDims& d,
                                        const Cursor& c, int lane) {
  constexpr int64_t kTileElems = static_cast<int64_t>(D) * B;
  PairCursor<typename Tile::Elem> pc;
  pc.k = cx.k;
  pc.v = cx.v;
  pc.trow = cx.tables + table_offset<B, kShare>(d, c);
  const int64_t span = kTileElems * tile_span(d.kv_mul);  // paired pools: K and V tiles
  pc.block_stride = span * d.Hkv;
  pc.head_off = span * c.g;
  pc.nb = d.NB;
  pc.nblk = (c.L + B - 1) / B;
  r.load(pc, c.t, lane);
}

// First q/out row of a (sequence, KV head) pair.  In the prefix pass the rows
// of group member qi are those of sequence first + qi (q is [S][Hq][D]).
template <bool kCausal, int kShare = 0>
__device__ __forceinline__ int64_t pair_row(const DecodeDims& d, const Cursor& c) {
  if constexpr (kShare == 1) return static_cast<int64_t>(c.x) * d.Hq + c.g * d.G;
  if constexpr (kCausal)  // rows of the wave's chunk of query tokens
    return (c.s * static_cast<int64_t>(d.Qmax) + d.chunk * d.Qc) * d.Hq + c.g * d.G;
  return c.s * static_cast<int64_t>(d.Hq) + c.g * d.G;
}

// Rows of a pair (R = G in decode launches).
template <bool kCausal>
__device__ __forceinline__ int32_t pair_rows(const DecodeDims& d) {
  return kCausal ? d.R : d.G;
}

// True when column j of this lane is a row the launch computes.
template <int NC, bool kCausal>
__device__ __forceinline__ bool live(const Cols<NC>& cl, int j, const Cursor& c) {
  return cl.row[j] >= 0 && (!kCausal || cl.qi[j] < c.Tq);
}

// Score MFMA B operand: lane holds q[row of column j][c*32 + (lane/16)*8 .. +7]
// (with fp8 K, the permuted dims (c/2)*64 + (lane/16)*16 + (c%2)*8 .. +7); zeros
// for columns the launch does not compute.
template <int D, int NC, bool kCausal, bool kFp8, int kShare = 0, typename Cx>
__device__ __forceinline__ void load_q(bf16x8_t (&qop)[NC][D / 32], const Cx& cx,
                                       const DecodeDims& d, const Cursor& c, const Cols<NC>& cl,
                                       int lane) {
  const int64_t r0 = pair_row<kCausal, kShare>(d, c);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (live<NC, kCausal>(cl, j, c)) {
      if constexpr (kFp8) {
        const uint16_t* qr = cx.q + (r0 + cl.row[j]) * D + (lane >> 4) * 16;
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
          qop[j][k] = __builtin_bit_cast(
              bf16x8_t, *reinterpret_cast<const u32x4_t*>(qr + (k / 2) * 64 + (k % 2) * 8));
      } else {
        const uint16_t* qr = cx.q + (r0 + cl.row[j]) * D + (lane >> 4) * 8;
#pragma unroll
        for (int k = 0; k < D / 32; ++k)
          qop[j][k] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qr + k * 32));
      }
    } else {
#pragma unroll
      for (int k = 0; k < D / 32; ++k)
        qop[j][k] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
    }
  }
}

// Prefix softmax states of a shared-prefix launch: one record of record_floats(Hq,
// D) floats per sequence (O[Hq][D], then m[Hq], then l[Hq]), unnormalised: O and l
// are sums weighted by 2^(score - m).  Row `gr` (= sequence * Hq + head) has its O
// at state_o(gr), m at state_m(gr) and l at state_m(gr) + Hq.
template <int D>
__device__ __forceinline__ int64_t state_o(const DecodeDims& d, int64_t gr) {
  const int64_t s = gr / d.Hq;
  return s * record_floats(d.Hq, D) + (gr - s * d.Hq) * D;
}
template <int D>
__device__ __forceinline__ int64_t state_m(const DecodeDims& d, int64_t gr) {
  const int64_t s = gr / d.Hq;
  return s * record_floats(d.Hq, D) + static_cast<int64_t>(d.Hq) * D + (gr - s * d.Hq);
}

// Descriptors (and record pairs) of a launch: one per wave (nch waves per planned
// range in multi-token launches whose chunks share ranges), then in the passes of a
// shared-prefix launch one per (group or sequence, KV head) pair.
template <int kShare>
__host__ __device__ __forceinline__ int64_t descriptor_count(const DecodeDims& d) {
  return static_cast<int64_t>(d.n_workers) * (d.nch > 1 ? d.nch : 1) +
         (kShare != 0 ? static_cast<int64_t>(d.S) * d.Hkv : 0);
}

// End of a segment: the output rows when it covered the whole pair, else a partial
// record (O, then m, then l) in slot `rec`.  The prefix pass writes a whole pair's
// rows as prefix states instead of outputs.
template <int D, int NC, bool kCausal, int kShare = 0, typename Cx>
__device__ void finish_segment(const Cx& cx, const DecodeDims& d, const SegState<D> (&st)[NC],
                               const Cursor& c, const Cols<NC>& cl, bool whole, int64_t rec,
                               int lane) {
  const int64_t r0 = pair_row<kCausal, kShare>(d, c);
  const int32_t R = pair_rows<kCausal>(d);
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    if (!live<NC, kCausal>(cl, j, c)) continue;
    const float l_tot = st[j].l[0];
    if (kShare == 1 && whole) {
      const int64_t gr = r0 + cl.row[j];
      float* orow = cx.state + state_o<D>(d, gr) + (lane >> 4) * 4;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) *reinterpret_cast<f32x4_t*>(orow + mt * 16) = st[j].o[mt];
      if (lane < 16) {
        float* ml = cx.state + state_m<D>(d, gr);
        ml[0] = st[j].m;
        ml[d.Hq] = l_tot;
      }
    } else if (whole) {
      const float inv = d.v_scale / l_tot;
      uint16_t* orow = cx.out + (r0 + cl.row[j]) * D + (lane >> 4) * 4;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        bf16x4_t y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = static_cast<__bf16>(st[j].o[mt][i] * inv);
        *reinterpret_cast<u32x2_t*>(orow + mt * 16) = __builtin_bit_cast(u32x2_t, y);
      }
    } else {
      const int32_t n = j * 16 + (lane & 15);
      float* base = cx.ws + rec * record_floats(R, D);
      float* orow = base + n * D + (lane >> 4) * 4;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) *reinterpret_cast<f32x4_t*>(orow + mt * 16) = st[j].o[mt];
      if (lane < 16) {
        base[R * D + n] = st[j].m;
        base[R * D + R + n] = l_tot;
      }
    }
  }
}

// Decode with append: the pair's newest position (the one past its tiles) joins
// the segment holding the pair's last tile, from k_new / v_new, the way
// compute_tile treats a position: score in the log2 domain, the same lazy
// rescaling, the weight rounded to bf16 for the weighted sum of values.  The
// worker also writes the new rows into their slot (the caller has made the block
// private, so no other worker reads it).  bf16 pools only: over fp8 pools the new
// rows are quantised by the append kernel in a launch of their own (folded in
// here, the encoding's registers pushed the whole tile loop into spills).
// This lane's parts of a pair's newest rows: the key dims of its score operand
// and the value dims of its O entries (read ahead by fetch_new).
template <int D>
struct NewRow {
  u32x4_t k[D / 32];
  u32x2_t v[D / 16];
};

template <int D, typename Cx>
__device__ __forceinline__ void fetch_new(NewRow<D>& nr, const Cx& cx, const DecodeDims& d,
                                          const Cursor& c, int lane) {
  const int64_t row = (static_cast<int64_t>(c.s) * d.Hkv + c.g) * D;
  const int gq = lane >> 4;
#pragma unroll
  for (int k = 0; k < D / 32; ++k)
    nr.k[k] = *reinterpret_cast<const u32x4_t*>(cx.k_new + row + k * 32 + gq * 8);
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
    nr.v[mt] = *reinterpret_cast<const u32x2_t*>(cx.v_new + row + mt * 16 + gq * 4);
}

template <int D, int B, typename Cx>
__device__ __forceinline__ void append_token(SegState<D>& st, const bf16x8_t (&qop)[D / 32],
                                             const NewRow<D>& nr, const Cx& cx,
                                             const DecodeDims& d, const Cursor& c, int lane) {
  const int gq = lane >> 4;
  const int32_t p = c.L;                 // the tiles hold positions 0 .. p - 1
  // A table entry outside the pool names no slot: the rows are attended to but not
  // stored (the append kernel skips such a token the same way), so a broken entry
  // never overwrites a block of another sequence.
  const int32_t raw = cx.tables[static_cast<int64_t>(c.s) * d.M + p / B];
  const bool in_pool = raw >= 0 && raw < d.NB;
  const int32_t b = in_pool ? raw : 0;
  const bool writer = in_pool && (lane & 15) == 0;  // lanes 0, 16, 32, 48 cover every dim once
  const int32_t ob = p % B;
  const int64_t tile =
      (static_cast<int64_t>(b) * d.Hkv + c.g) * D * B * tile_span(d.kv_mul);  // elements
  // score: this lane's query dims (the score MFMA operand layout) against the new key
  float part = 0.f;
#pragma unroll
  for (int k = 0; k < D / 32; ++k) {
    const int d0 = k * 32 + gq * 8;
    const u32x4_t x = nr.k[k];
    if (writer) *reinterpret_cast<u32x4_t*>(cx.kw + tile + ((d0 / 8) * B + ob) * 8) = x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      part = fmaf(static_cast<float>(qop[k][2 * e]), lo_bf16(x[e]), part);
      part = fmaf(static_cast<float>(qop[k][2 * e + 1]), hi_bf16(x[e]), part);
    }
  }
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  const float sc = part * d.c;
  float x = sc - st.m;
  if (x > kRescaleThreshold) {  // also when nothing has been seen (m = -inf)
    const float alpha = __builtin_amdgcn_exp2f(st.m - sc);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] *= alpha;
    st.l *= alpha;
    st.m = sc;
    x = 0.f;
  }
  const float wgt = static_cast<float>(static_cast<__bf16>(__builtin_amdgcn_exp2f(x)));
  st.l += wgt;
  constexpr int32_t kRun = B < kTile ? B : kTile;  // positions of one V run
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    const int d0 = mt * 16 + gq * 4;  // this lane's four dims of O
    const u32x2_t vv = nr.v[mt];
    const uint32_t pair[2] = {vv.x, vv.y};
    if (writer) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        cx.vw[tile + ((ob / kRun) * D + d0 + i) * kRun + ob % kRun] =
            static_cast<uint16_t>(pair[i / 2] >> (16 * (i % 2)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (i % 2) ? hi_bf16(pair[i / 2]) : lo_bf16(pair[i / 2]);
      st.o[mt][i] = fmaf(wgt, v, st.o[mt][i]);
    }
  }
}

// Decode with append, a sequence whose only position is the new one: every
// query head's output is that position's value, and the rows go into slot 0 (not
// stored when the table entry lies outside the pool, as in append_token).
template <int D, int B, typename Cx>
__device__ void one_token(const Cx& cx, const DecodeDims& d, int64_t s, int lane) {
  const int32_t raw = cx.tables[s * d.M];
  const bool in_pool = raw >= 0 && raw < d.NB;
  const int32_t b = in_pool ? raw : 0;
  constexpr int32_t kRun = B < kTile ? B : kTile;
  for (int32_t e = lane; e < d.Hkv * D; e += kWave) {
    const int32_t g = e / D, dd = e % D;
    const int64_t tile = (static_cast<int64_t>(b) * d.Hkv + g) * D * B * tile_span(d.kv_mul);
    const uint16_t kx = cx.k_new[s * d.Hkv * D + e];
    const uint16_t vx = cx.v_new[s * d.Hkv * D + e];
    if (in_pool) {
      cx.kw[tile + (dd / 8) * B * 8 + dd % 8] = kx;
      cx.vw[tile + dd * kRun] = vx;
    }
    // softmax over one position: the output is the value
    for (int32_t j = 0; j < d.G; ++j) cx.out[(s * d.Hq + g * d.G + j) * D + dd] = vx;
  }
}

// One worker: the n tiles of its range in order, with loads running kPipe-1
// tiles ahead of the arithmetic across (sequence, head) boundaries; the query of a
// pair is fetched with the pair's first tile.  Returns the descriptor of the split
// pair this worker opens (s = -1 if none).  The passes of a shared-prefix launch
// also write pair descriptors (see the end of a segment below).
template <int D, int B, int NC, bool kCausal, bool kFp8, bool kAppend, int kShare = 0,
          typename Cx>
__device__ int4 run_worker(const Cx& cx, const DecodeDims& d, const WorkerPlan& pl, int64_t w,
                           int lane, uint64_t& t_first) {
  const int32_t cap = d.M * B;
  const int32_t n = pl.n;
  const Cols<NC> cl = make_cols<NC, kCausal>(d, lane);
  Cursor lc;
  lc.start = pl.start;
  lc.s = pl.s;
  lc.L = pl.L;
  lc.Tq = pl.Tq;
  lc.x = (kShare != 0 || kCausal) ? seq_len<kCausal, kShare>(cx.lens, cx.qlens, d, cap, pl.s).x
                                  : 0;
  lc.T = tiles_of(lc.L);
  lc.g = pl.g;
  lc.t = pl.t;
  Cursor cc = lc;

  constexpr int kPipe = pipe_depth<D, NC, kFp8>();
  TileOf<D, B, kFp8> r[kPipe];
  bf16x8_t qb[kPipe][NC][D / 32];
  bf16x8_t qc[NC][D / 32];
  SegState<D> st[NC];
  int32_t lim_abs[NC];  // last position column j sees (multi-token launches)
  int32_t seg_t0 = cc.t;
  int64_t rec = 2 * w;  // first segment -> slot 0, later ones -> slot 1
  int4 opened = {-1, 0, 0, 0};

  // Decode with append: the newest rows of the pair whose last tile the next
  // compute step takes, read before that step's tile loads are issued, so that
  // waiting for them does not wait for the tiles loaded after.
  NewRow<D> nr;
  auto fetch_step = [&]() {
    if constexpr (kAppend) {
      if (cc.t == cc.T - 1) fetch_new<D>(nr, cx, d, cc, lane);
    }
  };
  auto load_step = [&](int slot, int32_t li) {
    if (lc.t == 0 || li == 0) load_q<D, NC, kCausal, kFp8, kShare>(qb[slot], cx, d, lc, cl, lane);
    load_at<D, B, kShare>(r[slot], cx, d, lc, lane);
    advance<kCausal, kShare>(lc, cx, d, cap);
  };
  auto compute_step = [&](int slot, int32_t i) {
    if (cc.t == 0 || i == 0) {
#pragma unroll
      for (int j = 0; j < NC; ++j) {
#pragma unroll
        for (int k = 0; k < D / 32; ++k) qc[j][k] = qb[slot][j][k];
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) st[j].o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st[j].l = f32x4_t{0.f, 0.f, 0.f, 0.f};
        st[j].m = -INFINITY;
        // query token qi sits at position L - Tq + qi; other columns (and every
        // row of the prefix pass) see the whole context
        lim_abs[j] = (kShare == 0 && kCausal && live<NC, kCausal>(cl, j, cc))
                         ? cc.L - cc.x + cl.qi[j]
                         : cc.L - 1;
      }
      seg_t0 = cc.t;
    }
    const int32_t valid = min(kTile, cc.L - cc.t * kTile);
#ifdef PKV_TIMELINE
    if (i == 0) t_first = __builtin_amdgcn_s_memrealtime();
#endif
    if constexpr (kCausal) {
      int32_t lim[NC];
#pragma unroll
      for (int j = 0; j < NC; ++j) lim[j] = lim_abs[j] - cc.t * kTile;
      compute_tile<D, NC, true>(r[slot], qc, st, d.c, valid,
                                (kShare == 1 ? cc.L - 1 : cc.L - cc.x) - cc.t * kTile, lim,
                                lane);
    } else {
      const int32_t lim[NC] = {valid - 1};
      compute_tile<D, NC, false>(r[slot], qc, st, d.c, valid, valid - 1, lim, lane);
      if constexpr (kAppend) {
        static_assert(NC == 1, "decode with append has one query row per head");
        if (cc.t == cc.T - 1) append_token<D, B>(st[0], qc[0], nr, cx, d, cc, lane);
      }
    }
    if (cc.t == cc.T - 1 || i == n - 1) {
      bool whole = seg_t0 == 0 && cc.t == cc.T - 1;
      int64_t rec_at = rec;
      if constexpr (kShare == 1) {
        // prefix pass (split launches): the segment holding a pair's first tile
        // names where the tail merge finds the pair's prefix: its state (whole
        // pair, x = -1) or the records of waves x .. y, the first in slot z.  Pair
        // (v, 0) also maps each member sequence to (v, member index).
        if (seg_t0 == 0 && !d.pair_mode) {
          const int64_t pair = static_cast<int64_t>(cc.s) * d.Hkv + cc.g;
          int4 pd = {-1, 0, 0, 0};
          if (!whole)
            pd = int4{static_cast<int32_t>(w),
                      static_cast<int32_t>(worker_of(cc.start + static_cast<int64_t>(cc.g) *
                                                                    pair_units(cc.T, d) +
                                                         d.hdr + static_cast<int64_t>(d.unit) * (cc.T - 1),
                                                     pl.U, pl.N)),
                      static_cast<int32_t>(rec - 2 * w), 0};
          if (lane == 0) cx.desc[d.n_workers + pair] = pd;
          if (cc.g == 0)
            for (int32_t m = lane; m < cc.Tq; m += kWave) {
              cx.gmap[2 * (cc.x + m)] = cc.s;
              cx.gmap[2 * (cc.x + m) + 1] = m;
            }
        }
      }
      if constexpr (kShare == 2) {
        // tail pass: the segment holding a pair's first tile names the pair's
        // record set for the merge (pair descriptor n_workers + pair).  A whole
        // pair with a prefix leaves a record in the pair's own slot (the merge
        // folds it after the prefix); other pairs get none: whole ones write
        // their rows here, split ones are named by the opener's descriptor.
        if (seg_t0 == 0) {
          const int64_t pair = static_cast<int64_t>(cc.s) * d.Hkv + cc.g;
          const int32_t k = static_cast<int32_t>(d.n_workers + pair);
          int4 pd = {-1, 0, 0, 0};
          if (whole && cc.x > 0) {
            pd = int4{cc.s, cc.g, k, 2};
            rec_at = 2 * static_cast<int64_t>(k);
          }
          if (lane == 0) cx.desc[k] = pd;
        }
      }
      finish_segment<D, NC, kCausal, kShare>(cx, d, st, cc, cl, whole && rec_at == rec, rec_at,
                                             lane);
      if (!whole && seg_t0 == 0) {
        // this worker holds the first share of a pair that later workers continue;
        // the worker holding the pair's last tile closes it (worked out here, mid-
        // stream, rather than after the last tile where it would lengthen the tail)
        const int64_t last_unit = cc.start + static_cast<int64_t>(cc.g) * pair_units(cc.T, d) +
                                  d.hdr + static_cast<int64_t>(d.unit) * (cc.T - 1);
        // slot | Tq << 1 (multi-token), or slot | 2 when the pair has a prefix (tail pass)
        const int32_t slot_tq = static_cast<int32_t>(rec - 2 * w) |
                                (kCausal ? cc.Tq << 1 : (kShare == 2 && cc.x > 0 ? 2 : 0));
        // the closing worker's range, as the wave that takes this wave's rows there
        const int64_t wb = worker_of(last_unit, pl.U, pl.N) * max(d.nch, 1) + d.chunk;
        opened = int4{cc.s, cc.g, static_cast<int32_t>(wb), slot_tq};
      }
      rec = 2 * w + 1;
    }
    advance<kCausal, kShare>(cc, cx, d, cap);
  };

#pragma unroll
  for (int k = 0; k < kPipe - 1; ++k)
    if (k < n) load_step(k, k);
  int32_t i = 0;
  // Whole groups of kPipe steps in which every step has a tile to load.
  while (i + 2 * kPipe - 1 <= n) {
#pragma unroll
    for (int k = 0; k < kPipe; ++k) {
      fetch_step();
      load_step((k + kPipe - 1) % kPipe, i + k + kPipe - 1);
      compute_step(k, i + k);
    }
    i += kPipe;
  }
  const int32_t rem = n - i;  // fewer than 2*kPipe-1 tiles left, kPipe-1 of them loading
#pragma unroll
  for (int k = 0; k < 2 * kPipe - 2; ++k) {
    if (k < rem) {
      fetch_step();
      if (k + kPipe - 1 < rem) load_step((k + kPipe - 1) % kPipe, i + k + kPipe - 1);
      compute_step(k % kPipe, i + k);
    }
  }
  return opened;
}

// The decode kernel (NC = 1, no position mask) and the multi-token kernel.
// Workspace: partial records ([n_workers][2] of record_floats), then one
// descriptor per worker: (s, g, wb, first_slot | Tq << 1) of the split pair whose
// first share this worker holds, or s = -1 (Tq only in multi-token launches).
// fp8 single-tile launches cap registers for two waves per SIMD; the others keep
// one.  kShare: 0, or the prefix (1) or tail (2) pass of a shared-prefix launch
// (seq_len), whose prefix states are at `state`.  Multi-token launches with
// d.nch > 1: wave `wave` takes chunk wave % nch of the query tokens over the
// range of worker (slot) wave / nch; records and descriptors are per wave.
template <int D, int B, int NC, bool kCausal, bool kFp8, bool kAppend, int kShare>
__device__ __forceinline__ void decode_body(const Ctx<typename TileOf<D, B, kFp8>::Elem>& cx,
                                            DecodeDims d, int64_t wave) {
  static_assert(!(kFp8 && kAppend), "over fp8 pools the new rows are appended in their own launch");
  const int32_t* __restrict__ lens = cx.lens;
  const int32_t* __restrict__ qlens = cx.qlens;
  uint16_t* __restrict__ out = cx.out;
  float* __restrict__ state = cx.state;
  int4* __restrict__ desc = cx.desc;
  const int lane = __lane_id();
  int64_t w = wave;  // the planned range (slot) this wave takes
  if constexpr (kCausal && kShare == 0) {
    const int32_t nch = max(d.nch, 1);
    w = wave / nch;
    d.chunk = static_cast<int32_t>(wave - w * nch);
  }
  if (w >= d.n_workers) return;
  const int32_t cap = d.M * B;
#ifdef PKV_TIMELINE
  const uint64_t t_entry = __builtin_amdgcn_s_memrealtime();
#endif
  uint64_t t_first = 0;

  int4 opened = {-1, 0, 0, 0};
  WorkerPlan pl;
  const bool has = d.pair_mode ? plan_pair<kCausal, kShare>(lens, qlens, d, cap, w, pl)
                               : plan_worker<kCausal, kShare>(lens, qlens, d, cap, w, lane, pl);
#ifdef PKV_TIMELINE
  const uint64_t t_plan = __builtin_amdgcn_s_memrealtime();
#endif
  if (has)
    opened = run_worker<D, B, NC, kCausal, kFp8, kAppend, kShare>(cx, d, pl, wave, lane, t_first);
#ifdef PKV_TIMELINE
  {
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    WorkerStamp st;
    st.t_entry = t_entry;
    st.d_plan = static_cast<uint32_t>(t_plan - t_entry);
    st.d_first = has ? static_cast<uint32_t>(t_first - t_entry) : 0xFFFFFFFFu;
    st.d_end = static_cast<uint32_t>(t_end - t_entry);
    st.xcc = xcc & 0xF;
    st.tiles = has ? static_cast<uint32_t>(pl.n) : 0u;
    st.group = blockIdx.x;
    // stamps follow the descriptors (split launches only: the workspace of a
    // pair-mode launch is sized for its worker slots); one lane writes 32 bytes
    if (lane == 0 && !d.pair_mode)
      reinterpret_cast<WorkerStamp*>(desc + descriptor_count<kShare>(d))[wave] = st;
  }
#endif

  // Rows no tile reaches are zeros: every row of an empty sequence, and in a
  // multi-token launch the rows past a sequence's query tokens (done last: off
  // the path to the first loads).  The prefix pass writes no output rows; in the
  // tail pass a sequence whose context is all prefix is left to the merge.
  const int32_t row_elems = d.Hq * D;
  if constexpr (kShare == 1) {
    if (!d.pair_mode && lane == 0) desc[wave] = opened;
    return;
  }
  if constexpr (kShare == 2) {
    // a sequence whose context is all prefix has no tail tile: with a prefix its
    // pairs' rows come from the merge (prefix state only), else they are zeros
    for (int64_t se = w; se < d.S; se += d.n_workers) {
      const SeqLen sl = seq_len<false, 2>(lens, qlens, d, cap, static_cast<int32_t>(se));
      if (sl.L != 0) continue;
      for (int32_t g = lane; g < d.Hkv; g += kWave) {
        const int32_t kd = static_cast<int32_t>(d.n_workers + se * d.Hkv + g);
        desc[kd] = sl.x > 0 ? int4{static_cast<int32_t>(se), g, kd - 1, 2} : int4{-1, 0, 0, 0};
      }
      if (sl.x > 0) continue;
      uint16_t* row = out + se * row_elems;
      for (int32_t e = lane * 8; e < row_elems; e += kWave * 8)
        *reinterpret_cast<u32x4_t*>(row + e) = u32x4_t{0, 0, 0, 0};
    }
    if (!d.pair_mode && lane == 0) desc[wave] = opened;
    return;
  }
  for (int64_t se = w; se < d.S; se += d.n_workers) {
    int32_t first = 0;
    if constexpr (kCausal) {
      first = seq_len<true>(lens, qlens, d, cap, static_cast<int32_t>(se)).T;
    } else {
      const int32_t Lt = clamp_len(lens[se], cap);
      if constexpr (kAppend) {
        if (Lt == 1) one_token<D, B>(cx, d, se, lane);
      }
      if (Lt != 0) continue;
    }
    // this wave's chunk of query tokens (never past max_query_len)
    const int32_t rows = kCausal ? min(d.Qc, d.Qmax - d.q_off - d.chunk * d.Qc) : 1;
    for (int32_t qi = first; qi < rows; ++qi) {
      uint16_t* row = out + (kCausal ? se * d.Qmax + d.chunk * d.Qc + qi : se) * row_elems;
      for (int32_t e = lane * 8; e < row_elems; e += kWave * 8)
        *reinterpret_cast<u32x4_t*>(row + e) = u32x4_t{0, 0, 0, 0};
    }
  }
  if (!d.pair_mode && lane == 0) desc[wave] = opened;
}

template <int D, int B, int NC, bool kCausal, bool kFp8, bool kAppend, int kShare = 0>
__global__ __launch_bounds__(kWave* kWavesPerGroup,
                             (kFp8 && NC == 1) ? 2 : 1) void decode_kernel(
    const uint16_t* __restrict__ q, const typename TileOf<D, B, kFp8>::Elem* __restrict__ k,
    const typename TileOf<D, B, kFp8>::Elem* __restrict__ v,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ qlens, uint16_t* __restrict__ out, float* __restrict__ ws,
    int4* __restrict__ desc, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, typename TileOf<D, B, kFp8>::Elem* kw,
    typename TileOf<D, B, kFp8>::Elem* vw, float* __restrict__ state, DecodeDims d) {
  const Ctx<typename TileOf<D, B, kFp8>::Elem> cx{q,     k,  v,  tables, lens, qlens, out,
                                                  ws,    k_new, v_new, kw, vw, state, desc,
                                                  nullptr};
  decode_body<D, B, NC, kCausal, kFp8, kAppend, kShare>(
      cx, d, static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + uniform(threadIdx.x / kWave));
}

// Both passes of a shared-prefix call in one launch: work-groups below
// prefix_groups run the prefix pass (NCp column tiles of group-member rows), the
// others the tail pass, each over its own workers, records and descriptors.
struct SharedArgs {
  Ctx<uint16_t> p, t;  // prefix pass, tail pass
  DecodeDims a, d;     // their sizes
  int32_t prefix_groups;
};

template <int D, int B, int NCp>
__global__ __launch_bounds__(kWave* kWavesPerGroup, 1) void shared_kernel(SharedArgs sa) {
  const int64_t wi = uniform(threadIdx.x / kWave);
  if (static_cast<int32_t>(blockIdx.x) < sa.prefix_groups)
    decode_body<D, B, NCp, true, false, false, 1>(
        sa.p, sa.a, static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + wi);
  else
    decode_body<D, B, 1, false, false, false, 2>(
        sa.t, sa.d, static_cast<int64_t>(blockIdx.x - sa.prefix_groups) * kWavesPerGroup + wi);
}

// Merge of split pairs.  Work-group b reads the descriptors of its slice of
// workers in one parallel pass and keeps the valid ones in LDS (each names a split
// pair opened by worker wa and closed by wb).  The (pair, output) items of those
// pairs are spread over the threads, kItems per thread at a time; an item folds
// the records of wa..wb in worker order with a running max, kChunk records per
// batch, and the loads of all of a thread's items are issued together.  The order
// is fixed, so the result does not depend on timing.  In multi-token launches the
// rows past the pair's query tokens are left to the decode kernel.
//
// Shapes (measured): pairs split over more than 11 workers take one item of 16
// records per batch (one round trip for a 16-way split; a pair spread over 12
// workers' ranges has 13 records, which would take two 12-record batches);
// otherwise two items of 12 records each, so that more independent loads are in
// flight, or of 10 records when the launch has many items (held to 128 registers,
// so that two work-groups share a CU; see launch_merge).
constexpr int kMergeThreads = 512;
constexpr int kMergeSlice = 64;  // most descriptors one work-group scans
constexpr int kMergeWideSplit = 11;
// Outputs of a pair one merge work-group takes (a decode pair at G = 4, D = 128);
// pairs with more rows (multi-token and prefix launches) spread over more groups.
constexpr int kMergeSpan = 512;


// The 10-record shape asks for 4 waves per SIMD (two 512-thread groups per CU, at
// most 128 registers).
template <int kChunk>
constexpr bool kTwoPerCu = kChunk == 10;

// Where the merge of a shared-prefix launch's tail pass finds the prefix of a
// pair: the prefix pass's records (R rows each) and pair descriptors (none: every
// prefix is a whole pair, whose state the prefix pass wrote), and the member map.
struct PrefixView {
  const float* ws;
  const int4* pdesc;
  const int32_t* gmap;
  int32_t R, groups, waves;  // rows per record, groups, prefix waves (records 2 * waves)
};

//
// Tail pass of a shared-prefix launch (kShare = 2): a pair with a prefix folds its
// prefix first, from the prefix state (a whole prefix pair) or from the prefix
// pass's records of its rows (a split one), then its own records.
template <int D, bool kCausal, int kChunk, int kItems, int kShare = 0>
__global__ __launch_bounds__(kMergeThreads, (kTwoPerCu<kChunk> ? 4 : 1)) void merge_kernel(
    const int4* __restrict__ desc, uint16_t* __restrict__ out, const float* __restrict__ ws,
    DecodeDims d, PrefixView pv, const float* __restrict__ state) {
  // record loads by 32-bit byte offsets from ws: in decode launches (records of at
  // most 4 waves per CU, a few tens of MB; the 12-record merge in 132 instead of 246
  // registers) and in the 10-record shape, which launch_merge takes only while the
  // launch's records stay below 4 GiB.  The other multi-token and shared-prefix
  // shapes keep 64-bit addresses.
  constexpr bool kOffsets32 = (kShare == 0 && !kCausal) || kTwoPerCu<kChunk>;
  __shared__ int4 s_desc[kMergeSlice];
  __shared__ int32_t s_wa[kMergeSlice];
  __shared__ int4 s_pp[kShare == 2 ? kMergeSlice : 1];
  __shared__ int32_t s_count;
  const int tid = threadIdx.x;
  // descriptors are per wave: nch waves per planned range in multi-token launches
  // whose chunks share ranges; a pair's records are then every nch-th wave's.  The
  // tail pass of a shared-prefix launch adds one descriptor per pair.
  const int32_t nch = kCausal ? max(d.nch, 1) : 1;
  const int64_t n_waves = descriptor_count<kShare>(d);
  const int64_t per = (n_waves + gridDim.x - 1) / gridDim.x;
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t w1 = min(w0 + per, n_waves);
  if (tid == 0) s_count = 0;
  __syncthreads();
  if (w0 + tid < w1) {
    const int4 ds = desc[w0 + tid];
    if (ds.x >= 0) {
      const int32_t slot = atomicAdd(&s_count, 1);
      s_desc[slot] = ds;
      s_wa[slot] = static_cast<int32_t>(w0 + tid);
      if constexpr (kShare == 2) {
        // the prefix of a pair with one: {first wave, last wave, first slot, member}
        // of its split prefix pair, or x = -1 (the prefix state)
        int4 pp = {-1, 0, 0, 0};
        if ((ds.w & 2) && pv.pdesc) {
          const int32_t grp = min(max(pv.gmap[2 * ds.x], 0), pv.groups - 1);
          const int32_t mem = min(max(pv.gmap[2 * ds.x + 1], 0), pv.R / d.G - 1);
          const int4 pd = pv.pdesc[static_cast<int64_t>(grp) * d.Hkv + ds.y];
          // clamped into the prefix pass's records: a batch that breaks the group
          // contract (a member with a prefix whose group has none) reads descriptors
          // of an earlier call, and gets meaningless rows, never memory outside
          if (pd.x >= 0) {
            const int32_t a = min(pd.x, pv.waves - 1);
            pp = int4{a, min(max(pd.y, a), pv.waves - 1), pd.z & 1, mem};
          }
        }
        s_pp[slot] = pp;
      }
    }
  }
  __syncthreads();
  const int64_t rf = record_floats(d.R, D);
  const int32_t RD = d.R * D;
  // the outputs of a pair are split over gridDim.y work-groups: this one takes
  // outputs oi0 .. oi0 + span - 1 of each of its pairs
  const int32_t per_y = (RD + gridDim.y - 1) / gridDim.y;
  const int32_t oi0 = static_cast<int32_t>(blockIdx.y) * per_y;
  const int32_t span = max(min(per_y, RD - oi0), 0);
  const int32_t total = s_count * span;
  for (int32_t base = tid; base < total; base += kMergeThreads * kItems) {
    float run_m[kItems], run_l[kItems], acc[kItems];
    int64_t wa[kItems], wb[kItems], first[kItems];
    int32_t pi[kItems], oi[kItems];
    bool act[kItems];
    // tail pass of a shared-prefix launch: np prefix records (of prefix waves pwa ..,
    // the first in slot pslot) precede the pair's own, their entry (prow, pcol)
    int32_t np[kItems], pwa[kItems], pslot[kItems], prow[kItems], pcol[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      const int32_t item = base + it * kMergeThreads;
      run_m[it] = -INFINITY;
      run_l[it] = 0.f;
      acc[it] = 0.f;
      np[it] = 0;
      pwa[it] = pslot[it] = prow[it] = pcol[it] = 0;
      pi[it] = item < total ? item / span : 0;
      oi[it] = item < total ? oi0 + (item - pi[it] * span) : 0;
      act[it] = item < total;
      if constexpr (kCausal) act[it] = act[it] && (oi[it] / D) / d.G < (s_desc[pi[it]].w >> 1);
      wa[it] = s_wa[pi[it]];
      wb[it] = act[it] ? static_cast<int64_t>(s_desc[pi[it]].z) : wa[it] - 1;  // none
      first[it] = (2 * wa[it] + (s_desc[pi[it]].w & 1)) * rf;
      if constexpr (kShare == 2) {
        // a pair with a prefix starts from its prefix
        const int4 ds = s_desc[pi[it]];
        if (act[it] && (ds.w & 2)) {
          const int32_t row = oi[it] / D;
          const int32_t col = oi[it] - row * D;
          const int4 pp = s_pp[pi[it]];
          if (pp.x < 0) {
            const int64_t gr = static_cast<int64_t>(ds.x) * d.Hq + ds.y * d.G + row;
            const int64_t mo = state_m<D>(d, gr);
            run_m[it] = state[mo];
            run_l[it] = state[mo + d.Hq];
            acc[it] = state[state_o<D>(d, gr) + col];
          } else {
            // the records of prefix waves pp.x .. pp.y come first, row member*G + row
            np[it] = pp.y - pp.x + 1;
            pwa[it] = pp.x;
            pslot[it] = pp.z;
            prow[it] = pp.w * d.G + row;
            pcol[it] = col;
          }
        }
      }
    }
    // folds one batch of kChunk records per item into the running (m, l, acc)
    auto fold = [&](float (&m)[kItems][kChunk], const float (&l)[kItems][kChunk],
                    const float (&o)[kItems][kChunk]) {
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        float cm = run_m[it];
#pragma unroll
        for (int k = 0; k < kChunk; ++k) cm = fmaxf(cm, m[it][k]);
        if (cm == -INFINITY) continue;  // item past the end, or no record in this chunk
        const float scale = __builtin_amdgcn_exp2f(run_m[it] - cm);
        run_l[it] *= scale;
        acc[it] *= scale;
        run_m[it] = cm;
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
          const float e = __builtin_amdgcn_exp2f(m[it][k] - cm);
          run_l[it] += e * l[it][k];
          acc[it] += e * o[it][k];
        }
      }
    };
    if constexpr (kShare == 2) {
      // the prefix pass's records of the item's row, before the pair's own
      int32_t pmax = 0;
#pragma unroll
      for (int it = 0; it < kItems; ++it) pmax = max(pmax, np[it]);
      const int64_t rfp = record_floats(pv.R, D);
      for (int32_t c = 0; c < pmax; c += kChunk) {
        float m[kItems][kChunk], l[kItems][kChunk], o[kItems][kChunk];
#pragma unroll
        for (int it = 0; it < kItems; ++it) {
          const int32_t mo = pv.R * D + prow[it];  // m of the row; l follows R later
          const int32_t oo = prow[it] * D + pcol[it];
#pragma unroll
          for (int k = 0; k < kChunk; ++k) {
            const int32_t pk = c + k;
            if (pk < np[it]) {
              const float* rec = pv.ws + (pk == 0 ? 2 * static_cast<int64_t>(pwa[it]) + pslot[it]
                                                  : 2 * static_cast<int64_t>(pwa[it] + pk)) * rfp;
              m[it][k] = rec[mo];
              l[it][k] = rec[mo + pv.R];
              o[it][k] = rec[oo];
            } else {
              m[it][k] = -INFINITY;
              l[it][k] = 0.f;
              o[it][k] = 0.f;
            }
          }
        }
        fold(m, l, o);
      }
    }
    // the item's records: the first at `first`, record k >= 1 (wave wa + k*nch,
    // slot 0) k*stride floats after wave wa's slot 0
    int32_t cnt[kItems];
    int32_t kmax = 0;
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      cnt[it] = static_cast<int32_t>((wb[it] - wa[it]) / nch + 1);
      kmax = max(kmax, cnt[it]);
    }
    const int64_t stride = 2 * static_cast<int64_t>(nch) * rf;
    for (int32_t c = 0; c < kmax; c += kChunk) {
      float m[kItems][kChunk], l[kItems][kChunk], o[kItems][kChunk];
#pragma unroll
      for (int it = 0; it < kItems; ++it) {
        const int32_t h = oi[it] / D;
        const float* base = ws + 2 * wa[it] * rf;
        // kOffsets32: byte offsets from ws, so that each load takes ws as its
        // scalar base and one 32-bit register of offset
        const uint32_t b0 = static_cast<uint32_t>(2 * wa[it] * rf * 4);
        const uint32_t f0 = static_cast<uint32_t>(first[it] * 4);
#pragma unroll
        for (int k = 0; k < kChunk; ++k) {
          if (c + k < cnt[it]) {
            if constexpr (!kOffsets32) {
              const float* rec = c + k == 0 ? ws + first[it] : base + (c + k) * stride;
              m[it][k] = rec[RD + h];
              l[it][k] = rec[RD + d.R + h];
              o[it][k] = rec[oi[it]];
            } else {
              const uint32_t r =
                  c + k == 0 ? f0 : b0 + static_cast<uint32_t>((c + k) * stride * 4);
              const char* rec = reinterpret_cast<const char*>(ws) + r;
              m[it][k] = *reinterpret_cast<const float*>(rec + (RD + h) * 4);
              l[it][k] = *reinterpret_cast<const float*>(rec + (RD + d.R + h) * 4);
              o[it][k] = *reinterpret_cast<const float*>(rec + oi[it] * 4);
            }
          } else {
            m[it][k] = -INFINITY;
            l[it][k] = 0.f;
            o[it][k] = 0.f;
          }
        }
      }
      fold(m, l, o);
    }
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
      if (act[it]) {
        const int4 ds = s_desc[pi[it]];
        int64_t idx;
        if constexpr (kCausal) {
          const int32_t row = oi[it] / D;  // row = qi * G + head
          const int32_t qi = row / d.G;
          const int32_t chunk = static_cast<int32_t>(s_wa[pi[it]] % nch);  // the opener's
          idx = ((static_cast<int64_t>(ds.x) * d.Qmax + chunk * d.Qc + qi) * d.Hq + ds.y * d.G +
                 (row - qi * d.G)) *
                    D +
                (oi[it] - row * D);
        } else {
          idx = (static_cast<int64_t>(ds.x) * d.Hq + ds.y * d.G) * D + oi[it];
        }
        out[idx] = __builtin_bit_cast(uint16_t,
                                      static_cast<__bf16>(acc[it] / run_l[it] * d.v_scale));
      }
    }
  }
}

// Descriptors of a launch: after its records in the workspace.
template <int D, int kShare>
int4* descriptors(const DecodeBuffers& b, const DecodeDims& d) {
  return reinterpret_cast<int4*>(reinterpret_cast<char*>(b.ws) +
                                 records_bytes(descriptor_count<kShare>(d), d.R, D));
}

// The merge launch of a split launch.  Records per split pair: about the workers
// per (sequence, KV head) pair; a pair's outputs are spread over ny = ceil(R * D /
// kMergeSpan) work-groups, and the descriptor slices shrink to about merge_groups
// / ny (a 12- or 16-record merge work-group fills a CU: more than one per CU would
// run in rounds; merges with many items take the 10-record shape, two per CU, see
// below), each still scanning at most kMergeSlice descriptors.
template <int D, bool kCausal, int kShare>
hipError_t launch_merge(const DecodeBuffers& b, const DecodeDims& d, int merge_groups,
                        hipStream_t stream, const PrefixView& pv = PrefixView{}) {
  const int64_t n_desc = descriptor_count<kShare>(d);
  const int64_t pairs = static_cast<int64_t>(d.S) * d.Hkv;
  const int ny = (d.R * D + kMergeSpan - 1) / kMergeSpan;
  // Merges with many items take the 10-record shape (at most 128 registers) at two
  // work-groups per CU: when the split (pair, chunk) sets could hold more than one
  // item per thread of one group per CU, some groups would otherwise take a second
  // pass.  Measured faster on the chat and mix decode merges, 16 and 32 query tokens
  // on the long context, 8 and 16 on the chat batch and the shared-prefix tail
  // merge; with fewer items the larger grid only costs (89.2 -> 91.2 us at 4 tokens,
  // which stays below the bound).
  const bool wide = pairs > 0 && d.n_workers > kMergeWideSplit * pairs;
  const int64_t items = min(pairs * max(d.nch, 1), n_desc) * d.R * D;
  // (that shape addresses records by 32-bit byte offsets: taken only while the
  // launch's records stay below 4 GiB, which a shared-prefix tail pass, with a record
  // per (sequence, KV head) pair, could pass)
  const bool small_ws = records_bytes(n_desc, d.R, D) < (int64_t(1) << 32);
  const int per_cu =
      kShare != 1 && small_ws && !wide &&
              items > static_cast<int64_t>(merge_groups) * kMergeThreads
          ? 2
          : 1;
  const int nx = max(max(per_cu * merge_groups / ny,
                         static_cast<int>((n_desc + kMergeSlice - 1) / kMergeSlice)),
                     1);
  const dim3 grid(nx, ny);
  int4* desc = descriptors<D, kShare>(b, d);
  if (wide)
    hipLaunchKernelGGL((merge_kernel<D, kCausal, 16, 1, kShare>), grid, dim3(kMergeThreads), 0,
                       stream, desc, b.out, b.ws, d, pv, b.state);
  else if (per_cu == 2) {
    if constexpr (kShare != 1)  // per_cu is 2 only there
      hipLaunchKernelGGL((merge_kernel<D, kCausal, 10, 2, kShare>), grid, dim3(kMergeThreads),
                         0, stream, desc, b.out, b.ws, d, pv, b.state);
  } else
    hipLaunchKernelGGL((merge_kernel<D, kCausal, 12, 2, kShare>), grid, dim3(kMergeThreads), 0,
                       stream, desc, b.out, b.ws, d, pv, b.state);
  return hipGetLastError();
}

template <int D, int B, int NC, bool kCausal, bool kFp8, bool kAppend, int kShare>
hipError_t launch_t(const DecodeBuffers& b, const DecodeDims& d, int merge_groups,
                    hipStream_t stream) {
  using Elem = typename TileOf<D, B, kFp8>::Elem;
  const int64_t waves = static_cast<int64_t>(d.n_workers) * (kCausal ? max(d.nch, 1) : 1);
  const int groups = static_cast<int>((waves + kWavesPerGroup - 1) / kWavesPerGroup);
  if (groups <= 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<D, B, NC, kCausal, kFp8, kAppend, kShare>), dim3(groups),
                     dim3(kWave * kWavesPerGroup), 0, stream, b.q, static_cast<const Elem*>(b.k),
                     static_cast<const Elem*>(b.v), b.tables, b.lens, b.qlens, b.out, b.ws,
                     descriptors<D, kShare>(b, d), b.k_new, b.v_new, static_cast<Elem*>(b.kw),
                     static_cast<Elem*>(b.vw), b.state, d);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (d.pair_mode) return hipSuccess;  // nothing is split: no merge
  return launch_merge<D, kCausal, kShare>(b, d, merge_groups, stream);
}

// Both passes of a shared-prefix call (bp, a: prefix pass; bt, d: tail pass) in
// one launch, then one merge: the tail pass's, which folds each pair's prefix
// (prefix state, or the prefix pass's records) before its own records.  gmap:
// two int32 per sequence (its group, its member index).
template <int D, int B, int NCp>
hipError_t launch_shared_t(const DecodeBuffers& bp, const DecodeDims& a, const DecodeBuffers& bt,
                           const DecodeDims& d, int32_t* gmap, int merge_groups_tail,
                           hipStream_t stream) {
  auto ctx = [gmap](const DecodeBuffers& b, int4* desc) {
    return Ctx<uint16_t>{b.q,  static_cast<const uint16_t*>(b.k), static_cast<const uint16_t*>(b.v),
                         b.tables, b.lens, b.qlens, b.out, b.ws, nullptr, nullptr, nullptr,
                         nullptr, b.state, desc, gmap};
  };
  SharedArgs sa;
  sa.p = ctx(bp, descriptors<D, 1>(bp, a));
  sa.t = ctx(bt, descriptors<D, 2>(bt, d));
  sa.a = a;
  sa.d = d;
  sa.prefix_groups = (a.n_workers + kWavesPerGroup - 1) / kWavesPerGroup;
  const int groups = sa.prefix_groups + (d.n_workers + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL((shared_kernel<D, B, NCp>), dim3(groups), dim3(kWave * kWavesPerGroup), 0,
                     stream, sa);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  PrefixView pv;
  pv.ws = bp.ws;
  pv.pdesc = a.pair_mode ? nullptr : descriptors<D, 1>(bp, a) + a.n_workers;
  pv.gmap = gmap;
  pv.R = a.R;
  pv.groups = a.S;
  pv.waves = a.n_workers;
  return launch_merge<D, false, 2>(bt, d, merge_groups_tail, stream, pv);
}

template <int NC, bool kCausal, bool kFp8, bool kAppend = false, int kShare = 0>
hipError_t dispatch(const DecodeBuffers& b, const DecodeDims& d, int D, int B, int merge_groups,
                    hipStream_t stream) {
  if (D == 128) {
    if (B == 16) return launch_t<128, 16, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
    if (B == 32) return launch_t<128, 32, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
    if (B == 8) return launch_t<128, 8, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
  } else if (D == 64) {
    if (B == 16) return launch_t<64, 16, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
    if (B == 32) return launch_t<64, 32, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
    if (B == 8) return launch_t<64, 8, NC, kCausal, kFp8, kAppend, kShare>(b, d, merge_groups, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

}  // namespace pkv
