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
// Work decomposition.  The unit of work is a 16-token tile of one (sequence, KV
// head) pair.  Units are numbered sequence-major, then KV head, then tile, and the
// N workers (one wave each) take equal contiguous ranges of that numbering, so
// every worker streams the same number of K/V bytes whatever the mix of context
// lengths.  A worker's range is cut into segments at (sequence, head) boundaries.
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

#include <math.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kPipe = 3;                  // tile buffers in registers (kPipe-1 loads in flight)
constexpr float kRescaleThreshold = 8.0f;  // log2 units: weights stay below 2^8

__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ int32_t clamp_len(int32_t L, int32_t cap) {
  return L < 0 ? 0 : (L > cap ? cap : L);
}

__device__ __forceinline__ int32_t tiles_of(int32_t L) { return (L + kTile - 1) / kTile; }

__device__ __forceinline__ int32_t clamp_block(int32_t b, int64_t nb) {
  return b < 0 ? 0 : (b >= nb ? static_cast<int32_t>(nb - 1) : b);
}

__device__ __forceinline__ int32_t wave_sum(int32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Work units (tiles) of sequences [0, s_end): Hkv * sum ceil(L_s / 16).
__device__ int64_t units_before(const int32_t* __restrict__ lens, const DecodeDims& d,
                                int32_t cap, int32_t s_end, int lane) {
  int64_t tot = 0;
  for (int32_t base = 0; base < s_end; base += kWave) {
    const int32_t s = base + lane;
    const int32_t T = s < s_end ? tiles_of(clamp_len(lens[s], cap)) : 0;
    tot += uniform(wave_sum(T));
  }
  return tot * d.Hkv;
}

// The sequence whose unit range contains unit u, and the first unit of that range.
__device__ void locate(const int32_t* __restrict__ lens, const DecodeDims& d, int32_t cap,
                       int64_t u, int lane, int32_t& s_out, int64_t& start_out) {
  int64_t acc = 0;
  for (int32_t base = 0; base < d.S; base += kWave) {
    const int32_t s = base + lane;
    const int32_t T = s < d.S ? tiles_of(clamp_len(lens[s], cap)) : 0;
    const int32_t incl = wave_inclusive_scan(T, lane);
    const int64_t chunk_units =
        static_cast<int64_t>(__builtin_amdgcn_readlane(incl, kWave - 1)) * d.Hkv;
    if (u < acc + chunk_units) {
      const uint64_t hit = __ballot(acc + static_cast<int64_t>(incl) * d.Hkv > u);
      const int32_t first = uniform(__builtin_ctzll(hit));
      s_out = base + first;
      start_out = acc + static_cast<int64_t>(__builtin_amdgcn_readlane(incl - T, first)) * d.Hkv;
      return;
    }
    acc += chunk_units;
  }
  s_out = d.S;
  start_out = acc;
}

// Range of worker w: units [w*U/N, (w+1)*U/N).  worker_of(u) is the largest w
// whose range starts at or before u.
__device__ __forceinline__ int64_t range_begin(int64_t w, int64_t U, int64_t N) {
  return w * U / N;
}

__device__ __forceinline__ int64_t worker_of(int64_t u, int64_t U, int64_t N) {
  return ((u + 1) * N - 1) / U;
}

// A worker's share of the batch: total units U, active workers N, its range
// [u, u_end), the sequence s holding unit u and the first unit `start` of s.
struct WorkerPlan {
  int64_t U, N, u, u_end, start;
  int32_t s;
};

// Returns false when worker w has no range.  With at most kWave sequences the
// lengths are read once and scanned in registers; otherwise in two passes.
__device__ bool plan_worker(const int32_t* __restrict__ lens, const DecodeDims& d, int32_t cap,
                            int64_t w, int lane, WorkerPlan& p) {
  if (d.S <= kWave) {
    const int32_t T = lane < d.S ? tiles_of(clamp_len(lens[lane], cap)) : 0;
    const int32_t incl = wave_inclusive_scan(T, lane);
    p.U = static_cast<int64_t>(__builtin_amdgcn_readlane(incl, kWave - 1)) * d.Hkv;
    p.N = min(static_cast<int64_t>(d.n_workers), p.U);
    if (w >= p.N) return false;
    p.u = range_begin(w, p.U, p.N);
    p.u_end = range_begin(w + 1, p.U, p.N);
    const uint64_t hit = __ballot(static_cast<int64_t>(incl) * d.Hkv > p.u);
    const int32_t first = uniform(__builtin_ctzll(hit));
    p.s = first;
    p.start = static_cast<int64_t>(__builtin_amdgcn_readlane(incl - T, first)) * d.Hkv;
    return true;
  }
  p.U = units_before(lens, d, cap, d.S, lane);
  p.N = min(static_cast<int64_t>(d.n_workers), p.U);
  if (w >= p.N) return false;
  p.u = range_begin(w, p.U, p.N);
  p.u_end = range_begin(w + 1, p.U, p.N);
  locate(lens, d, cap, p.u, lane, p.s, p.start);
  return true;
}

template <int D, int B>
struct TileRegs {
  u32x4_t k[D / 32];  // score MFMA A operand: token lane%16, dims c*32 + (lane/16)*8 .. +7
  u32x2_t v[D / 16];  // value MFMA A operand: dim mt*16 + lane%16, tokens (lane/16)*4 .. +3
};

// Where one (sequence, KV head) pair's tiles come from.
struct PairCursor {
  const uint16_t* k;        // K pool
  const uint16_t* v;        // V pool
  const int32_t* trow;      // block-table row of the sequence
  int64_t head_off;         // g * (elements of one (block, head) tile)
  int64_t block_stride;     // elements of one block (all heads)
  int64_t nb;
  int32_t nblk;             // ceil(L / B)
};

// Issue the loads of tile t.
template <int D, int B>
__device__ __forceinline__ void load_tile(TileRegs<D, B>& r, const PairCursor& pc, int32_t t,
                                          int lane) {
  const int32_t tok0 = t * kTile;
  if constexpr (B >= kTile) {
    const int32_t b = clamp_block(pc.trow[tok0 / B], pc.nb);
    const int32_t ob = tok0 % B;
    const int64_t base = static_cast<int64_t>(b) * pc.block_stride + pc.head_off;
    const uint16_t* kt = pc.k + base;
    const uint16_t* vt = pc.v + base;
    const uint32_t koff = static_cast<uint32_t>(((lane >> 4) * B + ob + (lane & 15)) * 8);
    const uint32_t voff = static_cast<uint32_t>((lane & 15) * B + ob + (lane >> 4) * 4);
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      r.k[c] = *reinterpret_cast<const u32x4_t*>(kt + koff + c * 4 * B * 8);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      r.v[mt] = *reinterpret_cast<const u32x2_t*>(vt + voff + mt * 16 * B);
  } else {
    // B == 8: the tile spans logical blocks 2t and 2t+1 (the second clamped to the
    // sequence's last block; its lanes are masked when it lies past the context).
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
    for (int c = 0; c < D / 32; ++c) r.k[c] = *reinterpret_cast<const u32x4_t*>(kt + c * 4 * B * 8);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
      r.v[mt] = *reinterpret_cast<const u32x2_t*>(vt + mt * 16 * B);
  }
}

// Softmax state of one wave over one segment.
template <int D>
struct SegState {
  f32x4_t o[D / 16];  // O^T[dim mt*16 + (lane/16)*4 + i][head lane%16]
  f32x4_t l;          // every entry: sum of the bf16 weights of head lane%16
  float m;            // reference max of head lane%16 (log2 domain)
};

// One tile: scores, softmax weights, value and sum accumulation.  `valid` is the
// number of tokens of the tile inside the context (16 except in the last tile).
template <int D, int B>
__device__ __forceinline__ void compute_tile(TileRegs<D, B>& r, const bf16x8_t (&qop)[D / 32],
                                             SegState<D>& st, float c, int32_t valid, int lane) {
  f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cc = 0; cc < D / 32; ++cc)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k[cc]), qop[cc],
                                                 sc, 0, 0, 0);
  const int32_t tq = (lane >> 4) * 4;  // first of the four tokens this lane scores
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = fmaf(sc[i], c, -st.m);
  if (valid < kTile) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (tq + i >= valid) x[i] = -INFINITY;
    const int32_t n = valid - tq;
    const uint64_t keep = n >= 4 ? ~0ull : (n <= 0 ? 0ull : ((1ull << (16 * n)) - 1));
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      r.v[mt].x &= static_cast<uint32_t>(keep);
      r.v[mt].y &= static_cast<uint32_t>(keep >> 32);
    }
  }
  const bool over = x[0] > kRescaleThreshold || x[1] > kRescaleThreshold ||
                    x[2] > kRescaleThreshold || x[3] > kRescaleThreshold;
  if (__ballot(over)) {
    // Move the reference max of every head up to its max over everything seen so
    // far (always taken on a segment's first tile, where m = -inf and x = +inf).
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = (valid < kTile && tq + i >= valid) ? -INFINITY : sc[i] * c;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] *= alpha;
    st.l *= alpha;
    st.m = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = sv[i] - m_new;
  }
  bf16x4_t pb;
#pragma unroll
  for (int i = 0; i < 4; ++i) pb[i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(x[i]));
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
    st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, r.v[mt]), pb,
                                                         st.o[mt], 0, 0, 0);
  const bf16x4_t ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f),
                         static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  st.l = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones, pb, st.l, 0, 0, 0);
}

struct Ctx {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  const int32_t* __restrict__ tables;
  const int32_t* __restrict__ lens;
  uint16_t* __restrict__ out;
  float* __restrict__ ws;
};

// Position in a worker's stream of tiles: tile t of (sequence s, KV head g); L
// and T are the length and tile count of s, `start` the first unit of s.
struct Cursor {
  int64_t start;
  int32_t s, g, t, T, L;
};

__device__ __forceinline__ void advance(Cursor& c, const int32_t* __restrict__ lens,
                                        const DecodeDims& d, int32_t cap) {
  if (++c.t < c.T) return;
  c.t = 0;
  if (++c.g < d.Hkv) return;
  c.g = 0;
  c.start += static_cast<int64_t>(d.Hkv) * c.T;
  do {
    ++c.s;
    c.L = c.s < d.S ? clamp_len(lens[c.s], cap) : 1;  // past the batch only at the very end
  } while (c.L == 0);
  c.T = tiles_of(c.L);
}

template <int D, int B>
__device__ __forceinline__ void load_at(TileRegs<D, B>& r, const Ctx& cx, const DecodeDims& d,
                                        const Cursor& c, int lane) {
  constexpr int64_t kTileElems = static_cast<int64_t>(D) * B;
  PairCursor pc;
  pc.k = cx.k;
  pc.v = cx.v;
  pc.trow = cx.tables + static_cast<int64_t>(c.s) * d.M;
  pc.block_stride = kTileElems * d.Hkv;
  pc.head_off = kTileElems * c.g;
  pc.nb = d.NB;
  pc.nblk = (c.L + B - 1) / B;
  load_tile<D, B>(r, pc, c.t, lane);
}

// Score MFMA B operand: lane holds q[head lane%16][c*32 + (lane/16)*8 .. +7].
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qop)[D / 32], const Ctx& cx, const DecodeDims& d,
                                       const Cursor& c, int lane) {
  const int32_t h = lane & 15;
  if (h < d.G) {
    const uint16_t* qr =
        cx.q + (static_cast<int64_t>(c.s) * d.Hq + c.g * d.G + h) * D + (lane >> 4) * 8;
#pragma unroll
    for (int k = 0; k < D / 32; ++k)
      qop[k] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qr + k * 32));
  } else {
#pragma unroll
    for (int k = 0; k < D / 32; ++k) qop[k] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
  }
}

// End of a segment: the output rows when it covered the whole pair, else a partial
// record (O, then m, then l) in slot `rec`.
template <int D>
__device__ void finish_segment(const Ctx& cx, const DecodeDims& d, const SegState<D>& st,
                               const Cursor& c, bool whole, int64_t rec, int lane) {
  const int32_t h = lane & 15;
  if (h >= d.G) return;
  const float l_tot = st.l[0];
  if (whole) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow =
        cx.out + (static_cast<int64_t>(c.s) * d.Hq + c.g * d.G + h) * D + (lane >> 4) * 4;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      bf16x4_t y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = static_cast<__bf16>(st.o[mt][i] * inv);
      *reinterpret_cast<u32x2_t*>(orow + mt * 16) = __builtin_bit_cast(u32x2_t, y);
    }
  } else {
    float* base = cx.ws + rec * record_floats(d.G, D);
    float* orow = base + h * D + (lane >> 4) * 4;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) *reinterpret_cast<f32x4_t*>(orow + mt * 16) = st.o[mt];
    if (lane < 16) {
      base[d.G * D + h] = st.m;
      base[d.G * D + d.G + h] = l_tot;
    }
  }
}

// One worker: the tiles of units [u, u_end) in order, with loads running kPipe-1
// tiles ahead of the arithmetic across (sequence, head) boundaries; the query of a
// pair is fetched with the pair's first tile.  Returns the descriptor of the split
// pair this worker opens (s = -1 if none).
template <int D, int B>
__device__ int4 run_worker(const Ctx& cx, const DecodeDims& d, const WorkerPlan& pl, int64_t w,
                           int lane) {
  const int32_t cap = d.M * B;
  const int32_t n = static_cast<int32_t>(pl.u_end - pl.u);
  Cursor lc;
  lc.start = pl.start;
  lc.s = pl.s;
  lc.L = clamp_len(cx.lens[pl.s], cap);
  lc.T = tiles_of(lc.L);
  lc.g = static_cast<int32_t>((pl.u - pl.start) / lc.T);
  lc.t = static_cast<int32_t>((pl.u - pl.start) - static_cast<int64_t>(lc.g) * lc.T);
  Cursor cc = lc;

  TileRegs<D, B> r[kPipe];
  bf16x8_t qb[kPipe][D / 32];
  bf16x8_t qc[D / 32];
  SegState<D> st;
  int32_t seg_t0 = cc.t;
  int64_t rec = 2 * w;  // first segment -> slot 0, later ones -> slot 1
  int4 opened = {-1, 0, 0, 0};

  auto load_step = [&](int slot, int32_t li) {
    if (lc.t == 0 || li == 0) load_q<D>(qb[slot], cx, d, lc, lane);
    load_at<D, B>(r[slot], cx, d, lc, lane);
    advance(lc, cx.lens, d, cap);
  };
  auto compute_step = [&](int slot, int32_t i) {
    if (cc.t == 0 || i == 0) {
#pragma unroll
      for (int k = 0; k < D / 32; ++k) qc[k] = qb[slot][k];
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) st.o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st.l = f32x4_t{0.f, 0.f, 0.f, 0.f};
      st.m = -INFINITY;
      seg_t0 = cc.t;
    }
    compute_tile<D, B>(r[slot], qc, st, d.c, min(kTile, cc.L - cc.t * kTile), lane);
    if (cc.t == cc.T - 1 || i == n - 1) {
      const bool whole = seg_t0 == 0 && cc.t == cc.T - 1;
      finish_segment<D>(cx, d, st, cc, whole, rec, lane);
      if (!whole && seg_t0 == 0) {
        // this worker holds the first share of a pair that later workers continue
        const int64_t u0 = cc.start + static_cast<int64_t>(cc.g) * cc.T;
        opened = int4{cc.s, cc.g, static_cast<int32_t>(worker_of(u0 + cc.T - 1, pl.U, pl.N)),
                      static_cast<int32_t>(rec - 2 * w)};
      }
      rec = 2 * w + 1;
    }
    advance(cc, cx.lens, d, cap);
  };

#pragma unroll
  for (int k = 0; k < kPipe - 1; ++k)
    if (k < n) load_step(k, k);
  int32_t i = 0;
  // Whole groups of kPipe steps in which every step has a tile to load.
  while (i + 2 * kPipe - 1 <= n) {
#pragma unroll
    for (int k = 0; k < kPipe; ++k) {
      load_step((k + kPipe - 1) % kPipe, i + k + kPipe - 1);
      compute_step(k, i + k);
    }
    i += kPipe;
  }
  const int32_t rem = n - i;  // fewer than 2*kPipe-1 tiles left, kPipe-1 of them loading
#pragma unroll
  for (int k = 0; k < 2 * kPipe - 2; ++k) {
    if (k < rem) {
      if (k + kPipe - 1 < rem) load_step((k + kPipe - 1) % kPipe, i + k + kPipe - 1);
      compute_step(k % kPipe, i + k);
    }
  }
  return opened;
}

// The decode kernel.  Workspace: partial records ([n_workers][2] of
// record_floats), then one descriptor per worker: (s, g, wb, first_slot) of the
// split pair whose first share this worker holds, or s = -1.
template <int D, int B>
__global__ __launch_bounds__(kWave* kWavesPerGroup, 1) void decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ tables, const int32_t* __restrict__ lens,
    uint16_t* __restrict__ out, float* __restrict__ ws, int4* __restrict__ desc, DecodeDims d) {
  const Ctx cx{q, k, v, tables, lens, out, ws};
  const int lane = __lane_id();
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + uniform(threadIdx.x / kWave);
  if (w >= d.n_workers) return;
  const int32_t cap = d.M * B;

  int4 opened = {-1, 0, 0, 0};
  WorkerPlan pl;
  if (plan_worker(lens, d, cap, w, lane, pl)) opened = run_worker<D, B>(cx, d, pl, w, lane);

  // Rows of empty sequences are zeros (done last: off the path to the first loads).
  for (int64_t se = w; se < d.S; se += d.n_workers) {
    if (clamp_len(lens[se], cap) == 0) {
      uint16_t* row = out + se * d.Hq * D;
      for (int32_t i = lane * 8; i < d.Hq * D; i += kWave * 8)
        *reinterpret_cast<u32x4_t*>(row + i) = u32x4_t{0, 0, 0, 0};
    }
  }
  if (lane == 0) desc[w] = opened;
}

// Merge of split pairs.  Work-group b reads the descriptors of its slice of
// workers in one parallel pass and keeps the valid ones in LDS (each names a split
// pair opened by worker wa and closed by wb).  The (pair, output) items of those
// pairs are spread over the threads, kMergeItems per thread at a time; an item
// folds the records of wa..wb in worker order with a running max, kMergeChunk
// records per batch, and the loads of all of a thread's items are issued together.
// The order is fixed, so the result does not depend on timing.
constexpr int kMergeThreads = 512;
constexpr int kMergeChunk = 8;
constexpr int kMergeItems = 2;
constexpr int kMergeSlice = 64;  // most descriptors one work-group scans

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const int4* __restrict__ desc,
                                                              uint16_t* __restrict__ out,
                                                              const float* __restrict__ ws,
                                                              DecodeDims d) {
  __shared__ int4 s_desc[kMergeSlice];
  __shared__ int32_t s_wa[kMergeSlice];
  __shared__ int32_t s_count;
  const int tid = threadIdx.x;
  const int64_t per = (d.n_workers + gridDim.x - 1) / gridDim.x;
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * per;
  const int64_t w1 = min(w0 + per, static_cast<int64_t>(d.n_workers));
  if (tid == 0) s_count = 0;
  __syncthreads();
  if (w0 + tid < w1) {
    const int4 ds = desc[w0 + tid];
    if (ds.x >= 0) {
      const int32_t slot = atomicAdd(&s_count, 1);
      s_desc[slot] = ds;
      s_wa[slot] = static_cast<int32_t>(w0 + tid);
    }
  }
  __syncthreads();
  const int64_t rf = record_floats(d.G, D);
  const int32_t GD = d.G * D;
  const int32_t total = s_count * GD;
  for (int32_t base = tid; base < total; base += kMergeThreads * kMergeItems) {
    float run_m[kMergeItems], run_l[kMergeItems], acc[kMergeItems];
    int64_t wa[kMergeItems], wb[kMergeItems], first[kMergeItems];
    int32_t pi[kMergeItems], oi[kMergeItems];
#pragma unroll
    for (int it = 0; it < kMergeItems; ++it) {
      const int32_t item = base + it * kMergeThreads;
      run_m[it] = -INFINITY;
      run_l[it] = 0.f;
      acc[it] = 0.f;
      pi[it] = item < total ? item / GD : 0;
      oi[it] = item < total ? item - pi[it] * GD : 0;
      wa[it] = s_wa[pi[it]];
      wb[it] = item < total ? static_cast<int64_t>(s_desc[pi[it]].z) : wa[it] - 1;  // none
      first[it] = (2 * wa[it] + s_desc[pi[it]].w) * rf;
    }
    int64_t kmax = 0;
#pragma unroll
    for (int it = 0; it < kMergeItems; ++it) kmax = max(kmax, wb[it] - wa[it] + 1);
    for (int64_t c = 0; c < kmax; c += kMergeChunk) {
      float m[kMergeItems][kMergeChunk], l[kMergeItems][kMergeChunk], o[kMergeItems][kMergeChunk];
#pragma unroll
      for (int it = 0; it < kMergeItems; ++it) {
        const int32_t h = oi[it] / D;
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
          const int64_t wk = wa[it] + c + k;
          if (wk <= wb[it]) {
            const float* rec = ws + (c + k == 0 ? first[it] : 2 * wk * rf);
            m[it][k] = rec[GD + h];
            l[it][k] = rec[GD + d.G + h];
            o[it][k] = rec[oi[it]];
          } else {
            m[it][k] = -INFINITY;
            l[it][k] = 0.f;
            o[it][k] = 0.f;
          }
        }
      }
#pragma unroll
      for (int it = 0; it < kMergeItems; ++it) {
        float cm = run_m[it];
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) cm = fmaxf(cm, m[it][k]);
        if (cm == -INFINITY) continue;  // item past the end, or no record in this chunk
        const float scale = __builtin_amdgcn_exp2f(run_m[it] - cm);
        run_l[it] *= scale;
        acc[it] *= scale;
        run_m[it] = cm;
#pragma unroll
        for (int k = 0; k < kMergeChunk; ++k) {
          const float e = __builtin_amdgcn_exp2f(m[it][k] - cm);
          run_l[it] += e * l[it][k];
          acc[it] += e * o[it][k];
        }
      }
    }
#pragma unroll
    for (int it = 0; it < kMergeItems; ++it) {
      if (base + it * kMergeThreads < total) {
        const int4 ds = s_desc[pi[it]];
        out[(static_cast<int64_t>(ds.x) * d.Hq + ds.y * d.G) * D + oi[it]] =
            __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[it] / run_l[it]));
      }
    }
  }
}

template <int D, int B>
hipError_t launch_t(const DecodeBuffers& b, const DecodeDims& d, int merge_groups,
                    hipStream_t stream) {
  const int groups = (d.n_workers + kWavesPerGroup - 1) / kWavesPerGroup;
  if (groups <= 0) return hipSuccess;
  int4* desc = reinterpret_cast<int4*>(reinterpret_cast<char*>(b.ws) +
                                       records_bytes(d.n_workers, d.G, D));
  hipLaunchKernelGGL((decode_kernel<D, B>), dim3(groups), dim3(kWave * kWavesPerGroup), 0, stream,
                     b.q, b.k, b.v, b.tables, b.lens, b.out, b.ws, desc, d);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((merge_kernel<D>), dim3(merge_groups), dim3(kMergeThreads), 0, stream, desc,
                     b.out, b.ws, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeBuffers& b, const DecodeDims& d, int D, int B,
                         int merge_groups, hipStream_t stream) {
  if (D == 128) {
    if (B == 16) return launch_t<128, 16>(b, d, merge_groups, stream);
    if (B == 32) return launch_t<128, 32>(b, d, merge_groups, stream);
    if (B == 8) return launch_t<128, 8>(b, d, merge_groups, stream);
  } else if (D == 64) {
    if (B == 16) return launch_t<64, 16>(b, d, merge_groups, stream);
    if (B == 32) return launch_t<64, 32>(b, d, merge_groups, stream);
    if (B == 8) return launch_t<64, 8>(b, d, merge_groups, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
