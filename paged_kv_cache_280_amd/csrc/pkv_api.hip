// C ABI of the library (declared in include/pkv.h): host-side argument checks,
// launch sizing and dispatch to the kernels.  No call allocates device memory; the
// one static array below is the scratch of the no-allocation decode entry point.

#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>

#include "pkv.h"
#include "pkv_internal.h"

// Scratch of paged_attn_decode_noalloc: split-K records and worker descriptors.
// Every device the library runs on holds its own copy until the process ends.  On
// the host this name only stands for the array: host code uses the device address
// that hipGetSymbolAddress reports for the current device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace pkv {
namespace {

constexpr int kMaxDevices = 64;
// Resident decode workers per CU, measured best: 3 for bf16 pools (the HBM stream
// saturates with 768 waves), 4 for fp8 pools (half the bytes per tile).
constexpr int kDefaultWavesPerCu = 3;
constexpr int kDefaultWavesPerCuFp8 = 4;

// Compute units of each device, read once (0 = not read yet).
std::atomic<int> g_cu_count[kMaxDevices];

int current_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    return -1;
  if (dev < kMaxDevices) g_cu_count[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

// Device address of the current device's scratch array, looked up once per device
// (with that device current) and kept; nullptr when the runtime cannot report it.
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

void* noalloc_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    g_scratch[dev].store(addr, std::memory_order_release);
    p = addr;
  }
  return p;
}

// Resident decode workers (waves) per compute unit; PKV_WAVES_PER_CU overrides
// the defaults for launch-shape sweeps.
int waves_per_cu(bool fp8) {
  static const int v = [] {
    const char* e = getenv("PKV_WAVES_PER_CU");
    const int x = e ? atoi(e) : 0;
    return (x >= 1 && x <= 32) ? x : 0;
  }();
  return v ? v : (fp8 ? kDefaultWavesPerCuFp8 : kDefaultWavesPerCu);
}

// Pair mode (one worker per (sequence, KV head) pair, no split, no merge kernel)
// for batches of short contexts: at most kPairModeTiles tiles per pair and no more
// pairs than resident worker slots.  PKV_PAIR_MODE=0 or 1 forces it off or on
// (when legal) for measurements.
constexpr int64_t kPairModeTiles = 16;

bool use_pair_mode(int cu, int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                   bool fp8) {
  static const int forced = [] {
    const char* e = getenv("PKV_PAIR_MODE");
    return e ? atoi(e) : -1;
  }();
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  const int64_t tiles = (static_cast<int64_t>(max_context_len) + kTile - 1) / kTile;
  const bool legal = pairs <= static_cast<int64_t>(cu) * waves_per_cu(fp8) * 2;
  if (forced >= 0) return forced == 1 && legal;
  return legal && tiles <= kPairModeTiles && pairs <= static_cast<int64_t>(cu) * waves_per_cu(fp8);
}

bool supported_head_dim(int32_t d) { return d == 64 || d == 128; }
bool supported_block_size(int32_t b) { return b == 8 || b == 16 || b == 32; }

// Number of decode workers: one per resident wave slot, never more than the
// tiles a batch bounded by max_context_len can hold.
int64_t worker_count(int cu, int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                     bool fp8 = false) {
  const int64_t tiles_bound = static_cast<int64_t>(num_seqs) * num_kv_heads *
                              ((static_cast<int64_t>(max_context_len) + kTile - 1) / kTile);
  int64_t n = static_cast<int64_t>(cu) * waves_per_cu(fp8);
  if (tiles_bound < n) n = tiles_bound;
  return n < 1 ? 1 : n;
}

size_t workspace_for(int64_t workers, int32_t group, int32_t head_dim) {
  return static_cast<size_t>(workspace_bytes_for(workers, group, head_dim));
}

// Merge work-groups: one per compute unit, each scanning at most 64 worker slots.
int merge_groups_for(int64_t workers, int cu) {
  int64_t g = workers < cu ? workers : cu;
  if (g * 64 < workers) g = (workers + 63) / 64;
  return static_cast<int>(g);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Pool form of a call: 2 when v_cache starts one (block, head) tile after k_cache,
// the two halves of one pool whose entries hold a K tile and then a V tile; else
// 1, two separate pools.  Separate pools of more than one tile cannot start one
// tile apart (V would begin inside K), and over a single tile both readings
// address the same bytes, so the form needs no flag of its own.
int32_t pool_form(const void* k, const void* v, int32_t head_dim, int32_t block_size, bool fp8) {
  const uintptr_t tile = static_cast<uintptr_t>(head_dim) * block_size * (fp8 ? 1u : 2u);
  return reinterpret_cast<uintptr_t>(v) == reinterpret_cast<uintptr_t>(k) + tile ? 2 : 1;
}

int32_t check_shapes(int32_t block_size, float scale, int32_t num_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                     int64_t num_blocks, int32_t max_context_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || max_context_len < 0 || !isfinite(scale))
    return PKV_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size)) return PKV_ERR_UNSUPPORTED;
  if (num_q_heads / num_kv_heads > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  // the work plan counts a row's units in 32-bit lane scans
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > kMaxRowPositions)
    return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Work units of a tile and of a pair's query and output rows (rows * head_dim * 2
// bytes each way).  Batches of more than 64 sequences weigh pairs: a tile is 4
// units and the rows count in quarters of a tile's K/V bytes (16 positions *
// head_dim * 2 bytes, bf16; half that for fp8), plus kPairFixedUnits for what a
// pair costs whatever its rows (switching the stream to it, its query fetch, the
// rounding and store of its output).  Smaller batches count tiles only (measured:
// the weighting moves nothing there and the lighter plan starts the first loads
// sooner).
//
// kPairFixedUnits measured on the continuous-batching mix (256 sequences, 2,048
// pairs): workers holding 20+ short pairs finished ~12 us after single-pair
// workers with rows alone; 3 to 5 extra units level them (3 and 4 best): bf16
// 384.8 -> 381 us (B = 16) and 392 -> 383 us (B = 32), fp8 222.8 -> 216 / 213 us.
constexpr int32_t kPairFixedUnits = 3;

void set_units(DecodeDims& d, int32_t rows, bool fp8) {
  const bool weigh = d.S > kWave;
  d.unit = weigh ? 4 : 1;
  d.hdr = weigh ? (fp8 ? (rows + 1) / 2 : (rows + 2) / 4) + kPairFixedUnits : 0;
}

// fp8: the pools hold E4M3FN codes; keys are code * k_scale, values code * v_scale.
int32_t decode_impl(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t block_size,
                    float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int64_t num_blocks, int32_t max_context_len, void* workspace,
                    size_t workspace_bytes, void* stream, bool fp8, float k_scale,
                    float v_scale, const void* k_new = nullptr, const void* v_new = nullptr) {
  const bool append = k_new != nullptr || v_new != nullptr;
  const int32_t st = check_shapes(block_size, scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  max_blocks_per_seq, num_blocks, max_context_len);
  if (st != PKV_OK) return st;
  if (!isfinite(k_scale) || !isfinite(v_scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !workspace)
    return PKV_ERR_NULL;
  if (append && (!k_new || !v_new)) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return PKV_ERR_ALIGNMENT;
  if (append && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGNMENT;
  const int cu = current_cu_count();
  if (cu <= 0) return PKV_ERR_DEVICE;
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t workers = worker_count(cu, num_seqs, num_kv_heads, max_context_len, fp8);
  if (workspace_bytes < workspace_for(workers, group, head_dim)) return PKV_ERR_WORKSPACE;

  DecodeBuffers b{};
  b.q = static_cast<const uint16_t*>(q);
  b.k = k_cache;
  b.v = v_cache;
  b.tables = block_tables;
  b.lens = context_lens;
  b.qlens = nullptr;
  b.out = static_cast<uint16_t*>(out);
  b.ws = static_cast<float*>(workspace);
  if (append) {
    b.k_new = static_cast<const uint16_t*>(k_new);
    b.v_new = static_cast<const uint16_t*>(v_new);
    b.kw = const_cast<void*>(k_cache);
    b.vw = const_cast<void*>(v_cache);
  }
  DecodeDims d{};
  d.S = num_seqs;
  d.Hq = num_q_heads;
  d.Hkv = num_kv_heads;
  d.G = group;
  d.M = max_blocks_per_seq;
  d.pair_mode = use_pair_mode(cu, num_seqs, num_kv_heads, max_context_len, fp8) ? 1 : 0;
  d.n_workers = d.pair_mode ? num_seqs * num_kv_heads : static_cast<int32_t>(workers);
  d.NB = num_blocks;
  d.kv_mul = pool_form(k_cache, v_cache, head_dim, block_size, fp8);
  // scores in the log2 domain; an fp8 K pool's scale folds into the same factor
  d.c = static_cast<float>(static_cast<double>(scale) * static_cast<double>(k_scale) *
                           1.4426950408889634);  // log2(e)
  d.Qmax = 1;
  d.Qc = 1;
  d.q_off = 0;
  d.R = group;
  set_units(d, group, fp8);
  d.v_scale = v_scale;
  d.k_scale = k_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Decode with append over bf16 pools folds each pair's newest position into the
  // worker holding its last tile, which reads the new rows once per pair it closes.
  // When workers hold several pairs each that costs more than one more launch, and
  // over fp8 pools it always does (the encoding's registers push the tile loop into
  // spills: long context 2.23 against 1.89 ms per 32-layer step, chat 0.71 against
  // 0.56 ms): then the rows are written by the append kernel first and a plain
  // decode follows (same results up to rounding, same pools).
  const bool fused = append && !fp8 &&
                     (d.pair_mode || static_cast<int64_t>(num_seqs) * num_kv_heads <= d.n_workers);
  if (append && !fused) {
    AppendBuffers ab{};
    ab.k_new = static_cast<const uint16_t*>(k_new);
    ab.v_new = static_cast<const uint16_t*>(v_new);
    ab.k_cache = const_cast<void*>(k_cache);
    ab.v_cache = const_cast<void*>(v_cache);
    ab.tables = block_tables;
    ab.token_pos = context_lens;
    AppendDims ad{};
    ad.T = num_seqs;
    ad.S = num_seqs;
    ad.Hkv = num_kv_heads;
    ad.B = block_size;
    ad.M = max_blocks_per_seq;
    ad.NB = num_blocks;
    ad.kv_mul = pool_form(k_cache, v_cache, head_dim, block_size, fp8);
    ad.k_scale = k_scale;
    ad.v_scale = v_scale;
    ad.newest = 1;
    if ((fp8 ? launch_append_fp8(ab, ad, head_dim, s) : launch_append(ab, ad, head_dim, s)) !=
        hipSuccess)
      return PKV_ERR_LAUNCH;
  }
  d.len_off = fused ? 1 : 0;
  const int mg = merge_groups_for(workers, cu);
  const hipError_t e = fused ? launch_decode_append(b, d, head_dim, block_size, mg, s)
                       : fp8 ? launch_decode_fp8(b, d, head_dim, block_size, mg, s)
                             : launch_decode(b, d, head_dim, block_size, mg, s);
  if (e != hipSuccess) return PKV_ERR_LAUNCH;
  return PKV_OK;
}

// Query tokens of one chunk (one wave's rows): as many as fill two 16-column MFMA
// tiles (kMaxRows), or one when no context exceeds kShortContext positions (at
// least one token, never more than max_query_len).  Measured at G = 4: the chat
// batch (64 sequences of 114..1,500 positions) takes 76.7 us per call at 8 query
// tokens with one 32-row chunk and 71.1 us with two 16-row chunk waves (16 tokens:
// 103.1 against 98.7 us); 8 x 16,000 positions take 93.7 against 103.1 us at 8
// tokens and 112.0 against 171.4 us at 16.  Short pairs switch often, and one
// column tile keeps a deeper tile pipeline.
constexpr int32_t kShortContext = 2048;

int32_t tokens_per_launch(int32_t group, int32_t max_query_len, int32_t max_context_len) {
  const int32_t rows = max_context_len <= kShortContext ? 16 : kMaxRows;
  const int32_t t = rows / group > 0 ? rows / group : 1;
  return t < max_query_len ? t : max_query_len;
}

// Chunks of `per` query tokens one multi-token launch takes, given `left` still
// to do: 1, 2 or 4, so that a slot's waves sit in one work-group (three take a
// launch of four whose last chunk is empty).
int32_t chunks_per_launch(int32_t left) { return left >= 3 ? 4 : left; }

// Slots (planned tile ranges) of a multi-token launch of nch chunks: the
// resident waves shared out nch to a slot, never more slots than the tiles a
// batch bounded by max_context_len can hold.  Launches whose slots have two or
// four waves fill every compute unit (a work-group of four waves each): their
// waves compute more per byte fetched, and measured on 8 x 16,000 positions at
// G = 4 the extra quarter of the compute units takes 16 query tokens from 146 to
// 120 us and 32 from 263 to 205 us (one-chunk launches: no change).
int64_t multi_slots(int cu, int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                    bool fp8, int32_t nch) {
  const int64_t tiles_bound = static_cast<int64_t>(num_seqs) * num_kv_heads *
                              ((static_cast<int64_t>(max_context_len) + kTile - 1) / kTile);
  const int wpc = nch > 1 ? std::max(waves_per_cu(fp8), kWavesPerGroup) : waves_per_cu(fp8);
  int64_t n = static_cast<int64_t>(cu) * wpc / nch;
  if (tiles_bound < n) n = tiles_bound;
  return n < 1 ? 1 : n;
}

// Most waves any launch of the call runs (records and descriptors are per wave).
int64_t multi_waves(int cu, int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                    bool fp8) {
  int64_t w = 0;
  for (int32_t nch = 1; nch <= 4; nch *= 2)
    w = std::max(w, nch * multi_slots(cu, num_seqs, num_kv_heads, max_context_len, fp8, nch));
  return w;
}

size_t multi_workspace_for(int64_t waves, int32_t group, int32_t head_dim, int32_t max_query_len,
                           int32_t max_context_len) {
  return static_cast<size_t>(workspace_bytes_for(
      waves, group * tokens_per_launch(group, max_query_len, max_context_len), head_dim));
}

int32_t multi_impl(const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_lens, int32_t max_query_len, int32_t block_size,
                   float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                   int64_t num_blocks, int32_t max_context_len, void* workspace,
                   size_t workspace_bytes, void* stream, bool fp8, float k_scale,
                   float v_scale) {
  const int32_t st = check_shapes(block_size, scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  max_blocks_per_seq, num_blocks, max_context_len);
  if (st != PKV_OK) return st;
  if (max_query_len < 0) return PKV_ERR_SHAPE;
  if (!isfinite(k_scale) || !isfinite(v_scale)) return PKV_ERR_SHAPE;
  if (num_seqs == 0 || max_query_len == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_lens || !out ||
      !workspace)
    return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return PKV_ERR_ALIGNMENT;
  const int cu = current_cu_count();
  if (cu <= 0) return PKV_ERR_DEVICE;
  const int32_t group = num_q_heads / num_kv_heads;
  if (workspace_bytes < multi_workspace_for(multi_waves(cu, num_seqs, num_kv_heads,
                                                       max_context_len, fp8),
                                           group, head_dim, max_query_len, max_context_len))
    return PKV_ERR_WORKSPACE;

  DecodeDims d{};
  d.S = num_seqs;
  d.Hq = num_q_heads;
  d.Hkv = num_kv_heads;
  d.G = group;
  d.M = max_blocks_per_seq;
  d.pair_mode = use_pair_mode(cu, num_seqs, num_kv_heads, max_context_len, fp8) ? 1 : 0;
  d.NB = num_blocks;
  d.kv_mul = pool_form(k_cache, v_cache, head_dim, block_size, fp8);
  d.c = static_cast<float>(static_cast<double>(scale) * static_cast<double>(k_scale) *
                           1.4426950408889634);  // log2(e); an fp8 K scale folds in
  d.Qmax = max_query_len;
  d.v_scale = v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t per = tokens_per_launch(group, max_query_len, max_context_len);
  const int64_t token_elems = static_cast<int64_t>(num_q_heads) * head_dim;
  // One launch pair (attention, merge) per run of up to four chunks of `per`
  // query tokens: the chunk waves of a slot walk one tile range together, so a
  // K/V tile is fetched from memory once for all of the run's tokens.
  for (int32_t off = 0; off < max_query_len;) {
    const int32_t left = (max_query_len - off + per - 1) / per;
    d.nch = chunks_per_launch(left);
    d.q_off = off;
    d.Qc = per < max_query_len - off ? per : max_query_len - off;
    d.R = group * d.Qc;
    d.n_workers = d.pair_mode ? num_seqs * num_kv_heads
                              : static_cast<int32_t>(multi_slots(cu, num_seqs, num_kv_heads,
                                                                 max_context_len, fp8, d.nch));
    set_units(d, d.R, fp8);
    DecodeBuffers b{};
    b.q = static_cast<const uint16_t*>(q) + off * token_elems;
    b.k = k_cache;
    b.v = v_cache;
    b.tables = block_tables;
    b.lens = context_lens;
    b.qlens = query_lens;
    b.out = static_cast<uint16_t*>(out) + off * token_elems;
    b.ws = static_cast<float*>(workspace);
    if (launch_multi(b, d, head_dim, block_size,
                     merge_groups_for(static_cast<int64_t>(d.n_workers) * d.nch, cu), s,
                     fp8) != hipSuccess)
      return PKV_ERR_LAUNCH;
    off += d.nch * per;
  }
  return PKV_OK;
}

// Shared-prefix decode runs its two passes side by side in one launch, each with
// about half of the compute units' worker slots (a work-group of four waves per
// CU between them).
// Workspace: the prefix pass's records and descriptors (its workers', then one
// per (group, KV head) pair), the tail pass's (its workers', then one per
// (sequence, KV head) pair), the prefix states (one record of
// record_floats(num_q_heads, head_dim) floats per sequence), then the member map
// (two int32 per sequence); each part 256-byte aligned.
struct SharedLayout {
  int64_t workers_prefix, workers_tail;
  int32_t rows_prefix;
  int64_t tail_off, state_off, gmap_off, bytes;
};

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

SharedLayout shared_layout(int cu, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t max_context_len, int32_t num_groups,
                           int32_t max_group_size, int32_t max_prefix_len) {
  SharedLayout l;
  const int32_t group = num_q_heads / num_kv_heads;
  l.rows_prefix = group * max_group_size;
  // PKV_SHARED_WAVES=total,prefix overrides the split for launch-shape sweeps
  static const std::pair<int, int> forced = [] {
    const char* e = getenv("PKV_SHARED_WAVES");
    int t = 0, p = 0;
    if (e && sscanf(e, "%d,%d", &t, &p) == 2 && t > p && p > 0) return std::make_pair(t, p);
    return std::make_pair(0, 0);
  }();
  const int64_t half = static_cast<int64_t>(cu) * kWavesPerGroup / 2;
  const int64_t tiles_prefix = static_cast<int64_t>(num_groups) * num_kv_heads *
                               ((static_cast<int64_t>(max_prefix_len) + kTile - 1) / kTile);
  const int64_t tiles_tail = static_cast<int64_t>(num_seqs) * num_kv_heads *
                             ((static_cast<int64_t>(max_context_len) + kTile - 1) / kTile);
  const int64_t total = forced.first > 0 ? forced.first : 2 * half;
  const int64_t want_prefix = forced.first > 0 ? forced.second : half;
  l.workers_prefix = std::max<int64_t>(1, std::min(want_prefix, tiles_prefix));
  l.workers_tail = std::max<int64_t>(1, std::min(total - l.workers_prefix, tiles_tail));
  const int64_t pairs = static_cast<int64_t>(num_seqs) * num_kv_heads;
  const int64_t group_pairs = static_cast<int64_t>(num_groups) * num_kv_heads;
  l.tail_off =
      align256(workspace_bytes_for(l.workers_prefix + group_pairs, l.rows_prefix, head_dim));
  l.state_off = align256(l.tail_off + workspace_bytes_for(l.workers_tail + pairs, group, head_dim));
  l.gmap_off = align256(l.state_off + static_cast<int64_t>(num_seqs) *
                                          record_floats(num_q_heads, head_dim) *
                                          static_cast<int64_t>(sizeof(float)));
  l.bytes = l.gmap_off + static_cast<int64_t>(num_seqs) * 2 * static_cast<int64_t>(sizeof(int32_t));
  return l;
}

int32_t check_shared(int32_t num_q_heads, int32_t num_kv_heads, int32_t num_seqs,
                     int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len,
                     int32_t max_context_len) {
  if (num_groups < 0 || max_group_size <= 0 || max_prefix_len < 0 ||
      max_prefix_len > max_context_len || (num_seqs > 0 && num_groups == 0))
    return PKV_ERR_SHAPE;
  if ((num_q_heads / num_kv_heads) * max_group_size > kMaxRows) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

int32_t shared_impl(const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* group_first, const int32_t* prefix_lens, int32_t num_groups,
                    int32_t max_group_size, int32_t max_prefix_len, int32_t block_size,
                    float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int64_t num_blocks, int32_t max_context_len, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int32_t st = check_shapes(block_size, scale, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_blocks_per_seq, num_blocks, max_context_len);
  if (st != PKV_OK) return st;
  st = check_shared(num_q_heads, num_kv_heads, num_seqs, num_groups, max_group_size,
                    max_prefix_len, max_context_len);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !group_first ||
      !prefix_lens || !out || !workspace)
    return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return PKV_ERR_ALIGNMENT;
  const int cu = current_cu_count();
  if (cu <= 0) return PKV_ERR_DEVICE;
  const SharedLayout lay = shared_layout(cu, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len, num_groups, max_group_size,
                                         max_prefix_len);
  if (static_cast<int64_t>(workspace_bytes) < lay.bytes) return PKV_ERR_WORKSPACE;
  const int32_t group = num_q_heads / num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);

  DecodeBuffers b{};
  b.q = static_cast<const uint16_t*>(q);
  b.k = k_cache;
  b.v = v_cache;
  b.tables = block_tables;
  b.out = static_cast<uint16_t*>(out);
  b.ws = static_cast<float*>(workspace);
  b.state = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.state_off);
  DecodeDims d{};
  d.Hq = num_q_heads;
  d.Hkv = num_kv_heads;
  d.G = group;
  d.M = max_blocks_per_seq;
  d.NB = num_blocks;
  d.kv_mul = pool_form(k_cache, v_cache, head_dim, block_size, false);
  d.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);  // log2(e)
  d.v_scale = 1.0f;
  d.k_scale = 1.0f;
  d.pre_align = block_size > kTile ? block_size : kTile;
  d.pre_cap = max_prefix_len;
  d.seqs = num_seqs;

  const bool prefix_pass = max_prefix_len >= d.pre_align && num_groups > 0;
  if (!prefix_pass) d.pre_cap = 0;  // no prefix anywhere: the tail pass is a plain decode

  // tail pass: every sequence from its prefix on, each segment from an empty
  // state; its merge starts each pair that has a prefix from that prefix
  DecodeBuffers bt = b;
  bt.lens = context_lens;
  bt.qlens = prefix_lens;
  bt.ws = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.tail_off);
  DecodeDims dt = d;
  dt.S = num_seqs;
  dt.pair_mode = 0;
  dt.n_workers = static_cast<int32_t>(lay.workers_tail);
  dt.Qmax = 1;
  dt.Qc = 1;
  dt.q_off = 0;
  dt.R = group;
  set_units(dt, group, false);
  const int mgt = merge_groups_for(dt.n_workers, cu);
  if (!prefix_pass) {
    if (launch_shared_tail(bt, dt, head_dim, block_size, mgt, s) != hipSuccess)
      return PKV_ERR_LAUNCH;
    return PKV_OK;
  }
  // prefix pass: group v's members are its T query tokens (rows member * G + head);
  // whole prefix pairs leave prefix states, split ones records, for the tail merge
  DecodeBuffers bp = b;
  bp.lens = prefix_lens;
  bp.qlens = group_first;
  DecodeDims a = d;
  a.S = num_groups;
  a.pair_mode = use_pair_mode(cu, num_groups, num_kv_heads, max_prefix_len, false) ? 1 : 0;
  a.n_workers = a.pair_mode ? num_groups * num_kv_heads : static_cast<int32_t>(lay.workers_prefix);
  a.Qmax = max_group_size;
  a.Qc = max_group_size;
  a.q_off = 0;
  a.R = lay.rows_prefix;
  set_units(a, a.R, false);
  int32_t* gmap = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + lay.gmap_off);
  if (launch_shared(bp, a, bt, dt, head_dim, block_size, gmap, mgt, s) != hipSuccess)
    return PKV_ERR_LAUNCH;
  return PKV_OK;
}

int32_t append_impl(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                    const int32_t* block_tables, const int32_t* token_seq,
                    const int32_t* token_pos, int32_t num_tokens, int32_t num_seqs,
                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t max_blocks_per_seq, int64_t num_blocks, void* stream, bool fp8,
                    float k_scale, float v_scale) {
  if (num_tokens < 0 || num_seqs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0)
    return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > 0x7fffffffLL) return PKV_ERR_SHAPE;
  if (!isfinite(k_scale) || !isfinite(v_scale) || k_scale == 0.0f || v_scale == 0.0f)
    return PKV_ERR_SHAPE;
  if (!supported_head_dim(head_dim) || !supported_block_size(block_size))
    return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !k_cache || !v_cache || !block_tables || !token_seq || !token_pos)
    return PKV_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_ERR_ALIGNMENT;
  AppendBuffers b{};
  b.k_new = static_cast<const uint16_t*>(k_new);
  b.v_new = static_cast<const uint16_t*>(v_new);
  b.k_cache = k_cache;
  b.v_cache = v_cache;
  b.tables = block_tables;
  b.token_seq = token_seq;
  b.token_pos = token_pos;
  AppendDims a{};
  a.T = num_tokens;
  a.S = num_seqs;
  a.Hkv = num_kv_heads;
  a.B = block_size;
  a.M = max_blocks_per_seq;
  a.NB = num_blocks;
  a.kv_mul = pool_form(k_cache, v_cache, head_dim, block_size, fp8);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = fp8 ? launch_append_fp8(b, a, head_dim, s) : launch_append(b, a, head_dim, s);
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // namespace
}  // namespace pkv

extern "C" {

int32_t pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int32_t status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "inconsistent sizes";
    case PKV_ERR_UNSUPPORTED: return "head_dim, block_size or group size not supported";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_ALIGNMENT: return "a buffer is not 16-byte aligned";
    case PKV_ERR_DEVICE: return "could not query the current HIP device";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t max_context_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0 || !pkv::supported_head_dim(head_dim) ||
      !pkv::supported_block_size(block_size) || num_q_heads / num_kv_heads > pkv::kMaxGroup)
    return 0;
  const int cu = pkv::current_cu_count();
  if (cu <= 0) return 0;
  // enough for either pool format (fp8 decode launches more workers)
  const int64_t workers =
      std::max(pkv::worker_count(cu, num_seqs, num_kv_heads, max_context_len, false),
               pkv::worker_count(cu, num_seqs, num_kv_heads, max_context_len, true));
  return pkv::workspace_for(workers, num_q_heads / num_kv_heads, head_dim);
}

size_t paged_attn_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_context_len,
                                                int32_t num_groups, int32_t max_group_size,
                                                int32_t max_prefix_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0 || !pkv::supported_head_dim(head_dim) ||
      !pkv::supported_block_size(block_size) || num_q_heads / num_kv_heads > pkv::kMaxGroup)
    return 0;
  if (pkv::check_shared(num_q_heads, num_kv_heads, num_seqs, num_groups, max_group_size,
                        max_prefix_len, max_context_len) != PKV_OK)
    return 0;
  const int cu = pkv::current_cu_count();
  if (cu <= 0) return 0;
  return static_cast<size_t>(pkv::shared_layout(cu, num_seqs, num_q_heads, num_kv_heads,
                                                head_dim, max_context_len, num_groups,
                                                max_group_size, max_prefix_len)
                                 .bytes);
}

int32_t paged_attn_decode_shared(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* group_first, const int32_t* prefix_lens,
                                 int32_t num_groups, int32_t max_group_size,
                                 int32_t max_prefix_len, int32_t block_size, float scale,
                                 void* out, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return pkv::shared_impl(q, k_cache, v_cache, block_tables, context_lens, group_first,
                          prefix_lens, num_groups, max_group_size, max_prefix_len, block_size,
                          scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                          max_blocks_per_seq, num_blocks, max_context_len, workspace,
                          workspace_bytes, stream);
}

int32_t paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t block_size, float scale, void* out, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int64_t num_blocks,
                          int32_t max_context_len, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return pkv::decode_impl(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          num_blocks, max_context_len, workspace, workspace_bytes, stream, false,
                          1.0f, 1.0f);
}

int32_t paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t block_size, float scale, void* out, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_context_len, void* stream) {
  // Sizes are checked before the device is asked for anything.  The scratch stands
  // in for the workspace; decode_impl rejects sizes that need more
  // (PKV_ERR_WORKSPACE) before anything is enqueued.
  const int32_t st = pkv::check_shapes(block_size, scale, num_seqs, num_q_heads, num_kv_heads,
                                       head_dim, max_blocks_per_seq, num_blocks, max_context_len);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return PKV_OK;
  void* ws = pkv::noalloc_scratch();
  if (!ws) return PKV_ERR_DEVICE;
  return pkv::decode_impl(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          num_blocks, max_context_len, ws, PKV_NOALLOC_SCRATCH_BYTES, stream,
                          false, 1.0f, 1.0f);
}

int32_t paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t block_size, float scale, float k_scale, float v_scale,
                              void* out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t max_context_len, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return pkv::decode_impl(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          num_blocks, max_context_len, workspace, workspace_bytes, stream, true,
                          k_scale, v_scale);
}

int32_t paged_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t block_size, float scale,
                                 void* out, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
  return pkv::decode_impl(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          num_blocks, max_context_len, workspace, workspace_bytes, stream, false,
                          1.0f, 1.0f, k_new, v_new);
}

int32_t paged_attn_decode_append_fp8(const void* q, const void* k_new, const void* v_new,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t block_size, float scale,
                                     float k_scale, float v_scale, void* out, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t max_context_len, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
  if (k_scale == 0.0f || v_scale == 0.0f) return PKV_ERR_SHAPE;  // new rows are divided by them
  return pkv::decode_impl(q, k_cache, v_cache, block_tables, context_lens, block_size, scale, out,
                          num_seqs, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq,
                          num_blocks, max_context_len, workspace, workspace_bytes, stream, true,
                          k_scale, v_scale, k_new, v_new);
}

size_t paged_attn_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len,
                                        int32_t max_query_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      max_query_len < 0 || num_q_heads % num_kv_heads != 0 || !pkv::supported_head_dim(head_dim) ||
      !pkv::supported_block_size(block_size) || num_q_heads / num_kv_heads > pkv::kMaxGroup)
    return 0;
  const int cu = pkv::current_cu_count();
  if (cu <= 0) return 0;
  // enough for either pool format (fp8 launches more workers)
  const int64_t waves =
      std::max(pkv::multi_waves(cu, num_seqs, num_kv_heads, max_context_len, false),
               pkv::multi_waves(cu, num_seqs, num_kv_heads, max_context_len, true));
  return pkv::multi_workspace_for(waves, num_q_heads / num_kv_heads, head_dim,
                                  max_query_len > 0 ? max_query_len : 1, max_context_len);
}

int32_t paged_attn_multi(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_lens, int32_t max_query_len, int32_t block_size,
                         float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int64_t num_blocks, int32_t max_context_len, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return pkv::multi_impl(q, k_cache, v_cache, block_tables, context_lens, query_lens,
                         max_query_len, block_size, scale, out, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, max_context_len,
                         workspace, workspace_bytes, stream, false, 1.0f, 1.0f);
}

int32_t paged_attn_multi_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const int32_t* query_lens, int32_t max_query_len, int32_t block_size,
                             float scale, float k_scale, float v_scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return pkv::multi_impl(q, k_cache, v_cache, block_tables, context_lens, query_lens,
                         max_query_len, block_size, scale, out, num_seqs, num_q_heads,
                         num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, max_context_len,
                         workspace, workspace_bytes, stream, true, k_scale, v_scale);
}

int32_t kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* block_tables, const int32_t* token_seq,
                  const int32_t* token_pos, int32_t num_tokens, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq, int64_t num_blocks, void* stream) {
  return pkv::append_impl(k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos,
                          num_tokens, num_seqs, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, num_blocks, stream, false, 1.0f, 1.0f);
}

int32_t kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* token_seq,
                      const int32_t* token_pos, int32_t num_tokens, int32_t num_seqs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, float k_scale,
                      float v_scale, void* stream) {
  return pkv::append_impl(k_new, v_new, k_cache, v_cache, block_tables, token_seq, token_pos,
                          num_tokens, num_seqs, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, num_blocks, stream, true, k_scale, v_scale);
}

int32_t copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                    int64_t num_blocks, int64_t block_bytes, const int32_t* src_dst_pairs,
                    int32_t num_pairs, void* stream) {
  if (num_pairs < 0 || num_layers < 0 || num_blocks < 0 || block_bytes < 0) return PKV_ERR_SHAPE;
  if (num_pairs == 0 || num_layers == 0) return PKV_OK;
  if (!k_caches || !v_caches || !src_dst_pairs) return PKV_ERR_NULL;
  if (num_layers > pkv::kMaxLayers) return PKV_ERR_UNSUPPORTED;
  if (block_bytes == 0 || block_bytes % 16 != 0 || num_blocks == 0) return PKV_ERR_SHAPE;
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return PKV_ERR_NULL;
    if (!pkv::aligned16(k_caches[l]) || !pkv::aligned16(v_caches[l])) return PKV_ERR_ALIGNMENT;
  }
  if (pkv::launch_copy_blocks(k_caches, v_caches, num_layers, num_blocks, block_bytes,
                              src_dst_pairs, num_pairs, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return PKV_ERR_LAUNCH;
  return PKV_OK;
}

int32_t pkv_check_batch(const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* query_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t block_size, int32_t max_query_len,
                        int32_t* result, void* stream) {
  if (num_seqs < 0 || num_seqs >= (1 << 29) || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      block_size <= 0 || max_query_len < 0)
    return PKV_ERR_SHAPE;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX) return PKV_ERR_SHAPE;
  if (!result || (num_seqs > 0 && (!block_tables || !context_lens))) return PKV_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(result) & 3u) != 0) return PKV_ERR_ALIGNMENT;
  pkv::CheckDims c;
  c.S = num_seqs;
  c.M = max_blocks_per_seq;
  c.B = block_size;
  c.Qmax = max_query_len;
  c.NB = num_blocks;
  if (pkv::launch_check(block_tables, context_lens, query_lens, result, c,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return PKV_ERR_LAUNCH;
  return PKV_OK;
}

}  // extern "C"
