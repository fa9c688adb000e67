// Reference oracle for paged decode attention -- TEST INFRASTRUCTURE ONLY.
//
// Only the test-suite, the smoke check and the CPU-baseline leg of the benchmark
// may load this code.  The product library never links or calls it, and it shares
// no source, header, helper or table with the GPU path.
//
// What it computes (plain definition, written out):
//   * "KV cache, PagedAttention" (aiwiki.vn), paragraph on query/key/value: the
//     query of the current position is compared with the keys of every position it
//     may attend to, and the resulting attention weights combine the values.
//   * "PagedAttention (vLLM)" (troisinh.com), section "Cơ chế Block Table": the
//     cache is split into fixed-size blocks; a per-sequence block table maps the
//     logical block j (tokens j*B .. j*B+B-1) to a physical block anywhere in the
//     pool; a sequence of L tokens occupies ceil(L/B) blocks.
//   * same page, section "Tại sao nó hoạt động": the kernel follows the block
//     table to fetch K/V from scattered places, then takes a softmax.
//   * same page, section "Ý tưởng cốt lõi": physical placement does not matter,
//     only the logical position does.
//
// Readings where the pages are silent (each is listed in the design notes):
//   * scale is an argument; x_t = scale * (q . k_t), summed over d in ascending
//     order, multiplied by scale after the sum;
//   * query head h reads KV head h / (Hq/Hkv) (contiguous grouping);
//   * L = 0 gives an all-zero output;
//   * softmax is the max-subtracted form: w_t = exp(x_t - max), p_t = w_t / sum w;
//   * bf16 inputs are widened exactly to the accumulator type;
//   * pool layout (one pool per layer, per K and per V):
//       K  [num_blocks][Hkv][D/8][B][8]   element (b,g,o,d) at
//          (((b*Hkv + g)*(D/8) + d/8)*B + o)*8 + d%8
//       V  [num_blocks][Hkv][B/Bt][D][Bt] with Bt = min(B, 16): element (b,g,o,d)
//          at (((b*Hkv + g)*(B/Bt) + o/Bt)*D + d)*Bt + o%Bt (each 16-position
//          half of a block is its own [D][16] run; the whole block when B <= 16)
//   * block_tables is int32 [S][M] row-major; only the first ceil(L/B) entries of
//     row s are read.  Tail slots of the last block, padding entries of a table
//     row and unreferenced blocks are never read.
//   * fp8 KV blocks ("KV cache, PagedAttention" (aiwiki.vn), paragraph on cache
//     quantisation: fewer bytes per stored key/value): each element is an OCP
//     E4M3FN code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
//     infinities; S.1111.111 is NaN) times a per-call scale (one for K, one for
//     V).  Layouts:
//       K  [num_blocks][Hkv][D/16][B][16] element (b,g,o,d) at
//          (((b*Hkv + g)*(D/16) + d/16)*B + o)*16 + d%16
//       V  [num_blocks][Hkv][16][B/4][D/16][4] element (b,g,o,d) at
//          ((((b*Hkv + g)*16 + d%16)*(B/4) + o/4)*(D/16) + d/16)*4 + o%4
//     A stored code is decoded exactly, then multiplied by its scale in the
//     accumulator type.
//
// Precision: the accumulator type is a template parameter.  The fp32
// instantiation is the oracle the GPU is compared against; the fp64 one measures
// the fp32 oracle's own rounding error.  Sums run in ascending index order.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

// bf16 is the upper half of an IEEE binary32; widening is exact.
inline float bf16_bits_to_float(uint16_t bits) {
  uint32_t w = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &w, sizeof f);
  return f;
}

inline double exp_acc(double x) { return std::exp(x); }
inline float exp_acc(float x) { return std::exp(x); }  // libm expf

struct Shape {
  int32_t S, Hq, Hkv, D, B, M;
  int64_t NB;
};

inline int64_t k_index(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) {
  return (((b * sh.Hkv + g) * (sh.D / 8) + d / 8) * sh.B + o) * 8 + d % 8;
}

inline int64_t v_index(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) {
  const int64_t bt = sh.B < 16 ? sh.B : 16;
  return (((b * sh.Hkv + g) * (sh.B / bt) + o / bt) * sh.D + d) * bt + o % bt;
}

inline int64_t k8_index(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) {
  return (((b * sh.Hkv + g) * (sh.D / 16) + d / 16) * sh.B + o) * 16 + d % 16;
}

inline int64_t v8_index(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) {
  return ((((b * sh.Hkv + g) * 16 + d % 16) * (sh.B / 4) + o / 4) * (sh.D / 16) + d / 16) * 4 + o % 4;
}

// OCP E4M3FN: normal codes are (1 + m/8) * 2^(e-7), subnormal codes (e = 0) are
// (m/8) * 2^-6, and exponent 15 with mantissa 7 is NaN.
inline float e4m3_to_float(uint8_t code) {
  const int e = (code >> 3) & 15, m = code & 7;
  float v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = std::ldexp(static_cast<float>(m), -9);
  else
    v = std::ldexp(static_cast<float>(8 + m), e - 10);
  return (code & 0x80) ? -v : v;
}

// The E4M3FN code nearest to y (ties to the even mantissa), saturating at
// +-448 (the largest finite magnitude; S.1111.111 is NaN, not a number to round
// to); NaN gives 0x7F.  Written from the format's definition: magnitudes below
// 2^-6 are multiples of 2^-9 (subnormal codes), the others (1 + m/8) * 2^e.
inline uint8_t e4m3_from_float(float y) {
  if (std::isnan(y)) return 0x7F;
  const uint8_t sign = std::signbit(y) ? 0x80 : 0x00;
  const double a = std::fabs(static_cast<double>(y));
  if (a >= 448.0) return sign | 0x7E;
  if (a < std::ldexp(1.0, -6)) {
    const int m = static_cast<int>(std::nearbyint(std::ldexp(a, 9)));  // 0 .. 8
    return sign | static_cast<uint8_t>(m);  // m = 8 is the smallest normal, code 0x08
  }
  int e = 0;
  const double f = std::frexp(a, &e);  // a = f * 2^e, f in [0.5, 1)
  int exp = e - 1;                     // a = (2f) * 2^exp, 2f in [1, 2)
  int m = static_cast<int>(std::nearbyint((2.0 * f - 1.0) * 8.0));
  if (m == 8) {
    m = 0;
    ++exp;
  }
  if (exp + 7 > 15 || (exp + 7 == 15 && m == 7)) return sign | 0x7E;
  return sign | static_cast<uint8_t>(((exp + 7) << 3) | m);
}

// Where the keys and values are read: bf16 pools, or fp8 pools with their scales.
struct Bf16Kv {
  const uint16_t* kp;
  const uint16_t* vp;
  float k(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) const {
    return bf16_bits_to_float(kp[k_index(sh, b, g, o, d)]);
  }
  float v(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) const {
    return bf16_bits_to_float(vp[v_index(sh, b, g, o, d)]);
  }
};

struct Fp8Kv {
  const uint8_t* kp;
  const uint8_t* vp;
  float k_scale, v_scale;
  float k(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) const {
    return e4m3_to_float(kp[k8_index(sh, b, g, o, d)]) * k_scale;
  }
  float v(const Shape& sh, int64_t b, int64_t g, int64_t o, int64_t d) const {
    return e4m3_to_float(vp[v8_index(sh, b, g, o, d)]) * v_scale;
  }
};

// One query row attending to positions 0 .. L-1 of sequence s through its table
// row, with KV head g.  Returns 0, or -1 when a table entry lies outside the pool.
template <typename Acc, typename Kv>
int attend(const Shape& sh, const uint16_t* qrow, const Kv& kv, const int32_t* trow, int g, int L,
           Acc scale, Acc* out_row, Acc* probs_row /* may be null; length >= L */) {
  for (int d = 0; d < sh.D; ++d) out_row[d] = Acc(0);
  if (L == 0) return 0;
  std::vector<Acc> x(L);
  std::vector<int64_t> blk(L);
  for (int t = 0; t < L; ++t) {
    const int j = t / sh.B;
    const int64_t b = trow[j];
    if (b < 0 || b >= sh.NB) return -1;
    blk[t] = b;
    const int o = t % sh.B;
    Acc dot = Acc(0);
    for (int d = 0; d < sh.D; ++d)
      dot += Acc(bf16_bits_to_float(qrow[d])) * Acc(kv.k(sh, b, g, o, d));
    x[t] = scale * dot;
  }
  Acc m = x[0];
  for (int t = 1; t < L; ++t)
    if (x[t] > m) m = x[t];
  Acc z = Acc(0);
  for (int t = 0; t < L; ++t) {
    x[t] = exp_acc(x[t] - m);
    z += x[t];
  }
  for (int t = 0; t < L; ++t) x[t] = x[t] / z;  // x now holds the weights p_t
  if (probs_row)
    for (int t = 0; t < L; ++t) probs_row[t] = x[t];
  for (int d = 0; d < sh.D; ++d) {
    Acc acc = Acc(0);
    for (int t = 0; t < L; ++t)
      acc += x[t] * Acc(kv.v(sh, blk[t], g, t % sh.B, d));
    out_row[d] = acc;
  }
  return 0;
}

// One (sequence, query head) pair of a decode step: the query attends to all
// context_lens[s] cached positions.
template <typename Acc, typename Kv>
int decode_one(const Shape& sh, const uint16_t* q, const Kv& kv, const int32_t* tables,
               const int32_t* lens, Acc scale, int s, int h, Acc* out_row, Acc* probs_row) {
  const int G = sh.Hq / sh.Hkv;
  const uint16_t* qrow = q + (static_cast<int64_t>(s) * sh.Hq + h) * sh.D;
  return attend<Acc>(sh, qrow, kv, tables + static_cast<int64_t>(s) * sh.M, h / G, lens[s],
                     scale, out_row, probs_row);
}

template <typename Acc, typename Kv>
int decode_all(const uint16_t* q, const Kv& kv, const int32_t* tables, const int32_t* lens,
               int32_t B, double scale, Acc* out, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
               int32_t M, int64_t NB, int32_t threads) {
  if (!q || !kv.kp || !kv.vp || !tables || !lens || !out) return -2;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || M < 0 || NB < 0) return -3;
  if (Hq % Hkv != 0 || D % 8 != 0) return -3;
  for (int s = 0; s < S; ++s)
    if (lens[s] < 0 || static_cast<int64_t>(lens[s]) > static_cast<int64_t>(M) * B) return -4;
  const Shape sh{S, Hq, Hkv, D, B, M, NB};
  const int64_t pairs = static_cast<int64_t>(S) * Hq;
  int status = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
  for (int64_t i = 0; i < pairs; ++i) {
    const int s = static_cast<int>(i / Hq), h = static_cast<int>(i % Hq);
    const int rc = decode_one<Acc>(sh, q, kv, tables, lens, static_cast<Acc>(scale), s, h,
                                   out + i * D, nullptr);
    if (rc < status) status = rc;
  }
  return status;
}

// Several query tokens per sequence over either pool format (see the extern
// functions below for the contract).
template <typename Kv>
int multi_all(const uint16_t* q, const Kv& kv, const int32_t* block_tables,
              const int32_t* context_lens, const int32_t* query_lens, int32_t max_query_len,
              int32_t block_size, float scale, float* out, int32_t num_seqs, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
              int64_t num_blocks, int32_t threads) {
  if (!q || !kv.kp || !kv.vp || !block_tables || !context_lens || !query_lens || !out) return -2;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim % 8 != 0 ||
      num_q_heads % num_kv_heads != 0 || max_query_len < 0 || block_size <= 0)
    return -3;
  for (int s = 0; s < num_seqs; ++s) {
    const int L = context_lens[s], T = query_lens[s];
    if (L < 0 || static_cast<int64_t>(L) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
      return -4;
    if (T < 0 || T > L || T > max_query_len) return -5;
  }
  const Shape sh{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 num_blocks};
  const int G = num_q_heads / num_kv_heads;
  const int64_t rows = static_cast<int64_t>(num_seqs) * max_query_len * num_q_heads;
  int status = 0;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#pragma omp parallel for schedule(dynamic, 1) reduction(min : status)
#endif
  for (int64_t r = 0; r < rows; ++r) {
    const int s = static_cast<int>(r / (static_cast<int64_t>(max_query_len) * num_q_heads));
    const int i = static_cast<int>((r / num_q_heads) % max_query_len);
    const int h = static_cast<int>(r % num_q_heads);
    float* orow = out + r * head_dim;
    if (i >= query_lens[s]) {
      for (int d = 0; d < head_dim; ++d) orow[d] = 0.f;
      continue;
    }
    const int p = context_lens[s] - query_lens[s] + i;
    const int rc = attend<float>(sh, q + r * head_dim, kv,
                                 block_tables + static_cast<int64_t>(s) * max_blocks_per_seq,
                                 h / G, p + 1, scale, orow, nullptr);
    if (rc < status) status = rc;
  }
  return status;
}

}  // namespace

extern "C" {

// fp32 oracle.  q, k_pool, v_pool hold raw bf16 bit patterns.  out is float [S][Hq][D].
// Returns 0, -1 (a table entry outside [0, num_blocks)), -2 (null pointer),
// -3 (bad shape), -4 (a context length outside [0, M*B]).  threads <= 0 keeps the
// OpenMP default.
int oracle_paged_decode_f32(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, float scale, float* out, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int64_t num_blocks, int32_t threads) {
  return decode_all<float>(q, Bf16Kv{k_pool, v_pool}, block_tables, context_lens, block_size,
                           scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           max_blocks_per_seq, num_blocks, threads);
}

// The same computation with a double accumulator and double output.
int oracle_paged_decode_f64(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t block_size, double scale, double* out, int32_t num_seqs,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_blocks_per_seq, int64_t num_blocks, int32_t threads) {
  return decode_all<double>(q, Bf16Kv{k_pool, v_pool}, block_tables, context_lens, block_size,
                            scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_blocks_per_seq, num_blocks, threads);
}

// Decode over fp8 pools (layouts and decoding in the header comment): keys are
// code(K) * k_scale, values code(V) * v_scale; everything else as
// oracle_paged_decode_f32.  Also needs head_dim % 16 == 0 and block_size % 4 == 0.
int oracle_paged_decode_fp8_f32(const uint16_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t block_size, float scale, float k_scale, float v_scale,
                                float* out, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                int64_t num_blocks, int32_t threads) {
  if (head_dim % 16 != 0 || block_size % 4 != 0) return -3;
  return decode_all<float>(q, Fp8Kv{k_pool, v_pool, k_scale, v_scale}, block_tables, context_lens,
                           block_size, scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                           max_blocks_per_seq, num_blocks, threads);
}

// The E4M3FN decoding itself, for n codes.
void oracle_fp8_e4m3_to_f32(const uint8_t* codes, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_float(codes[i]);
}

// The E4M3FN encoding itself (nearest, ties to even, saturating), for n floats.
void oracle_fp8_e4m3_from_f32(const float* in, uint8_t* codes, int64_t n) {
  for (int64_t i = 0; i < n; ++i) codes[i] = e4m3_from_float(in[i]);
}

// KV append into fp8 pools: as oracle_kv_append, each element x (bf16) stored as
// the code of x / k_scale (keys) or x / v_scale (values), the division in fp32.
int oracle_kv_append_fp8(const uint16_t* k_new, const uint16_t* v_new, uint8_t* k_pool,
                         uint8_t* v_pool, const int32_t* block_tables, const int32_t* seq,
                         const int32_t* pos, int32_t num_tokens, int32_t num_seqs,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, int64_t num_blocks, float k_scale,
                         float v_scale) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim % 16 != 0 || block_size % 4 != 0 ||
      block_size <= 0)
    return -3;
  if (num_tokens == 0) return 0;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq || !pos) return -2;
  const Shape sh{num_seqs, num_kv_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 num_blocks};
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t s = seq[i], p = pos[i];
    if (s < 0 || s >= num_seqs || p < 0 ||
        static_cast<int64_t>(p) >= static_cast<int64_t>(max_blocks_per_seq) * block_size)
      continue;
    const int64_t b = block_tables[static_cast<int64_t>(s) * max_blocks_per_seq + p / block_size];
    if (b < 0 || b >= num_blocks) continue;
    const int o = p % block_size;
    for (int g = 0; g < num_kv_heads; ++g)
      for (int d = 0; d < head_dim; ++d) {
        const int64_t src = (static_cast<int64_t>(i) * num_kv_heads + g) * head_dim + d;
        k_pool[k8_index(sh, b, g, o, d)] = e4m3_from_float(bf16_bits_to_float(k_new[src]) / k_scale);
        v_pool[v8_index(sh, b, g, o, d)] = e4m3_from_float(bf16_bits_to_float(v_new[src]) / v_scale);
      }
  }
  return 0;
}

// Several query tokens per sequence (speculative verification, chunked prefill):
// sequence s holds context_lens[s] positions, the last query_lens[s] of which are
// its query tokens; query token i sits at position p = L - query_lens[s] + i and
// attends to positions 0 .. p (causal).  q and out are [S][max_query_len][Hq][D];
// rows i >= query_lens[s] of out are zero.  Returns 0 or a negative code (as
// oracle_paged_decode_f32, plus -5 for query lengths outside [0, min(L, qmax)]).
int oracle_paged_attn_multi_f32(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_lens, int32_t max_query_len,
                                int32_t block_size, float scale, float* out, int32_t num_seqs,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, int64_t num_blocks, int32_t threads) {
  return multi_all(q, Bf16Kv{k_pool, v_pool}, block_tables, context_lens, query_lens,
                   max_query_len, block_size, scale, out, num_seqs, num_q_heads, num_kv_heads,
                   head_dim, max_blocks_per_seq, num_blocks, threads);
}

// The same over fp8 pools (keys code * k_scale, values code * v_scale).
int oracle_paged_attn_multi_fp8_f32(const uint16_t* q, const uint8_t* k_pool,
                                    const uint8_t* v_pool, const int32_t* block_tables,
                                    const int32_t* context_lens, const int32_t* query_lens,
                                    int32_t max_query_len, int32_t block_size, float scale,
                                    float k_scale, float v_scale, float* out, int32_t num_seqs,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t max_blocks_per_seq, int64_t num_blocks,
                                    int32_t threads) {
  if (head_dim % 16 != 0 || block_size % 4 != 0) return -3;
  return multi_all(q, Fp8Kv{k_pool, v_pool, k_scale, v_scale}, block_tables, context_lens,
                   query_lens, max_query_len, block_size, scale, out, num_seqs, num_q_heads,
                   num_kv_heads, head_dim, max_blocks_per_seq, num_blocks, threads);
}

// Debug form for one (sequence, query head): writes the D outputs and the L
// softmax weights p_t (fp32).  probs must hold context_lens[seq] floats.
int oracle_paged_decode_probs_f32(const uint16_t* q, const uint16_t* k_pool,
                                  const uint16_t* v_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, int32_t block_size, float scale,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int64_t num_blocks, int32_t seq, int32_t head, float* out_row,
                                  float* probs) {
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out_row || !probs) return -2;
  if (seq < 0 || seq >= num_seqs || head < 0 || head >= num_q_heads) return -3;
  if (num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim % 8 != 0) return -3;
  const Shape sh{num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 num_blocks};
  return decode_one<float>(sh, q, Bf16Kv{k_pool, v_pool}, block_tables, context_lens, scale, seq,
                           head, out_row, probs);
}

// KV append ("Cơ chế Block Table", troisinh.com): token i of sequence seq[i] at
// position pos[i] lives in logical block pos/B at offset pos%B; the block table
// names the physical block.  Its K and V rows (bf16 [Hkv][D]) are copied there.
// Tokens whose sequence, position or block id is out of range are skipped.
// Returns 0, -2 (null), -3 (bad sizes).
int oracle_kv_append(const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_pool,
                     uint16_t* v_pool, const int32_t* block_tables, const int32_t* seq,
                     const int32_t* pos, int32_t num_tokens, int32_t num_seqs,
                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                     int32_t max_blocks_per_seq, int64_t num_blocks) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim % 8 != 0 || block_size <= 0) return -3;
  if (num_tokens == 0) return 0;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq || !pos) return -2;
  const Shape sh{num_seqs, num_kv_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                 num_blocks};
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int32_t s = seq[i], p = pos[i];
    if (s < 0 || s >= num_seqs || p < 0 ||
        static_cast<int64_t>(p) >= static_cast<int64_t>(max_blocks_per_seq) * block_size)
      continue;
    const int64_t b = block_tables[static_cast<int64_t>(s) * max_blocks_per_seq + p / block_size];
    if (b < 0 || b >= num_blocks) continue;
    const int o = p % block_size;
    for (int g = 0; g < num_kv_heads; ++g)
      for (int d = 0; d < head_dim; ++d) {
        const int64_t src = (static_cast<int64_t>(i) * num_kv_heads + g) * head_dim + d;
        k_pool[k_index(sh, b, g, o, d)] = k_new[src];
        v_pool[v_index(sh, b, g, o, d)] = v_new[src];
      }
  }
  return 0;
}

// Copy-on-write block copy ("Copy-on-Write cho Beam Search", troisinh.com): for
// every (src, dst) pair and every layer, the bytes of block dst become the bytes
// of block src, in K and in V; nothing else changes.  Pools are given as arrays of
// host pointers, one per layer.  Returns 0, -2 (null), -3 (bad sizes), -1 (a block
// id outside the pool).
int oracle_copy_blocks(uint8_t* const* k_pools, uint8_t* const* v_pools, int32_t num_layers,
                       int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                       int32_t num_pairs) {
  if (num_pairs < 0 || num_layers < 0 || block_bytes < 0) return -3;
  if (num_pairs == 0 || num_layers == 0) return 0;
  if (!k_pools || !v_pools || !pairs) return -2;
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return -1;
  }
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_pools[l] || !v_pools[l]) return -2;
    for (int32_t i = 0; i < num_pairs; ++i) {
      const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
      std::memmove(k_pools[l] + dst * block_bytes, k_pools[l] + src * block_bytes, block_bytes);
      std::memmove(v_pools[l] + dst * block_bytes, v_pools[l] + src * block_bytes, block_bytes);
    }
  }
  return 0;
}

}  // extern "C"
