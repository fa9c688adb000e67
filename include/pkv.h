/*
 * pkv.h -- C ABI of the paged KV-cache decode library (AMD MI355X, gfx950).
 *
 * The operation follows "PagedAttention (vLLM) - Virtual memory cho AI"
 * (troisinh.com) and "KV cache, PagedAttention" (aiwiki.vn):
 *   - the KV cache lives in fixed-size blocks of B tokens scattered over device
 *     memory; a per-sequence block table maps logical block j (tokens
 *     j*B .. j*B+B-1) to a physical block id (troisinh.com, section
 *     "Cơ chế Block Table"; aiwiki.vn, paragraph on paging);
 *   - decode attention: for every sequence s and query head h, the query is
 *     compared with the keys of the context_lens[s] cached positions, and the
 *     softmax weights combine the values (aiwiki.vn, paragraph on query, key
 *     and value); the kernel follows the block table to gather K/V from
 *     scattered places (troisinh.com, section "Tại sao nó hoạt động");
 *   - copy-on-write: sequences sharing a prefix share its physical blocks, and
 *     a shared block is copied before a sharer writes into it (troisinh.com,
 *     section "Copy-on-Write cho Beam Search").
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers owned by the caller, unless a
 *     comment says "host".  The library keeps no pointer after it returns and
 *     allocates no device memory (paged_attn_decode_noalloc's scratch is a static
 *     array of the library, one per GPU).
 *   - stream is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued on it and the call returns at once; buffers must stay alive until
 *     that work has finished.
 *   - Every check below is made on the host before anything is enqueued; on an
 *     error nothing is enqueued and a negative PKV_ERR_* code is returned.
 *   - bf16 means IEEE binary32 truncated to its upper 16 bits (stored as
 *     uint16); outputs are rounded to nearest, ties to even.
 *
 * KV pool layout (one K pool and one V pool per layer; B = block_size,
 * D = head_dim, Hkv = num_kv_heads, NB = num_blocks), bf16:
 *   K  [NB][Hkv][D/8][B][8] : element (block b, head g, slot o, dim d) at
 *                             (((b*Hkv + g)*(D/8) + d/8)*B + o)*8 + d%8
 *   V  [NB][Hkv][B/Bt][D][Bt], Bt = min(B, 16) : element (b, g, o, d) at
 *                             (((b*Hkv + g)*(B/Bt) + o/Bt)*D + d)*Bt + o%Bt
 *                             (B <= 16: [NB][Hkv][D][B]; B = 32: each 16-position
 *                             half of a block is its own [D][16] run)
 * Each (block, head) tile is one contiguous run of B*D*2 bytes, and a whole block
 * (all heads) is one contiguous run of Hkv*B*D*2 bytes.
 *
 * Paired form (every entry point that takes k_cache and v_cache, bf16 and fp8):
 * K and V may instead be the two halves of one pool [NB][Hkv][2][tile], whose
 * (block, head) entry holds the K tile and then the V tile, each in the layout
 * above.  Pass k_cache = the pool's start and v_cache = k_cache + one tile's bytes
 * (B*D*2 for bf16, B*D for fp8): the library recognises the form by that pointer
 * difference (two separate pools of more than one tile cannot start one tile
 * apart) and steps over both tiles per head and per block.  A tile's K and V then
 * lie in one run of twice the bytes: over fp8 pools, whose tiles are half as long,
 * the gathers of a many-sequence batch run about 5% faster (the results are the
 * same bits either way).  For copy_blocks the same two pointers per layer are
 * passed; block_bytes stays the bytes of one half's block.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1

/* Status codes. */
#define PKV_OK 0
#define PKV_ERR_NULL -1        /* a required pointer is NULL */
#define PKV_ERR_SHAPE -2       /* inconsistent sizes (e.g. num_q_heads % num_kv_heads != 0) */
#define PKV_ERR_UNSUPPORTED -3 /* head_dim, block_size or group size outside the built set,
                                  or max_blocks_per_seq*block_size above 2^26 */
#define PKV_ERR_WORKSPACE -4   /* workspace smaller than paged_attn_decode_workspace_bytes() */
#define PKV_ERR_ALIGNMENT -5   /* q, k_cache, v_cache, out or workspace not 16-byte aligned */
#define PKV_ERR_DEVICE -6      /* the HIP runtime could not report the current device */
#define PKV_ERR_LAUNCH -7      /* a kernel launch failed (hipGetLastError) */

/* Version of this ABI (PKV_ABI_VERSION of the build). */
int32_t pkv_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* pkv_status_string(int32_t status);

/*
 * Bytes of device scratch paged_attn_decode and paged_attn_decode_fp8 need for
 * these sizes on the current device (one figure covers both).  The scratch holds
 * the partial softmax states of (sequence, KV head) pairs whose context is split
 * across workers (split-K) and which worker opens each split pair.  Returns 0 for
 * sizes paged_attn_decode would reject.
 */
size_t paged_attn_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int32_t max_context_len);

/*
 * Paged decode attention (the operation described at the top of this file):
 *
 *   out[s][h][:] = sum_t p_t * V[b_t][g][o_t][:],
 *   p_t = softmax_t(scale * q[s][h][:] . K[b_t][g][o_t][:]),  t = 0 .. L-1,
 *
 * with L = context_lens[s], g = h / (num_q_heads / num_kv_heads),
 * b_t = block_tables[s][t / block_size], o_t = t % block_size.
 *
 *   q             bf16 [num_seqs][num_q_heads][head_dim]
 *   k_cache       bf16 K pool, layout above, num_blocks blocks
 *   v_cache       bf16 V pool, layout above
 *   block_tables  int32 [num_seqs][max_blocks_per_seq], row-major (a row addresses at
 *                 most 2^26 positions: max_blocks_per_seq*block_size <= 2^26); only the first
 *                 ceil(L/block_size) entries of row s are read, and each must lie
 *                 in [0, num_blocks).  Entries outside that range are clamped into
 *                 it (no memory outside the pool is read; that sequence's output
 *                 is then meaningless).
 *   context_lens  int32 [num_seqs]; 0 <= L <= max_blocks_per_seq*block_size.  L = 0
 *                 gives an all-zero output row.  Values outside the range are
 *                 clamped into it.
 *   block_size    8, 16 or 32
 *   scale         multiplier of q.k (for example 1/sqrt(head_dim))
 *   out           bf16 [num_seqs][num_q_heads][head_dim]; must not overlap an input
 *   num_q_heads   a multiple of num_kv_heads, with num_q_heads/num_kv_heads <= 16
 *   head_dim      64 or 128
 *   max_context_len  host-side upper bound of context_lens; it sizes the launch
 *                 (no device-to-host read happens).  A bound that is too small
 *                 only costs speed; it must be <= max_blocks_per_seq*block_size.
 *   workspace     device scratch of at least workspace_bytes >=
 *                 paged_attn_decode_workspace_bytes(...) bytes, 16-byte aligned;
 *                 contents need no initialisation and are overwritten.  Calls
 *                 that overlap in time must not share a workspace.
 *
 * Slots past L in a sequence's last block, table entries past ceil(L/B) and
 * blocks no table references are never read into the arithmetic.  Results are
 * deterministic: the same inputs give the same bits, and renumbering physical
 * blocks (with the tables rewritten to match) does not change a bit.
 * Enqueues two kernels: the decode kernel, then the merge of split pairs.
 */
int32_t paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t block_size, float scale, void* out, int32_t num_seqs,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                          int32_t max_blocks_per_seq, int64_t num_blocks,
                          int32_t max_context_len, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Paged decode attention over fp8 KV blocks ("KV cache, PagedAttention",
 * aiwiki.vn, paragraph on cache quantisation: keys and values stored with fewer
 * bytes).  Each pool element is one OCP E4M3FN code (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN); the key it stands
 * for is code * k_scale, the value code * v_scale.  The computation is
 * paged_attn_decode's on those keys and values.  fp8 pool layouts (B =
 * block_size, D = head_dim):
 *   K  [NB][Hkv][D/16][B][16]        : element (b, g, o, d) at
 *                                      (((b*Hkv + g)*(D/16) + d/16)*B + o)*16 + d%16
 *   V  [NB][Hkv][16][B/4][D/16][4]   : element (b, g, o, d) at
 *                                      ((((b*Hkv + g)*16 + d%16)*(B/4) + o/4)*(D/16)
 *                                       + d/16)*4 + o%4
 * A (block, head) tile is B*D contiguous bytes and a whole block Hkv*B*D bytes
 * (copy_blocks takes block_bytes = Hkv*B*D for these pools).  q and out are bf16 as
 * in paged_attn_decode.  k_scale and v_scale must be finite (else PKV_ERR_SHAPE);
 * the workspace is sized by paged_attn_decode_workspace_bytes.  All other
 * arguments, checks and guarantees are paged_attn_decode's.
 */
int32_t paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int32_t block_size, float scale, float k_scale, float v_scale,
                              void* out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int64_t num_blocks, int32_t max_context_len, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * One decode step with its KV append in one call: for every sequence s with
 * L = context_lens[s] >= 1 positions (the newest included), the newest position's
 * rows k_new[s] / v_new[s] are written into its slot (block_tables[s][(L-1)/B],
 * offset (L-1) % B) -- "PagedAttention (vLLM)" (troisinh.com), section "Cơ chế
 * Block Table": a position lives in logical block p / B at offset p % B -- and
 * attention runs over all L positions.  The pools end up as kv_append of those
 * rows leaves them, and the outputs equal paged_attn_decode's after it up to
 * rounding: when there are no more (sequence, KV head) pairs than decode workers,
 * the worker holding a pair's last tile folds the newest position in itself (its
 * weight formed on the vector units, scores summed in another order); with more
 * pairs the call enqueues the append and then the decode, and the outputs are
 * bit-identical to the two calls.  L = 0 writes nothing and gives zero rows.
 *
 *   k_new, v_new  bf16 [num_seqs][num_kv_heads][head_dim], 16-byte aligned
 *   k_cache, v_cache  written: only the newest position's slot of each sequence.
 *                 The caller's block manager has made those blocks private
 *                 (copy-on-write resolved) before the call.
 * All other arguments, checks and guarantees are paged_attn_decode's; the workspace
 * is sized by paged_attn_decode_workspace_bytes.
 */
int32_t paged_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 const int32_t* context_lens, int32_t block_size, float scale,
                                 void* out, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_append over fp8 pools: the newest rows are stored as
 * kv_append_fp8 stores them (code = E4M3(x / scale), nearest even, saturating,
 * NaN -> 0x7F) and attended to as those codes, as paged_attn_decode_fp8 does.
 * k_scale and v_scale must be finite and non-zero (else PKV_ERR_SHAPE).  The call
 * always enqueues the append and then the fp8 decode, so its outputs and pools are
 * bit-identical to kv_append_fp8 followed by paged_attn_decode_fp8.
 */
int32_t paged_attn_decode_append_fp8(const void* q, const void* k_new, const void* v_new,
                                     void* k_cache, void* v_cache, const int32_t* block_tables,
                                     const int32_t* context_lens, int32_t block_size, float scale,
                                     float k_scale, float v_scale, void* out, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t max_blocks_per_seq, int64_t num_blocks,
                                     int32_t max_context_len, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Bytes of device scratch paged_attn_multi and paged_attn_multi_fp8 need for these
 * sizes on the current device (the same role as paged_attn_decode_workspace_bytes).  Returns 0 for
 * sizes paged_attn_multi would reject.
 */
size_t paged_attn_multi_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_context_len,
                                        int32_t max_query_len);

/*
 * Multi-token paged attention with a causal mask: the attention of a prefill
 * chunk, or of the draft tokens a speculative decoding step verifies ("vLLM
 * PagedAttention: Bước đột phá về thông lượng suy luận LLM", vi.news.hada.io,
 * list of advanced features).  Sequence s holds L = context_lens[s] cached
 * positions, the last T = query_lens[s] of which are its query tokens (their K/V
 * already written, e.g. by kv_append).  Query token i sits at position
 * p = L - T + i and attends to positions 0 .. p:
 *
 *   out[s][i][h][:] = sum_{t <= p} w_t * V[b_t][g][o_t][:],
 *   w_t = softmax_{t <= p}(scale * q[s][i][h][:] . K[b_t][g][o_t][:]),
 *
 * for i < T, with g, b_t, o_t as in paged_attn_decode; rows i >= T of out are
 * zero.
 *
 *   q, out        bf16 [num_seqs][max_query_len][num_q_heads][head_dim]; rows
 *                 i >= query_lens[s] of q are not read
 *   query_lens    int32 [num_seqs]; 0 <= T <= min(L, max_query_len).  Values
 *                 outside the range are clamped into it.
 *   max_query_len 0 is a no-op
 *   workspace     at least paged_attn_multi_workspace_bytes(...) bytes
 * Every other argument is as in paged_attn_decode, with the same checks, the same
 * error codes (plus PKV_ERR_NULL for query_lens) and the same guarantees
 * (determinism, renumbering invariance).  With max_query_len = 1 and T = 1 for
 * every sequence of nonzero length the result equals paged_attn_decode's bit for
 * bit.  A wave computes a chunk of C query tokens (G = num_q_heads /
 * num_kv_heads; C = 32 / G, or 16 / G when max_context_len <= 2048, at least 1:
 * up to 32 MFMA columns of (token, head) rows).  Up to four chunks share one
 * launch, their waves reading each K/V tile together (it comes from memory once);
 * an attention kernel and a merge kernel are enqueued for each run of up to four
 * chunks, and each run reads the K/V its tokens see.
 */
int32_t paged_attn_multi(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_lens, int32_t max_query_len, int32_t block_size,
                         float scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                         int64_t num_blocks, int32_t max_context_len, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Multi-token paged attention over fp8 pools: paged_attn_multi's computation on
 * the keys code * k_scale and values code * v_scale of pools in the fp8 layouts
 * (see paged_attn_decode_fp8).  Workspace from paged_attn_multi_workspace_bytes,
 * which covers both pool formats.  k_scale and v_scale must be finite (else
 * PKV_ERR_SHAPE); everything else as paged_attn_multi.  With max_query_len = 1 and
 * one query token per non-empty sequence the result equals paged_attn_decode_fp8's
 * bit for bit.
 */
int32_t paged_attn_multi_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, const int32_t* context_lens,
                             const int32_t* query_lens, int32_t max_query_len, int32_t block_size,
                             float scale, float k_scale, float v_scale, void* out,
                             int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t max_blocks_per_seq, int64_t num_blocks,
                             int32_t max_context_len, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Paged decode attention over a batch whose sequences share a prefix physically
 * (parallel sampling and beam search keep the first blocks of a forked prompt in
 * one copy, "PagedAttention (vLLM)", troisinh.com, section "Copy-on-Write cho
 * Beam Search").  The result is paged_attn_decode's (same formula, same layouts);
 * the shared blocks are read once per group instead of once per sequence.
 *
 * Groups are runs of consecutive sequences: group v holds sequences
 * group_first[v] .. group_first[v+1] - 1.  Sequence s shares its first
 * prefix_lens[s] positions with the rest of its group: every member of a group has
 * the same prefix_lens value, at most its own context length, and block-table
 * entries 0 .. prefix_lens[s] / block_size - 1 equal to the group's first
 * member's.  A prefix length is used rounded down to a multiple of
 * max(16, block_size) and clamped to max_prefix_len; prefix length 0 (for example
 * a group of one) is a plain decode of that sequence.
 *
 *   group_first     int32 [num_groups + 1] (device): group_first[0] = 0,
 *                   non-decreasing, group_first[num_groups] = num_seqs
 *   prefix_lens     int32 [num_seqs] (device)
 *   num_groups      >= 1 when num_seqs > 0
 *   max_group_size  host-side bound of the group sizes; (num_q_heads /
 *                   num_kv_heads) * max_group_size <= 32 (else
 *                   PKV_ERR_UNSUPPORTED): the group's query rows fill at most two
 *                   16-column MFMA tiles.  Split larger groups.
 *   max_prefix_len  host-side bound of prefix_lens, <= max_context_len
 *   workspace       at least paged_attn_decode_shared_workspace_bytes(...) bytes,
 *                   16-byte aligned, no initialisation needed
 * Every other argument, check and error code is paged_attn_decode's (bf16 pools
 * only).  Data that breaks the group contract gives meaningless outputs for the
 * sequences concerned; no memory outside the arguments is touched.  Results are
 * deterministic.  Enqueues two kernels: one launch that runs, side by side on
 * about half of the compute units each, the prefix pass over the groups' shared
 * positions (rows: members x heads of a KV head) and the decode of every
 * sequence's remaining positions; then one merge, which starts each (sequence, KV
 * head) pair with a prefix from that prefix (the prefix pass's softmax state of a
 * whole (group, KV head) pair, or its partial records of the pair's rows) and
 * folds in the pair's own partial records.  Without a usable prefix (max_prefix_len
 * below max(16, block_size)) it is a plain decode: one decode kernel and its merge.
 */
size_t paged_attn_decode_shared_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_context_len,
                                                int32_t num_groups, int32_t max_group_size,
                                                int32_t max_prefix_len);

int32_t paged_attn_decode_shared(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* group_first, const int32_t* prefix_lens,
                                 int32_t num_groups, int32_t max_group_size,
                                 int32_t max_prefix_len, int32_t block_size, float scale,
                                 void* out, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int64_t num_blocks,
                                 int32_t max_context_len, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * KV append: write the key and value rows of num_tokens new tokens into their
 * slots.  Token i belongs to sequence token_seq[i] at position token_pos[i], and
 * its slot is (block_tables[seq][pos / block_size], pos % block_size): the block
 * table maps the token's logical block to a physical one ("PagedAttention
 * (vLLM)", troisinh.com, section "Cơ chế Block Table").  One decode step appends
 * one token per sequence (position = its new context length - 1); a prefill
 * chunk appends many.  The block manager must have made room first, including
 * any copy-on-write of a shared last block.
 *
 *   k_new, v_new  bf16 [num_tokens][num_kv_heads][head_dim], 16-byte aligned
 *   k_cache, v_cache  the pools (layout above), written in place
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   token_seq, token_pos  int32 [num_tokens]
 * A token whose sequence or position lies outside [0, num_seqs) x
 * [0, max_blocks_per_seq*block_size), or whose table entry lies outside
 * [0, num_blocks), is skipped on the device (nothing outside the pools is
 * written).  Two tokens must not name the same slot.  num_tokens = 0 is a no-op.
 * The written bytes equal the input bytes (bit-exact).
 */
int32_t kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                  const int32_t* block_tables, const int32_t* token_seq,
                  const int32_t* token_pos, int32_t num_tokens, int32_t num_seqs,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq, int64_t num_blocks, void* stream);

/*
 * KV append into fp8 pools (layouts under paged_attn_decode_fp8): as kv_append,
 * each element x of the new rows (bf16) is stored as the E4M3FN code nearest to
 * x / k_scale (keys) or x / v_scale (values), the division in IEEE fp32, ties to
 * the even code, magnitudes beyond 448 saturating to +-448 and NaN stored as 0x7F
 * ("KV cache, PagedAttention", aiwiki.vn, paragraph on cache quantisation).  The
 * written bytes equal that rule's codes exactly.  k_scale and v_scale must be
 * finite and nonzero (else PKV_ERR_SHAPE); block_size and head_dim as for
 * paged_attn_decode_fp8.  Other arguments, checks and skips are kv_append's.
 */
int32_t kv_append_fp8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                      const int32_t* block_tables, const int32_t* token_seq,
                      const int32_t* token_pos, int32_t num_tokens, int32_t num_seqs,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int64_t num_blocks, float k_scale,
                      float v_scale, void* stream);

/*
 * Copy-on-write block copy: for every pair i and every layer l,
 *   K_l[dst_i] := K_l[src_i]  and  V_l[dst_i] := V_l[src_i]   (whole blocks, bytes).
 *
 *   k_caches, v_caches  HOST arrays of num_layers device pointers, one pool per
 *                 layer (read during the call only; at most 128 layers)
 *   num_blocks    blocks per pool; pairs naming an id outside [0, num_blocks) are
 *                 skipped on the device (nothing outside the pools is touched)
 *   block_bytes   bytes of one block in one pool (num_kv_heads*block_size*head_dim*2
 *                 for bf16); a positive multiple of 16, pools 16-byte aligned.  A
 *                 layer whose v_caches[l] lies 1..block_bytes bytes after
 *                 k_caches[l] is taken to be in the paired form (layout notes at
 *                 the top): its blocks are runs of 2*block_bytes from k_caches[l]
 *   src_dst_pairs int32 [num_pairs][2] of (src, dst), DEVICE memory
 *   num_pairs     0 is a no-op
 * Destinations must be distinct and no destination may also be a source; then
 * the result does not depend on the order of the pairs and is bit-exact.
 */
int32_t copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                    int64_t num_blocks, int64_t block_bytes, const int32_t* src_dst_pairs,
                    int32_t num_pairs, void* stream);

/*
 * Check of the table contract the attention entry points assume (they clamp
 * block ids and lengths into range instead of checking them, so a caller that
 * breaks the contract gets meaningless rows for that sequence and no error).
 * The block-table walk is that of troisinh.com, section "Cơ chế Block Table":
 * position t of sequence s lives in the block block_tables[s][t / block_size].
 * For every sequence s, with L = context_lens[s]:
 *   kind 1: L < 0 or L > max_blocks_per_seq*block_size;
 *   kind 2: one of the first ceil(L'/block_size) entries of row s lies outside
 *           [0, num_blocks), L' being L clamped into [0, max_blocks_per_seq*block_size];
 *   kind 3: query_lens is not NULL and query_lens[s] < 0, > L' or > max_query_len.
 *
 *   block_tables, context_lens, query_lens (may be NULL): as in the attention calls
 *   max_query_len  rows per sequence of the multi-token q (ignored without query_lens)
 *   result        DEVICE int32, 4-byte aligned.  After the enqueued work finishes it
 *                 holds -1 when every sequence meets the contract, else 4*s + kind
 *                 for the smallest such s and the smallest kind it breaks.
 *   num_seqs      below 2^29 (0 writes -1)
 * Enqueues two kernels (a one-thread reset of *result, then one wave per sequence
 * with an atomic minimum); no memset, so the pair may be captured in a graph.
 * Reading *result is the caller's (it needs the stream to have finished).
 */
int32_t pkv_check_batch(const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* query_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                        int64_t num_blocks, int32_t block_size, int32_t max_query_len,
                        int32_t* result, void* stream);

/*
 * paged_attn_decode with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The split-K records and worker descriptors go to a scratch
 * array of PKV_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU: it is
 * found once per device on the first call made with that device current, and each
 * GPU holds it until the process ends.  The call itself allocates nothing and calls
 * no allocating routine.
 *
 * Arguments, checks, results and guarantees are paged_attn_decode's (the outputs are
 * bit-identical to a paged_attn_decode call with its own workspace), except:
 *   - PKV_ERR_WORKSPACE when these sizes need more scratch than
 *     PKV_NOALLOC_SCRATCH_BYTES (paged_attn_decode_workspace_bytes() above it;
 *     e.g. 16 query heads per KV head at head_dim 128 over long contexts);
 *   - PKV_ERR_DEVICE when the scratch of the current device cannot be located.
 * The scratch keeps whatever the last call left; nothing in it needs to start at
 * zero (every call rewrites what it reads).  All calls on one GPU share that GPU's
 * scratch: calls whose work overlaps in time on one GPU (two streams, or two host
 * threads) race and give meaningless results.  Calls in order on one stream are safe.
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

int32_t paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  int32_t block_size, float scale, void* out, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int64_t num_blocks,
                                  int32_t max_context_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
