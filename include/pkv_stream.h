/*
 * pkv_stream.h -- HBM read-stream probe for the paged decode library (MI355X, gfx950).
 *
 * Decode attention is bound by memory bandwidth ("vLLM PagedAttention: Bước đột phá
 * về thông lượng suy luận LLM", vi.news.hada.io, list of features), and paging
 * leaves the bytes to move unchanged ("PagedAttention (vLLM)", troisinh.com,
 * section "Giới hạn cần hiểu").  These kernels read memory the way the decode
 * kernel does, without its arithmetic, so that its measured bandwidth can be put
 * against what the same access pattern reaches on the same GPU in the same run.
 * They compute nothing of the method; each thread folds what it read into one
 * word (so no load is dead) and writes it to `sink`.
 *
 * All pointers are DEVICE pointers; stream is a hipStream_t as void*.  Returns 0,
 * or a negative PKV_ERR_* code of pkv.h (checked on the host, nothing enqueued).
 */
#ifndef PKV_STREAM_H_
#define PKV_STREAM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sequential read of n_bytes (a positive multiple of 16, src 16-byte aligned) with
 * 16-byte lane loads, by `groups` work-groups of 256 threads taking 16 KiB chunks
 * in turn.  sink: uint32 [groups * 256].
 */
int32_t pkv_stream_read(const void* src, size_t n_bytes, uint32_t* sink, int32_t groups,
                        void* stream);

/*
 * Paired gather of fixed-size units, as the decode kernel reads K and V tiles:
 * for i in [0, n_units), unit ids[i] of k_pool and unit ids[i] of v_pool (unit u at
 * byte offset u * unit_bytes).  `waves` persistent waves (4 per work-group) take
 * equal contiguous ranges of i and keep `depth` (3 or 6) units of each pool in
 * flight.  K is read with 16-byte lane loads; V with v_load_bytes-byte loads (8 or 16).
 *   unit_bytes   1024, 2048 or 4096
 *   pool_units   units in each pool (each pool holds pool_units * unit_bytes bytes)
 *   ids          int32 [n_units]; ids outside [0, pool_units) are clamped into it
 *   sink         uint32 [waves * 64]
 */
int32_t pkv_stream_read_pairs(const void* k_pool, const void* v_pool, int64_t pool_units,
                              const int32_t* ids, int32_t n_units, int32_t unit_bytes,
                              int32_t v_load_bytes, uint32_t* sink, int32_t waves,
                              int32_t depth, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_STREAM_H_ */
