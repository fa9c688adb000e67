// Copy-on-write block copy ("PagedAttention (vLLM)", troisinh.com, section
// "Copy-on-Write cho Beam Search"): before a sequence writes into a block it
// shares with others, the block's bytes move to a private block.  One block is
// one contiguous run of bytes in every pool, so the copy is a plain 16-byte-per-
// lane stream: each work-group moves 4 KiB of one (pair, pool).  A layer whose K
// and V are the two halves of one pool (each (block, head) entry a K tile and then
// a V tile) has one run of twice the bytes per block, copied from the K side.

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int64_t kCopyBytesPerGroup = kCopyThreads * 16;

struct PoolPtrs {
  uint8_t* p[2 * kMaxLayers];    // K pools of layers 0..L-1, then V pools
  uint8_t span[2 * kMaxLayers];  // block runs of block_bytes each: 1, 2 (paired), 0 (skip)
};

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(PoolPtrs pools,
                                                                   const int32_t* pairs,
                                                                   int64_t num_blocks,
                                                                   int64_t block_bytes,
                                                                   int32_t groups_per_block) {
  const int32_t pair = blockIdx.x / groups_per_block;
  const int32_t part = blockIdx.x % groups_per_block;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* pool = pools.p[blockIdx.y];
  const int64_t run = block_bytes * pools.span[blockIdx.y];
  const int64_t off = part * kCopyBytesPerGroup + static_cast<int64_t>(threadIdx.x) * 16;
  if (off >= run) return;
  const u32x4_t x = *reinterpret_cast<const u32x4_t*>(pool + src * run + off);
  *reinterpret_cast<u32x4_t*>(pool + dst * run + off) = x;
}

}  // namespace

hipError_t launch_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers,
                              int64_t num_blocks, int64_t block_bytes, const int32_t* pairs,
                              int32_t num_pairs, hipStream_t stream) {
  PoolPtrs pools = {};
  int64_t longest = block_bytes;
  for (int32_t l = 0; l < num_layers; ++l) {
    pools.p[l] = static_cast<uint8_t*>(k_caches[l]);
    pools.p[num_layers + l] = static_cast<uint8_t*>(v_caches[l]);
    // paired: V starts one tile after K, at most one block in; separate pools of
    // more than one block cannot (they would overlap), and for a one-block pool
    // both readings copy block 0 onto itself
    const uintptr_t k = reinterpret_cast<uintptr_t>(k_caches[l]);
    const uintptr_t v = reinterpret_cast<uintptr_t>(v_caches[l]);
    const bool paired = v > k && v - k <= static_cast<uintptr_t>(block_bytes);
    pools.span[l] = paired ? 2 : 1;
    pools.span[num_layers + l] = paired ? 0 : 1;
    if (paired) longest = 2 * block_bytes;
  }
  const int64_t gpb = (longest + kCopyBytesPerGroup - 1) / kCopyBytesPerGroup;
  const int64_t gx = gpb * num_pairs;
  if (gx > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(static_cast<uint32_t>(gx), 2 * num_layers),
                     dim3(kCopyThreads), 0, stream, pools, pairs, num_blocks, block_bytes,
                     static_cast<int32_t>(gpb));
  return hipGetLastError();
}

}  // namespace pkv
