// Whole-block copies: copy-on-write inside one pool, and transfers between
// two pools (a device pool and a pinned host pool when blocks are swapped).
//
// "PagedAttention 动态内存分页", section "写时复制与内存共享": sequences forked
// from one prompt reference the same physical blocks, and a shared block is
// copied only when one sharer has to write into it.  Section "动态块分配与回收":
// when device memory runs short, inactive blocks move to CPU memory and are
// loaded back when needed.  The host block manager decides the (src, dst)
// pairs; this kernel copies the K block and the V block of each pair, all
// block_size slots, as 16-byte vectors, and for FP8 pools the block's per-head
// scales with it.  Grid: x = pair, y = slice of the block, z = 0 for K / 1
// for V.
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void block_copy_kernel(
    uint4* dst_k, uint4* dst_v, const uint4* src_k, const uint4* src_v,
    const int64_t* __restrict__ pairs, int64_t src_blocks, int64_t dst_blocks,
    int64_t block_vecs, unsigned* err, BlockScales sc) {
  const int64_t p = blockIdx.x;
  const int64_t src = pairs[2 * p];
  const int64_t dst = pairs[2 * p + 1];
  if (static_cast<uint64_t>(src) >= static_cast<uint64_t>(src_blocks) ||
      static_cast<uint64_t>(dst) >= static_cast<uint64_t>(dst_blocks)) {
    if (threadIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) atomicOr(err, kErrCopyPair);
    return;
  }
  const uint4* s = (blockIdx.z ? src_v : src_k) + src * block_vecs;
  uint4* d = (blockIdx.z ? dst_v : dst_k) + dst * block_vecs;
  if (sc.src_ks && blockIdx.y == 0) {
    const float* ss = (blockIdx.z ? sc.src_vs : sc.src_ks) + src * sc.scales;
    float* ds = (blockIdx.z ? sc.dst_vs : sc.dst_ks) + dst * sc.scales;
    for (int i = threadIdx.x; i < sc.scales; i += blockDim.x) ds[i] = ss[i];
  }
  const int64_t stride = static_cast<int64_t>(gridDim.y) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.y) * blockDim.x + threadIdx.x; i < block_vecs;
       i += stride)
    d[i] = s[i];
}

}  // namespace

hipError_t launch_block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                             const int64_t* pairs, int64_t num_pairs, int64_t src_blocks,
                             int64_t dst_blocks, int64_t block_bytes, unsigned* err,
                             hipStream_t stream, const BlockScales& sc) {
  const int threads = 256;
  const int64_t block_vecs = block_bytes / 16;
  int64_t slices = (block_vecs + threads - 1) / threads;
  if (slices > 16) slices = 16;
  if (num_pairs > 0x7FFFFFFF) return hipErrorInvalidValue;
  block_copy_kernel<<<dim3(static_cast<unsigned>(num_pairs), static_cast<unsigned>(slices), 2),
                      dim3(threads), 0, stream>>>(
      static_cast<uint4*>(dst_k), static_cast<uint4*>(dst_v), static_cast<const uint4*>(src_k),
      static_cast<const uint4*>(src_v), pairs, src_blocks, dst_blocks, block_vecs, err, sc);
  return hipGetLastError();
}

}  // namespace pkv
