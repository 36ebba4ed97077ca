// Slot-mapping scatter: copy each new token's K and V row into its slot.
//
// "Paged KV" wiki, section "运行阶段": at decode every new token is written into
// the next slot of its sequence's active block (prefill fills blocks in order).
// The slot numbers come from the host block manager; the kernel only moves
// bytes.  One token row is num_kv_heads * head_dim elements (2 KiB for 8 kv
// heads x 128 bf16), moved as 16-byte vectors so that a wavefront covers
// whole rows with coalesced loads and stores.
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t n,
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    int64_t num_slots, int row_vecs, int tokens_per_wg, unsigned* err) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tokens_per_wg;
  const int per_token = 2 * row_vecs;  // K vectors, then V vectors
  const int total = tokens_per_wg * per_token;
  for (int f = threadIdx.x; f < total; f += blockDim.x) {
    const int tl = f / per_token;
    const int r = f - tl * per_token;
    const int64_t t = t0 + tl;
    if (t >= n) break;
    const int64_t s = slots[t];
    if (s < 0) continue;  // padding token
    if (s >= num_slots) {
      if (r == 0) atomicOr(err, kErrSlot);
      continue;
    }
    const bool is_v = r >= row_vecs;
    const int c = is_v ? r - row_vecs : r;
    const uint4* src = (is_v ? v : k) + t * row_vecs + c;
    uint4* dst = (is_v ? v_cache : k_cache) + s * row_vecs + c;
    *dst = *src;
  }
}

}  // namespace

hipError_t launch_kv_write(const void* k, const void* v, const int64_t* slots, int64_t n,
                           void* k_cache, void* v_cache, int64_t num_slots, int64_t row_bytes,
                           unsigned* err, hipStream_t stream) {
  const int row_vecs = static_cast<int>(row_bytes / 16);
  const int threads = 256;
  int tokens_per_wg = threads / (2 * row_vecs);
  if (tokens_per_wg < 1) tokens_per_wg = 1;
  const int64_t blocks = (n + tokens_per_wg - 1) / tokens_per_wg;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  kv_write_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(
      static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots, n,
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), num_slots, row_vecs,
      tokens_per_wg, err);
  return hipGetLastError();
}

}  // namespace pkv
