// Slot-mapping scatter: copy each new token's K and V row into its slot
// (bf16/fp32 pools), or encode it into its slot (E4M3 pools with per-block
// scales).
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

// Nearest E4M3 code (OCP: bias 7, no infinities, largest finite 448) of a
// binary32 value: round to nearest, ties to even, magnitudes beyond 448
// saturate to 448, NaN gives S.1111.111.  Normal results round the binary32
// word at its 20th bit (the carry moves into the exponent by itself); results
// below 2^-6 are multiples of 2^-9, rounded by rintf (ties to even).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a > 0x7F800000u) {
    code = 0x7Fu;                                   // NaN
  } else if (a >= 0x43E00000u) {
    code = 0x7Eu;                                   // >= 448
  } else if (a < 0x3C800000u) {
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.f));  // < 2^-6
  } else {
    uint32_t q = a >> 20;
    const uint32_t rem = a & 0xFFFFFu;
    q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
    code = q - (120u << 3);                         // rebias the exponent 127 -> 7
  }
  return code | sign;
}

// Each thread encodes 16 elements of one token row (K or V): 32 bytes of
// bf16 in, 16 bytes of E4M3 codes out.  The scale is that of the slot's
// block and the elements' kv head.
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, const int64_t* __restrict__ slots,
    int64_t n, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale, int64_t num_slots,
    int block_size, int num_kv_heads, int head_dim, int row_vecs, int tokens_per_wg,
    unsigned* err) {
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tokens_per_wg;
  const int per_token = 2 * row_vecs;  // K vectors, then V vectors (16 elements each)
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
    const int64_t blk = s / block_size;
    const float sc = (is_v ? v_scale : k_scale)[blk * num_kv_heads + (c * 16) / head_dim];
    if (!(sc > 0.f) || !(sc <= 3.402823466e38f)) {
      atomicOr(err, kErrScale);
      continue;
    }
    const uint4* src = (is_v ? v : k) + (t * row_vecs + c) * 2;
    uint32_t words[8];
    const uint4 w0 = src[0], w1 = src[1];
    words[0] = w0.x; words[1] = w0.y; words[2] = w0.z; words[3] = w0.w;
    words[4] = w1.x; words[5] = w1.y; words[6] = w1.z; words[7] = w1.w;
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t e0 = e4m3_code(__fdiv_rn(__uint_as_float(words[2 * j] << 16), sc));
      const uint32_t e1 = e4m3_code(__fdiv_rn(__uint_as_float(words[2 * j] & 0xFFFF0000u), sc));
      const uint32_t e2 = e4m3_code(__fdiv_rn(__uint_as_float(words[2 * j + 1] << 16), sc));
      const uint32_t e3 =
          e4m3_code(__fdiv_rn(__uint_as_float(words[2 * j + 1] & 0xFFFF0000u), sc));
      out[j] = e0 | (e1 << 8) | (e2 << 16) | (e3 << 24);
    }
    (is_v ? v_cache : k_cache)[s * row_vecs + c] = make_uint4(out[0], out[1], out[2], out[3]);
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

hipError_t launch_kv_write_fp8(const void* k, const void* v, const int64_t* slots, int64_t n,
                               void* k_cache, void* v_cache, const float* k_scale,
                               const float* v_scale, int64_t num_slots, int block_size,
                               int num_kv_heads, int head_dim, unsigned* err, hipStream_t stream) {
  const int row_vecs = num_kv_heads * head_dim / 16;  // 16-byte vectors of E4M3 codes per row
  const int threads = 256;
  int tokens_per_wg = threads / (2 * row_vecs);
  if (tokens_per_wg < 1) tokens_per_wg = 1;
  const int64_t blocks = (n + tokens_per_wg - 1) / tokens_per_wg;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  kv_write_fp8_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(
      static_cast<const uint4*>(k), static_cast<const uint4*>(v), slots, n,
      static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), k_scale, v_scale, num_slots,
      block_size, num_kv_heads, head_dim, row_vecs, tokens_per_wg, err);
  return hipGetLastError();
}

}  // namespace pkv
