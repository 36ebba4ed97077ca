// Device helpers shared by the decode-attention kernels (attention_mfma.hip,
// attention_valu.hip).  Host code never includes this file.
#pragma once

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// 2^x on the hardware exp unit; scores are pre-multiplied by log2(e).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(m_old - m_new) with an empty side (-inf) weighted 0 even when both are -inf.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : exp2_hw(m_old - m_new);
}

// Eight bf16 values (a 16-byte load) widened exactly to fp32.
__device__ __forceinline__ void unpack_bf16x8(const u32x4_t& w, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(w[j] << 16);
    f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t i, float x) {
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[i] = f32_to_bf16_rne(x);
  else
    static_cast<float*>(a.out)[i] = x;
}

// Block-table entry bi of a row; an id outside the pool is flagged in the
// error word and replaced by block 0, so it is never dereferenced.
__device__ __forceinline__ int checked_block(const int32_t* bt, int bi, int64_t num_blocks,
                                             unsigned* err) {
  int phys = bt[bi];
  if (static_cast<uint64_t>(static_cast<int64_t>(phys)) >= static_cast<uint64_t>(num_blocks)) {
    atomicOr(err, kErrBlockId);
    phys = 0;
  }
  return phys;
}

// Length of sequence b clamped to [0, max_blocks_per_seq * block_size]; an
// out-of-range length is flagged when `report` is set.
__device__ __forceinline__ int clamped_len(const DecodeArgs& a, int block_size, int b, bool report) {
  int L = a.seq_lens[b];
  const int cap = a.max_blocks_per_seq * block_size;
  if (L < 0 || L > cap) {
    if (report) atomicOr(a.err, kErrSeqLen);
    L = L < 0 ? 0 : cap;
  }
  return L;
}

struct Partition {
  int len;                // clamped sequence length
  int begin, end, count;  // token range [begin, end) and partitions of the sequence
};

// Partition `part` of sequence b.  Returns false when it holds no token.
__device__ __forceinline__ bool setup_partition(const DecodeArgs& a, int block_size, int b,
                                                int part, bool report, Partition& p) {
  p.len = clamped_len(a, block_size, b, report && part == 0);
  p.begin = part * a.part_tokens;
  if (p.begin >= p.len) return false;
  p.end = min(p.len, p.begin + a.part_tokens);
  p.count = (p.len + a.part_tokens - 1) / a.part_tokens;
  return true;
}

}  // namespace
}  // namespace pkv
