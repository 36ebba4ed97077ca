// Internal declarations shared by the HIP translation units of libpagedkv.
// Kernels live next to their launchers; api.hip validates arguments and calls
// the launchers below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Bits of the per-device error word written by the kernels' range checks.
enum : unsigned {
  kErrSlot = 1u,       // slot >= num_blocks * block_size
  kErrBlockId = 2u,    // block-table entry outside [0, num_blocks)
  kErrSeqLen = 4u,     // seq_len < 0 or > max_blocks_per_seq * block_size
  kErrCopyPair = 8u,   // copy src/dst outside [0, num_blocks)
};

constexpr int kDefaultPartitionTokens = 512;

// Everything one decode launch needs; passed by value as a kernel argument.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_max;   // [B][Hq][max_parts]
  float* ws_sum;   // [B][Hq][max_parts]
  float* ws_acc;   // [B][Hq][max_parts][D]
  unsigned* err;
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t part_tokens;
  int32_t max_parts;
  int32_t out_bf16;
  float scale_log2e;   // softmax scale * log2(e): scores feed exp2
};

// Workspace carve-up shared by the size query and the launch.
struct WorkspaceLayout {
  size_t max_off, sum_off, acc_off, total;
};
WorkspaceLayout workspace_layout(int64_t num_seqs, int64_t num_q_heads, int64_t head_dim,
                                 int64_t max_parts);

hipError_t launch_kv_write(const void* k, const void* v, const int64_t* slots, int64_t n,
                           void* k_cache, void* v_cache, int64_t num_slots, int64_t row_bytes,
                           unsigned* err, hipStream_t stream);

hipError_t launch_block_copy(void* k_cache, void* v_cache, const int64_t* pairs,
                             int64_t num_pairs, int64_t num_blocks, int64_t block_bytes,
                             unsigned* err, hipStream_t stream);

// Chooses the kernel for (dtype, head_dim, block_size, group) and launches the
// main pass and, when max_parts > 1, the split-K reduce.  Returns
// hipErrorInvalidValue for a combination that has no kernel.
hipError_t launch_decode(const DecodeArgs& a, int bf16, int head_dim, int block_size,
                         int group, hipStream_t stream);

}  // namespace pkv
