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
  kErrShared = 16u,    // shared-prefix description disagrees with the tables or lengths
  kErrQuery = 32u,     // prefill query range out of order, past num_tokens or longer than seq_len
  kErrScale = 64u,     // FP8 block scale not a positive finite number
};

constexpr int kDefaultPartitionTokens = 512;
constexpr int kMaxPartitionTokens = 4096;  // bounds the LDS window of block-table entries
constexpr int kMaxBalancedSeqs = 2048;     // batch limit of the balanced schedule (LDS scan)

// Workgroups of the balanced schedule over all kv-head groups: one per CU.
constexpr int kBalancedWorkgroups = 256;

// Waves per workgroup of the matrix-core kernels: one per kv head, the
// largest of 8, 4, 2, 1 that divides num_kv_heads.
int mfma_waves_per_group(int num_kv_heads);

// Slices of the balanced schedule per kv-head group (a workgroup's waves
// cover one group of mfma_waves_per_group kv heads).
inline int balanced_slices(int num_kv_heads) {
  const int groups = num_kv_heads / mfma_waves_per_group(num_kv_heads);
  return (kBalancedWorkgroups + groups - 1) / groups;
}

// Everything one decode launch needs; passed by value as a kernel argument.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  // Partial results.  Partition grid: rows [B][Hq][max_parts].  Balanced
  // schedule: rows [slices][Hkv][2][G] (slices per kv-head group).  acc rows
  // hold D floats.
  float* ws_max;
  float* ws_sum;
  float* ws_acc;
  int* ws_desc;    // balanced schedule: per slice, (cut sequence ending there or -1, its first slice)
  unsigned* err;
  int64_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t part_tokens;
  int32_t max_parts;
  int32_t out_bf16;
  int32_t slices;      // > 0: balanced schedule with this many slices per kv head
  float scale_log2e;   // softmax scale * log2(e): scores feed exp2
  const float* k_scale;  // FP8 pools: per (block, kv head) scales, [num_blocks][num_kv_heads]
  const float* v_scale;
};

// Workspace carve-up shared by the size query and the launch.
struct WorkspaceLayout {
  size_t desc_off, max_off, sum_off, acc_off, total;
};
// Partition grid: `rows` = B * Hq * max_parts, no descriptors.  Balanced
// schedule: `rows` = slices * 2 * Hq, `desc_ints` = 2 * slices.
WorkspaceLayout workspace_layout(int64_t rows, int64_t head_dim, int64_t desc_ints);

hipError_t launch_kv_write(const void* k, const void* v, const int64_t* slots, int64_t n,
                           void* k_cache, void* v_cache, int64_t num_slots, int64_t row_bytes,
                           unsigned* err, hipStream_t stream);

// Whole-block copies from the (src_k, src_v) pools to the (dst_k, dst_v)
// pools, which may be the same pools (copy-on-write) or different ones
// (swapping); every pointer must be addressable by the device.
// Scales (FP8 pools): when src_ks is non-null, each pair also copies the
// `scales` K and V scales of its block (src_ks/src_vs -> dst_ks/dst_vs).
struct BlockScales {
  float* dst_ks = nullptr;
  float* dst_vs = nullptr;
  const float* src_ks = nullptr;
  const float* src_vs = nullptr;
  int scales = 0;
};
hipError_t launch_block_copy(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                             const int64_t* pairs, int64_t num_pairs, int64_t src_blocks,
                             int64_t dst_blocks, int64_t block_bytes, unsigned* err,
                             hipStream_t stream, const BlockScales& sc = BlockScales{});

// Chooses the kernel for (dtype, head_dim, block_size, group) and schedule
// (a.slices > 0: balanced; else the partition grid) and launches the main
// pass and, when partial results can exist, the matching reduce.  Returns
// hipErrorInvalidValue for a combination that has no kernel.  fp8: the pools
// hold E4M3 codes with the per-block scales a.k_scale / a.v_scale.
hipError_t launch_decode(const DecodeArgs& a, int bf16, int head_dim, int block_size, int group,
                         hipStream_t stream, bool fp8 = false);

// The head_dim-128 matrix-core kernels of either schedule (attention_mfma.hip),
// bf16 pools or (fp8 set) E4M3 pools with a.k_scale / a.v_scale.
hipError_t launch_mfma_decode(const DecodeArgs& a, int block_size, int group, hipStream_t stream,
                              bool fp8 = false);

// Slot-mapping write into E4M3 pools (kv_write.hip): bf16 rows in, each element
// divided by its block's scale and rounded to the nearest code.
hipError_t launch_kv_write_fp8(const void* k, const void* v, const int64_t* slots, int64_t n,
                               void* k_cache, void* v_cache, const float* k_scale,
                               const float* v_scale, int64_t num_slots, int block_size,
                               int num_kv_heads, int head_dim, unsigned* err, hipStream_t stream);

// Decode with shared prefixes (attention_shared.hip).  A prefix stream reads
// a group's shared blocks once for up to 16 * kSharedSets query columns, i.e.
// shared_members_per_stream(G) sequences of query group G.
constexpr int kSharedSets = 2;
inline int shared_members_per_stream(int group) { return 16 * kSharedSets / group; }

// Partial-result rows of the shared-prefix schedule: prefix pieces first,
// [NG + ceil(B / members) + slices][Hkv][16 * kSharedSets], then tail pieces,
// [B + slices][Hkv][G].
inline int64_t shared_prefix_rows(int num_seqs, int num_groups, int num_kv_heads, int group,
                                  int slices) {
  const int m = shared_members_per_stream(group);
  return (static_cast<int64_t>(num_groups) + (num_seqs + m - 1) / m + slices) * num_kv_heads *
         (16 * kSharedSets);
}
inline int64_t shared_tail_rows(int num_seqs, int num_q_heads, int slices) {
  return (static_cast<int64_t>(num_seqs) + slices) * num_q_heads;
}
constexpr int kSharedDescInts = 8;  // merge descriptor ints per sequence

struct SharedArgs {
  DecodeArgs d;                  // d.slices: slices per kv-head group; d.ws_desc: descriptors
  const int32_t* group_offsets;  // [num_groups + 1]: members of group g are
  const int32_t* group_seqs;     //   group_seqs[group_offsets[g] .. group_offsets[g + 1])
  const int32_t* group_lens;     // [num_groups]: tokens every member maps to the same slots
  int32_t num_groups;
  int64_t prefix_rows;           // partial rows of prefix pieces; tail rows follow
};

hipError_t launch_shared_decode(const SharedArgs& a, int block_size, int group, hipStream_t stream,
                                bool fp8 = false);

// Prefill attention (attention_prefill.hip): new tokens of sequence b are the
// query rows query_start[b] .. query_start[b + 1] - 1 of d.q and d.out.
struct PrefillArgs {
  DecodeArgs d;                 // no workspace
  const int32_t* query_start;   // [num_seqs + 1]
  int64_t num_tokens;           // rows of q and out
};

hipError_t launch_prefill(const PrefillArgs& a, int block_size, int group, hipStream_t s,
                          bool fp8 = false);

}  // namespace pkv
