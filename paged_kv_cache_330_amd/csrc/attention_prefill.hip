// Prefill attention over the paged pools: a chunk of new tokens per sequence
// (a whole prompt, or the next part of one after cached context) attends
// causally to the sequence's cached tokens.  bf16 pools with head_dim 128, on
// the matrix cores of gfx950.
//
// What is computed ("Paged KV" wiki, section "运行阶段": at prefill a sequence
// takes blocks in order and its K/V are filled in; section "Attention Kernel
// 的适配": K/V are read block by block through the block table): the new
// tokens' K/V are already in the cache (the slot-mapping write with N
// tokens), and the token at position p attends to the cached tokens 0 .. p.
// The decode step is the one-token case.
//
// Work split.  A work item is QT = 32 / G consecutive new tokens of one
// sequence (grid x: work items, grid y: kv-head groups); its QT x G queries
// fill the 32 columns of two 16-column MFMA sets (column 16 n + col: token
// (16 n + col) / G of the item, head col % G), so
// Q.K^T and P.V are dense products of each K/V tile with 32 queries.  A
// workgroup has one wave per kv head and takes one item: its waves stream the
// item's key range, tokens 0 .. (position of its last token), through the
// block table, each column masking the tokens after its own position.  Items
// are numbered sequence by sequence from the per-sequence counts (a prefix
// scan in LDS) and dispatched from the last to the first, so the longest key
// ranges of each sequence start early.
//
// Checks: a query range with query_start[b] < 0, query_start[b + 1] <
// query_start[b], query_start[b + 1] > num_tokens, or more new tokens than
// seq_lens[b] is flagged (kErrQuery) and that sequence is skipped.
#include "decode_mfma.h"

namespace pkv {
namespace {

constexpr int kCols = 16 * kSharedSets;  // query columns of a work item

template <int G, int BS>
__global__ __launch_bounds__(kMaxWaves * 64) void prefill_kernel(PrefillArgs pa) {
  static_assert(16 % G == 0, "group must divide 16");
  constexpr int QT = kCols / G;  // new tokens per work item
  const DecodeArgs& a = pa.d;
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[kMaxWaves * 16 * kKRowPad];
  __shared__ u32x4_t s_vt[kMaxWaves * 16 * kVRowPad];
  __shared__ int s_item[kMaxBalancedSeqs + 1];  // first work item of each sequence
  __shared__ int s_wsum[kMaxWaves];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
  const int kvh = blockIdx.y * (blockDim.x >> 6) + wave;
  const int B = a.num_seqs;
  const bool reporter = blockIdx.x == 0 && blockIdx.y == 0;
  const int32_t* qs = pa.query_start;

  // New tokens of sequence b, or -1 for an inconsistent range.
  auto new_tokens = [&](int b, bool report) {
    const int r0 = qs[b], r1 = qs[b + 1];
    const int L = clamped_len(a, BS, b, report);
    if (r0 < 0 || r1 < r0 || r1 > pa.num_tokens || r1 - r0 > L) {
      if (report) atomicOr(a.err, kErrQuery);
      return -1;
    }
    return r1 - r0;
  };
  const int W = block_scan(B, s_item, s_wsum, [&](int b) {
    const int n = new_tokens(b, reporter);
    return n > 0 ? (n + QT - 1) / QT : 0;
  });
  const int item = W - 1 - static_cast<int>(blockIdx.x);
  if (item < 0) return;
  const int b = last_at_most(s_item, B, item);
  const int n = new_tokens(b, false);  // > 0: b owns this item
  const int r0 = qs[b];
  const int pos0 = clamped_len(a, BS, b, false) - n;  // position of new token 0
  const int t0 = (item - s_item[b]) * QT;
  const int t1 = min(n, t0 + QT);

  // Columns: query rows and causal limits (a column past the item's last
  // token repeats it; its output is not stored).
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  bf16x8_t qop[kSharedSets][4];
  CausalTokens<kSharedSets> lim;
#pragma unroll
  for (int s = 0; s < kSharedSets; ++s) {
    const int t = min(t0 + (16 * s + col) / G, t1 - 1);
    load_qop(q + ((int64_t)(r0 + t) * a.num_q_heads + kvh * G + col % G) * kD, qr, qop[s]);
    lim.limit[s] = pos0 + t + 1;
  }
  MfmaState<kSharedSets> st;
  st.reset();
  attend_table<BS, 1, false>(a, s_bt, s_kt + wave * 16 * kKRowPad, s_vt + wave * 16 * kVRowPad,
                             a.block_tables + (int64_t)b * a.max_blocks_per_seq,
                             q + ((int64_t)r0 * a.num_q_heads + kvh * G) * kD, kvh, 0, pos0 + t1,
                             qop, st, TableCheck{nullptr, 0}, lim);

  // Normalised outputs of the item's columns.
#pragma unroll
  for (int s = 0; s < kSharedSets; ++s) {
    st.l[s] += __shfl_xor(st.l[s], 16);
    st.l[s] += __shfl_xor(st.l[s], 32);
    const int t = t0 + (16 * s + col) / G;
    if (t < t1) {
      const int64_t o = ((int64_t)(r0 + t) * a.num_q_heads + kvh * G + col % G) * kD + 4 * qr;
      const float inv = 1.f / st.l[s];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(a, o + 16 * j + i, st.o[s][j][i] * inv);
    }
  }
}

template <int G>
hipError_t launch_prefill_g(const PrefillArgs& a, int block_size, int kh, hipStream_t s) {
  constexpr int QT = kCols / G;
  // Work items: at most ceil(T / QT) + B when the query ranges are consistent.
  const int64_t items = (a.num_tokens + QT - 1) / QT + a.d.num_seqs;
  const dim3 grid(static_cast<unsigned>(items), a.d.num_kv_heads / kh);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: prefill_kernel<G, 8><<<grid, block, 0, s>>>(a); break;
    case 16: prefill_kernel<G, 16><<<grid, block, 0, s>>>(a); break;
    case 32: prefill_kernel<G, 32><<<grid, block, 0, s>>>(a); break;
    case 64: prefill_kernel<G, 64><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int block_size, int group, hipStream_t s) {
  if (a.d.num_seqs < 1 || a.d.num_seqs > kMaxBalancedSeqs || a.num_tokens < 1 ||
      a.num_tokens > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  const int kh = mfma_waves_per_group(a.d.num_kv_heads);
  switch (group) {
    case 1: return launch_prefill_g<1>(a, block_size, kh, s);
    case 2: return launch_prefill_g<2>(a, block_size, kh, s);
    case 4: return launch_prefill_g<4>(a, block_size, kh, s);
    case 8: return launch_prefill_g<8>(a, block_size, kh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
