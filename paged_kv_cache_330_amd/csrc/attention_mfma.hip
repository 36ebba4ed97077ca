// Decode-step attention over independent sequences, bf16 pools with head_dim
// 128, on the matrix cores of gfx950 (MI355X).  The per-wave work (Q.K^T,
// online softmax, P.V, the load pipeline) is in decode_mfma.h.
//
// Two schedules:
//  * decode_mfma_kernel, partition grid: workgroup (kv-head group, sequence,
//    partition of part_tokens tokens), highest partition dispatched first;
//    splitk_reduce_kernel merges the partitions of a sequence.
//  * decode_balanced_kernel: the sequences' 16-token chunks are laid end to
//    end and every workgroup takes a slice of that stream (equal, up to the
//    XCD-parity share; see the kernel), so the work per workgroup does not
//    depend on the length mix;
//    balanced_reduce_kernel merges the sequences that slices cut.
#include "decode_mfma.h"

namespace pkv {
namespace {

// ----------------------------------------------------------------------------
// Partition grid: workgroup (kv-head group, sequence, partition), partitions
// dispatched from the last to the first so that the full partitions of long
// sequences start early and the short tails of short ones fill the end.
// ----------------------------------------------------------------------------
template <int G, int BS, bool F8>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(16 % G == 0, "group must divide 16");
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[kMaxWaves * 16 * kKRowPad];
  __shared__ u32x4_t s_vt[kPvOnMfma<G> ? kMaxWaves * 16 * kVRowPad : 1];
  const int kh = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvh = blockIdx.x * kh + wave;
  const int b = blockIdx.y;
  const int part = gridDim.z - 1 - blockIdx.z;
  Partition pt;
  if (!setup_partition(a, BS, b, part, blockIdx.x == 0 && threadIdx.x == 0, pt)) {
    if (pt.len == 0 && part == 0) zero_rows<G>(a, b, kvh);
    return;
  }
  const int lane = threadIdx.x & 63;
  QueryOperand<F8> qop[1];
  load_query<G>(a, b, kvh, lane & 15, lane >> 4, qop);
  WaveState<G> st;
  st.reset();
  attend_range<G, BS, F8>(a, s_bt, s_kt + wave * 16 * kKRowPad,
                          s_vt + (kPvOnMfma<G> ? wave * 16 * kVRowPad : 0), b, kvh, pt.begin,
                          pt.end, qop, st);
  Sink sink{nullptr, nullptr, nullptr, 0, 0};
  if (pt.count > 1) {
    sink = Sink{a.ws_acc, a.ws_max, a.ws_sum,
                ((int64_t)b * a.num_q_heads + kvh * G) * a.max_parts + part, a.max_parts};
  }
  finish_wave<G>(a, st, b, kvh, sink);
}

// ----------------------------------------------------------------------------
// Balanced schedule (up to kMaxBalancedSeqs sequences).
//
// Every sequence is cut into 16-token chunks and the chunks of all sequences
// are laid end to end (sequence 0's, then sequence 1's, ...), each
// sequence's chunks preceded by kStartSeq units that stand for the start of
// its first piece.  For each kv-head group, gridDim.y workgroups take
// consecutive slices of that weighted stream of equal size (up to the
// XCD-parity share of SliceSplit), so every workgroup streams about the same
// number of K/V bytes whatever the length mix; a slice may cover the end of
// one sequence, several whole sequences and the start of another, or only a
// sequence's start-up units.  Each workgroup computes the prefix sums of the
// weighted counts in LDS.  A sequence that lies inside one slice is
// written to `out` directly; a sequence cut by slice boundaries leaves one
// partial (max, sum, unnormalised output) per piece and balanced_reduce_kernel
// merges them.  Partial slot of a piece in slice s: 1 if the piece starts its
// sequence (it then ends the slice), else 0 (it then starts the slice), so
// each slot of a slice holds at most one piece.  Partial rows:
// [slice][Hkv][slot][G].  A slice holds the final piece of at most one cut
// sequence (its first piece); its merge descriptor ws_desc[slice] names that
// sequence and the slice of its first piece, or -1.
// ----------------------------------------------------------------------------
// Start of a sequence's first piece in the balanced split, in chunks: per-piece
// timestamps fit about 2.4 us per piece against 2.34 us per chunk streamed
// (bf16 pools), 3.2-4.6 us against 1.2 us (FP8 pools).
template <bool F8>
constexpr int kStartSeq = F8 ? 4 : 1;

template <int G, int BS, bool F8>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_balanced_kernel(DecodeArgs a) {
  static_assert(16 % G == 0, "group must divide 16");
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[kMaxWaves * 16 * kKRowPad];
  __shared__ u32x4_t s_vt[kPvOnMfma<G> ? kMaxWaves * 16 * kVRowPad : 1];
  __shared__ int s_cc[kMaxBalancedSeqs + 1];
  __shared__ int s_len[kMaxBalancedSeqs];  // clamped sequence lengths
  __shared__ int s_wsum[kMaxWaves];
  __shared__ int s_prog[kMaxWaves];  // tiles streamed by each wave (issue balancing)

  const int nt = blockDim.x, nw = nt >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.x * nw + wave;
  const int slice = blockIdx.y, S = gridDim.y;
  const int B = a.num_seqs;
  const bool reporter = blockIdx.x == 0 && slice == 0;
  if (threadIdx.x < kMaxWaves) s_prog[threadIdx.x] = 0;  // visible after the scan's barriers
  // Merge descriptor of this slice: no split sequence ends here (yet).
  int* desc = a.ws_desc + 2 * slice;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    desc[0] = -1;
    desc[1] = 0;
  }

  // Exclusive prefix sums of the weighted chunk counts: a sequence with
  // chunks counts them plus kStartSeq units for the start of its first piece
  // (table window, queries, first tile), so that a slice that starts many
  // sequences gets fewer chunks; s_cc[b] = units before b.
  int carry = 0;
  for (int base = 0; base < B; base += nt) {
    const int j = base + threadIdx.x;
    const int len = j < B ? clamped_len(a, BS, j, reporter) : 0;
    if (j < B) s_len[j] = len;
    const int cnt = len > 0 ? ((len + 15) >> 4) + kStartSeq<F8> : 0;
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wsum[wave] = x;
    __syncthreads();
    int before = carry, total = 0;
    for (int w = 0; w < nw; ++w) {
      if (w < wave) before += s_wsum[w];
      total += s_wsum[w];
    }
    if (j < B) s_cc[j] = before + x - cnt;
    carry += total;
    __syncthreads();  // s_wsum is rewritten by the next round
  }
  if (threadIdx.x == 0) s_cc[B] = carry;
  __syncthreads();
  const int total = s_cc[B];
  const SliceSplit split = SliceSplit::make<F8>(total, S, gridDim.x);

  if (slice == 0)  // sequences of length 0 get zero rows
    zero_rows_where<G>(a, B, kvh, [&](int j) { return s_cc[j + 1] == s_cc[j]; });

  const int x_lo = min(total, split.begin(slice));
  const int x_hi = min(total, split.end(slice));
  if (x_lo >= x_hi) return;
  // first sequence of the slice: the largest b < B with s_cc[b] <= x_lo
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_cc[mid] <= x_lo) lo = mid; else hi = mid;
  }
  int b = lo;
  int x = x_lo;
  while (x < x_hi) {
    while (s_cc[b + 1] <= x) ++b;  // skip sequences with no chunks
    const int w0 = s_cc[b] + kStartSeq<F8>;     // unit of b's chunk 0
    const int n = s_cc[b + 1] - w0;             // b's chunks
    const int c0 = max(0, x - w0), c1 = min(n, x_hi - w0);  // this piece's chunks
    x = min(x_hi, s_cc[b + 1]);
    if (c1 <= c0) continue;  // only b's start-up units fall in this slice
    const int L = s_len[b];  // written before the scan's barriers
    const int tok_begin = c0 * 16;
    const int tok_end = min(c1 * 16, L);
    const bool first = c0 == 0, last = c1 == n;

    QueryOperand<F8> qop[1];
    load_query<G>(a, b, kvh, lane & 15, lane >> 4, qop);
    WaveState<G> st;
    st.reset();
    attend_range<G, BS, F8>(a, s_bt, s_kt + wave * 16 * kKRowPad,
                            s_vt + (kPvOnMfma<G> ? wave * 16 * kVRowPad : 0), b, kvh, tok_begin,
                            tok_end, qop, st, nw == 8 ? s_prog : nullptr);
    Sink sink{nullptr, nullptr, nullptr, 0, 0};
    if (!(first && last))
      sink = Sink{a.ws_acc, a.ws_max, a.ws_sum,
                  ((int64_t)(slice * a.num_kv_heads + kvh) * 2 + (first ? 1 : 0)) * G, 1};
    finish_wave<G>(a, st, b, kvh, sink);
    if (last && !first && blockIdx.x == 0 && threadIdx.x == 0) {
      // the final piece of a cut sequence: the reduce of this slice merges it
      desc[0] = b;
      desc[1] = split.slice_of(w0);  // slice of its first piece
    }
  }
}

// Merges the pieces of the sequence whose final piece lies in slice
// blockIdx.x (if any; with fewer sequences than slices, in the blockIdx.x-th
// slice that names one): workgroup (slice, kv-head group, query head g of the
// group), wave w for kv head kvg * KH + w, lane for output dims 2 lane and
// 2 lane + 1.  The pieces are merged with a running maximum,
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p (the loop is
// unrolled, so the loads of several pieces are in flight together).  One
// workgroup per query head keeps a long sequence's merge (one piece per
// slice it spans, e.g. 32 pieces for 32768 tokens over 256 slices) from
// resting on a single workgroup per kv-head group.
template <int G>
__global__ __launch_bounds__(kMaxWaves * 64) void balanced_reduce_kernel(DecodeArgs a) {
  int slice = blockIdx.x;
  if (gridDim.x < a.slices) {
    // Fewer workgroups than slices (there are fewer sequences than slices,
    // and each cut sequence names one slice): workgroup r takes the r-th
    // slice whose descriptor names a sequence, found by a ballot scan of all
    // descriptors, so that no workgroup is launched idle for the rest.
    __shared__ int s_cnt[kMaxWaves];
    __shared__ int s_pick;
    const int nw = blockDim.x >> 6, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (threadIdx.x == 0) s_pick = -1;
    int before = 0;
    for (int base = 0; base < a.slices; base += blockDim.x) {
      const int t = base + threadIdx.x;
      const bool named = t < a.slices && a.ws_desc[2 * t] >= 0;
      const unsigned long long m = __ballot(named);
      if (lane == 0) s_cnt[w] = __popcll(m);
      __syncthreads();
      int rank = before + __popcll(m & ((1ull << lane) - 1));
      int total = 0;
      for (int k = 0; k < nw; ++k) {
        if (k < w) rank += s_cnt[k];
        total += s_cnt[k];
      }
      if (named && rank == static_cast<int>(blockIdx.x)) s_pick = t;
      before += total;
      __syncthreads();  // s_cnt is rewritten by the next round; s_pick is final after the last
    }
    slice = s_pick;
    if (slice < 0) return;
  }
  const int b = a.ws_desc[2 * slice];
  if (b < 0) return;
  const int s0 = a.ws_desc[2 * slice + 1], s1 = slice;
  const int kvh = blockIdx.y * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int g = blockIdx.z;
  const int d = 2 * (threadIdx.x & 63);
  const float* __restrict__ wmax = a.ws_max;
  const float* __restrict__ wsum = a.ws_sum;
  const float* __restrict__ wacc = a.ws_acc;
  float M = -INFINITY, den = 0.f, num0 = 0.f, num1 = 0.f;
#pragma unroll 8
  for (int s = s0; s <= s1; ++s) {
    const int64_t r = ((int64_t)(s * a.num_kv_heads + kvh) * 2 + (s == s0 ? 1 : 0)) * G + g;
    const float m = wmax[r], l = wsum[r];
    const float2 acc = *reinterpret_cast<const float2*>(wacc + r * kD + d);
    const float Mn = fmaxf(M, m);
    const float c_old = rescale(M, Mn), c_new = exp2_hw(m - Mn);
    den = den * c_old + l * c_new;
    num0 = num0 * c_old + acc.x * c_new;
    num1 = num1 * c_old + acc.y * c_new;
    M = Mn;
  }
  const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G + g) * kD + d;
  store_out(a, o, num0 / den);
  store_out(a, o + 1, num1 / den);
}

template <int G, bool F8>
hipError_t launch_partitions_g(const DecodeArgs& a, int block_size, int kh, hipStream_t s) {
  const dim3 grid(a.num_kv_heads / kh, a.num_seqs, a.max_parts);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: decode_mfma_kernel<G, 8, F8><<<grid, block, 0, s>>>(a); break;
    case 16: decode_mfma_kernel<G, 16, F8><<<grid, block, 0, s>>>(a); break;
    case 32: decode_mfma_kernel<G, 32, F8><<<grid, block, 0, s>>>(a); break;
    case 64: decode_mfma_kernel<G, 64, F8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G, bool F8>
hipError_t launch_balanced_g(const DecodeArgs& a, int block_size, int kh, hipStream_t s) {
  const dim3 grid(a.num_kv_heads / kh, a.slices);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: decode_balanced_kernel<G, 8, F8><<<grid, block, 0, s>>>(a); break;
    case 16: decode_balanced_kernel<G, 16, F8><<<grid, block, 0, s>>>(a); break;
    case 32: decode_balanced_kernel<G, 32, F8><<<grid, block, 0, s>>>(a); break;
    case 64: decode_balanced_kernel<G, 64, F8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // At most one slice per sequence names a cut sequence to merge.
  const int reduce_wgs = a.num_seqs < a.slices ? a.num_seqs : a.slices;
  balanced_reduce_kernel<G><<<dim3(reduce_wgs, a.num_kv_heads / kh, G), block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int mfma_waves_per_group(int num_kv_heads) {
  for (int kh = kMaxWaves; kh > 1; kh >>= 1)
    if (num_kv_heads % kh == 0) return kh;
  return 1;
}

namespace {

template <bool F8>
hipError_t launch_mfma_typed(const DecodeArgs& a, int block_size, int group, hipStream_t s) {
  if (a.slices > 0) {
    const int kh = mfma_waves_per_group(a.num_kv_heads);
    if (a.num_seqs > kMaxBalancedSeqs) return hipErrorInvalidValue;
    switch (group) {
      case 1: return launch_balanced_g<1, F8>(a, block_size, kh, s);
      case 2: return launch_balanced_g<2, F8>(a, block_size, kh, s);
      case 4: return launch_balanced_g<4, F8>(a, block_size, kh, s);
      case 8: return launch_balanced_g<8, F8>(a, block_size, kh, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int kh = mfma_waves_per_group(a.num_kv_heads);
  switch (group) {
    case 1: return launch_partitions_g<1, F8>(a, block_size, kh, s);
    case 2: return launch_partitions_g<2, F8>(a, block_size, kh, s);
    case 4: return launch_partitions_g<4, F8>(a, block_size, kh, s);
    case 8: return launch_partitions_g<8, F8>(a, block_size, kh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_mfma_decode(const DecodeArgs& a, int block_size, int group, hipStream_t s,
                              bool fp8) {
  return fp8 ? launch_mfma_typed<true>(a, block_size, group, s)
             : launch_mfma_typed<false>(a, block_size, group, s);
}

}  // namespace pkv
