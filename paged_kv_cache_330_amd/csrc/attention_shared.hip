// Decode-step attention for groups of sequences that share a prefix of their
// KV cache, bf16 or E4M3 pools with head_dim 128, on the matrix cores of
// gfx950 (E4M3 tiles are widened to bf16 on load, as in the plain decode).
//
// What is shared ("PagedAttention 动态内存分页", section "写时复制与内存共享";
// "Paged KV" wiki, section "支持 Prefix Cache"): sequences forked from one
// prompt (parallel sampling, beam search) map the prompt's tokens to the same
// physical blocks, read-only, so the prompt's K/V is stored once.  Sharing
// changes where tokens are stored, not what attention computes, so the result
// is that of pkv_attention_decode over the same tables.  What changes here is
// how often a shared block is read: once per group of sharers instead of once
// per sequence.
//
// Each member's tokens split into the group's shared prefix [0, P) and its own
// tail [P, L), P = the group's shared length rounded down to a multiple of 16.
// Each part yields a running max, sum and unnormalised output per query head,
// and the parts merge by max/sum rescaling, the same merge that joins split
// token ranges of the plain decode ("Paged KV" wiki, "与 FlashAttention 的关系").
//
// Streams.  A prefix stream covers the prefix of up to M = 32 / G members of
// one group: its waves read the group's blocks through the first member's
// table and use all 32 query columns of two 16-column MFMA sets (column
// 16 n + col = member (16 n + col) / G, head col % G), so Q.K^T and P.V are
// dense products of the K/V tile with 32 queries.  A tail stream covers one
// sequence's own tokens with the G heads of its kv head, as in the plain
// decode.  The 16-token chunks of all prefix streams, then of all tail
// streams, are laid end to end, each stream preceded by a few units that
// stand for the start-up of its first piece, and every workgroup takes a
// slice of that weighted stream (equal up to the XCD-parity share, at least
// one unit), as in the balanced schedule of the plain decode.  Every workgroup derives the whole layout
// from the group description and seq_lens in LDS.
//
// Partial results.  A piece of stream st in slice s leaves its partial rows
// at piece id st + s: consecutive streams never share a piece id, because the
// next stream starts in the slice where this one ends or later.  Prefix
// pieces use rows [(st + s) * Hkv + kvh][32 columns], tail pieces rows
// [(b + s) * Hkv + kvh][G] after them.  A sequence with no prefix whose tail
// lies in one slice writes its output directly; every other sequence is
// completed by shared_merge_kernel from the descriptor workgroup (0, 0)
// leaves for it.
//
// Checks: group offsets that start above 0, decrease or pass num_seqs make the
// call ignore the sharing (plain decode) and flag kErrShared; a member id
// outside [0, num_seqs), a sequence listed twice, a shared length outside
// [0, seq_len] of a member, or a member whose table differs from the first
// member's over the prefix is flagged too (the output is then unspecified, but
// every access stays inside the buffers).
#include "decode_mfma.h"

namespace pkv {
namespace {

constexpr int kCols = 16 * kSharedSets;                      // query columns of a prefix stream
template <int G>
constexpr int kMembers = kCols / G;                          // sequences per prefix stream
constexpr int kMaxPrefixStreams = kMaxBalancedSeqs + kMaxBalancedSeqs / kMembers<8>;
constexpr int kMaxStreams = kMaxPrefixStreams + kMaxBalancedSeqs;
// Start-up of a stream's first piece, in chunks, charged in the split: before
// its first tile a prefix piece loads its members' queries and the lead's
// table and checks the members' tables, a tail piece loads its table window
// and queries.  Measured per piece, bf16 pools: prefix about 9 us and tail
// about 2.5 us against 2.6 us per chunk streamed; FP8 pools stream a chunk in
// about 1.5 us, so the same start-up is worth more chunks.
template <bool F8>
constexpr int kStartPrefix = F8 ? 8 : 5;
template <bool F8>
constexpr int kStartTail = F8 ? 2 : 1;

// Writes the partial results of a prefix piece: stream column cw = 16 n + col
// goes to row row0 + cw when cw < ncols (the columns of existing members).
template <int NS>
__device__ __forceinline__ void store_columns(const DecodeArgs& a, MfmaState<NS>& st, int64_t row0,
                                              int ncols) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    st.l[n] += __shfl_xor(st.l[n], 16);
    st.l[n] += __shfl_xor(st.l[n], 32);
    const int cw = 16 * n + col;
    if (cw < ncols) {
      const int64_t row = row0 + cw;
      float* dst = a.ws_acc + row * kD + 4 * qr;
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = st.o[n][j];
      if (qr == 0) {
        a.ws_max[row] = st.m[n];
        a.ws_sum[row] = st.l[n];
      }
    }
  }
}

// Workgroup (kv-head group, slice); wave w owns kv head blockIdx.x * KH + w.
template <int G, int BS, bool F8>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_shared_kernel(SharedArgs sa) {
  static_assert(16 % G == 0, "group must divide 16");
  constexpr int MPS = kMembers<G>;
  const DecodeArgs& a = sa.d;
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[kMaxWaves * 16 * kKRowPad];
  __shared__ u32x4_t s_vt[kMaxWaves * 16 * kVRowPad];  // prefix pieces: P.V on the matrix cores
  __shared__ int s_goff[kMaxBalancedSeqs + 1];  // member offsets of the groups
  __shared__ int s_gsp[kMaxBalancedSeqs + 1];   // first prefix stream of each group
  __shared__ int s_midx[kMaxBalancedSeqs];      // member index of each sequence, or -1
  __shared__ int s_gseq[kMaxBalancedSeqs];      // the member list (group_seqs) as given
  __shared__ int s_tail[kMaxBalancedSeqs];      // first token of each sequence's tail
  __shared__ int s_len[kMaxBalancedSeqs];       // clamped length of each sequence
  __shared__ int s_glen[kMaxBalancedSeqs];      // shared length of each group as given
  __shared__ int s_cc[kMaxStreams + 1];         // first chunk of each stream
  __shared__ int s_wsum[kMaxWaves];
  __shared__ int s_bad;
  __shared__ int s_prog[kMaxWaves];  // tiles streamed by each wave (issue balancing)

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
  const int kvh = blockIdx.x * (blockDim.x >> 6) + wave;
  const int slice = blockIdx.y, S = gridDim.y;
  const int B = a.num_seqs;
  const bool reporter = blockIdx.x == 0 && slice == 0;
  const int cap = a.max_blocks_per_seq * BS;
  u32x4_t* k_lds = s_kt + wave * 16 * kKRowPad;
  u32x4_t* v_lds = s_vt + wave * 16 * kVRowPad;

  // 1. One round of independent global loads: group offsets, shared lengths,
  //    sequence lengths.  Offsets must start at 0, not decrease and stay
  //    <= B; otherwise the sharing is ignored.
  int NG = sa.num_groups;  // 0: the group arrays may be NULL and are not read
  if (threadIdx.x == 0) s_bad = 0;
  if (threadIdx.x < kMaxWaves) s_prog[threadIdx.x] = 0;
  __syncthreads();
  int* prog = blockDim.x == 8 * 64 ? s_prog : nullptr;
  for (int g = threadIdx.x; g <= NG && NG > 0; g += blockDim.x) {
    const int o = sa.group_offsets[g];
    s_goff[g] = o;
    if ((g == 0 && o != 0) || o < 0 || o > B) s_bad = 1;
    if (g < NG) s_glen[g] = sa.group_lens[g];
  }
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    s_len[b] = clamped_len(a, BS, b, reporter);
    s_midx[b] = -1;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < NG; g += blockDim.x)
    if (s_goff[g] > s_goff[g + 1]) s_bad = 1;
  __syncthreads();
  if (s_bad) {
    if (reporter && threadIdx.x == 0) atomicOr(a.err, kErrShared);
    NG = 0;
  }
  const int M = NG > 0 ? s_goff[NG] : 0;
  // Prefix-stream tokens of group g: its shared length clamped to the table
  // width, rounded down to whole chunks.
  auto prefix_tokens = [&](int g) {
    const int P = s_glen[g];
    return (P < 0 ? 0 : min(P, cap)) & ~15;
  };

  // 2. Member index of every sequence (the last listing wins, deterministically).
  for (int i = threadIdx.x; i < M; i += blockDim.x) {
    const int seq = sa.group_seqs[i];
    s_gseq[i] = seq;
    if (static_cast<unsigned>(seq) >= static_cast<unsigned>(B)) {
      if (reporter) atomicOr(a.err, kErrShared);
    } else if (atomicMax(&s_midx[seq], i) >= 0) {
      if (reporter) atomicOr(a.err, kErrShared);  // listed twice
    }
  }

  // 3. Prefix streams: ceil(members / MPS) per group with a prefix of >= 16 tokens.
  const int NPS = block_scan(NG, s_gsp, s_wsum, [&](int g) {
    const int n = s_goff[g + 1] - s_goff[g];
    return prefix_tokens(g) > 0 ? (n + MPS - 1) / MPS : 0;
  });

  // 4. First tail token of every sequence: its group's prefix-stream length.
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int i = s_midx[b];
    int t = 0;
    if (i >= 0) {
      const int g = last_at_most(s_goff, NG, i);
      t = prefix_tokens(g);
      if (reporter && (s_glen[g] < 0 || s_glen[g] > s_len[b])) atomicOr(a.err, kErrShared);
    }
    s_tail[b] = t;
  }
  __syncthreads();

  // 5. The streams laid end to end: NPS prefix streams, then one tail per
  //    sequence.  Each non-empty stream counts its chunks plus the start-up
  //    its first piece costs, in chunks (kStartPrefix, kStartTail), so that a
  //    slice that starts many streams gets fewer chunks (each slice also
  //    continues one stream, so those start-ups even out).  s_cc holds these
  //    weighted positions; stream st's chunk j sits at s_cc[st] + K(st) + j.
  const int NST = NPS + B;
  auto stream_chunks = [&](int st) {
    if (st < NPS) return prefix_tokens(last_at_most(s_gsp, NG, st)) >> 4;
    const int b = st - NPS;
    return s_len[b] > s_tail[b] ? (s_len[b] - s_tail[b] + 15) >> 4 : 0;
  };
  const int total = block_scan(NST, s_cc, s_wsum, [&](int st) {
    const int n = stream_chunks(st);
    return n > 0 ? n + (st < NPS ? kStartPrefix<F8> : kStartTail<F8>) : 0;
  });
  const SliceSplit split = SliceSplit::make<F8>(total, S, gridDim.x);
  // start-up units and chunks of stream st, from its weighted span
  auto span = [&](int st, int& k, int& n) {
    const int w = s_cc[st + 1] - s_cc[st];
    k = w > 0 ? (st < NPS ? kStartPrefix<F8> : kStartTail<F8>) : 0;
    n = w - k;
  };

  // 6. Merge descriptors, one workgroup: (merge needed, tail slices [tf, tl],
  //    prefix stream or -1, its slices [pf, pl], the member's first column).
  //    A stream's pieces lie in the slices of its first and last chunks and
  //    every slice between.
  if (blockIdx.x == 0 && slice == 0) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      int k, n;
      span(NPS + b, k, n);
      int tf = 0, tl = -1, pst = -1, pf = 0, pl = -1, cb = 0;
      if (n > 0) {
        tf = split.slice_of(s_cc[NPS + b] + k);
        tl = split.slice_of(s_cc[NPS + b] + k + n - 1);
      }
      if (s_tail[b] > 0) {
        const int i = s_midx[b];
        const int g = last_at_most(s_goff, NG, i);
        const int m = i - s_goff[g];
        pst = s_gsp[g] + m / MPS;
        int pk, pn;
        span(pst, pk, pn);
        pf = split.slice_of(s_cc[pst] + pk);
        pl = split.slice_of(s_cc[pst] + pk + pn - 1);
        cb = (m % MPS) * G;
      }
      int* d = a.ws_desc + kSharedDescInts * b;
      d[0] = (pst >= 0 || tl > tf) ? 1 : 0;
      d[1] = tf;
      d[2] = tl;
      d[3] = pst;
      d[4] = pf;
      d[5] = pl;
      d[6] = cb;
      d[7] = 0;
    }
  }
  if (slice == 0)  // sequences with no token at all get zero rows
    zero_rows_where<G>(a, B, kvh, [&](int j) {
      return s_tail[j] == 0 && s_cc[NPS + j + 1] == s_cc[NPS + j];
    });

  // 7. This slice's part [x_lo, x_hi) of the weighted stream.
  const int x_lo = min(total, split.begin(slice));
  const int x_hi = min(total, split.end(slice));
  if (x_lo >= x_hi) return;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  int st = last_at_most(s_cc, NST, x_lo);
  int x = x_lo;
  while (x < x_hi) {
    while (s_cc[st + 1] <= x) ++st;  // skip empty streams and those ending at x
    int k, n;
    span(st, k, n);
    const int w0 = s_cc[st] + k;               // weighted position of chunk 0
    const int c0 = max(0, x - w0);             // this piece's chunks [c0, c1) of the stream
    const int c1 = min(n, x_hi - w0);
    x = min(x_hi, s_cc[st + 1]);
    if (c1 <= c0) continue;                    // only the stream's start-up falls here
    if (st < NPS) {
      // Prefix piece: members m0 .. m0 + nm - 1 of group g, through m0's table.
      const int g = last_at_most(s_gsp, NG, st);
      const int m0 = s_goff[g] + (st - s_gsp[g]) * MPS;
      const int nm = min(MPS, s_goff[g + 1] - m0);
      int lead = s_gseq[m0];
      if (static_cast<unsigned>(lead) >= static_cast<unsigned>(B)) lead = 0;
      QueryOperand<F8> qop[kSharedSets];
#pragma unroll
      for (int s2 = 0; s2 < kSharedSets; ++s2) {
        const int mi = (16 * s2 + col) / G;
        int seq = mi < nm ? s_gseq[m0 + mi] : lead;
        if (static_cast<unsigned>(seq) >= static_cast<unsigned>(B)) seq = lead;
        load_qop(q + ((int64_t)seq * a.num_q_heads + kvh * G + col % G) * kD, qr, qop[s2]);
      }
      MfmaState<kSharedSets> ps;
      ps.reset();
      attend_table<BS, true, F8>(a, s_bt, k_lds, v_lds,
                                 a.block_tables + (int64_t)lead * a.max_blocks_per_seq, kvh,
                                 c0 * 16, c1 * 16, qop, ps, TableCheck{s_gseq + m0, nm},
                                 WindowTokens{}, prog);
      store_columns(a, ps, ((int64_t)(st + slice) * a.num_kv_heads + kvh) * kCols, nm * G);
    } else {
      // Tail piece of sequence b: tokens T + 16 c0 .. of its own table.
      const int b = st - NPS;
      const int L = s_len[b];
      const int T = s_tail[b];
      QueryOperand<F8> qop[1];
      load_query<G>(a, b, kvh, col, qr, qop);
      WaveState<G> ws;
      ws.reset();
      attend_range<G, BS, F8>(a, s_bt, k_lds, v_lds, b, kvh, T + c0 * 16, min(T + c1 * 16, L),
                              qop, ws, prog);
      Sink sink{nullptr, nullptr, nullptr, 0, 0};
      if (!(T == 0 && c0 == 0 && c1 == n))
        sink = Sink{a.ws_acc, a.ws_max, a.ws_sum,
                    sa.prefix_rows + ((int64_t)(b + slice) * a.num_kv_heads + kvh) * G, 1};
      finish_wave<G>(a, ws, b, kvh, sink);
    }
  }
}

// Completes every sequence whose descriptor asks for it: workgroup (sequence,
// 4 query heads), wave w for head 4 blockIdx.y + w, lane for output dims
// 2 lane and 2 lane + 1.  The pieces are merged with a running maximum, so
// their loads are independent:
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p.
template <int G>
__global__ __launch_bounds__(256) void shared_merge_kernel(SharedArgs sa) {
  const DecodeArgs& a = sa.d;
  const int b = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= a.num_q_heads) return;
  const int* d = a.ws_desc + kSharedDescInts * b;
  if (d[0] == 0) return;
  const int kvh = h / G, hg = h % G;
  const int dd = 2 * (threadIdx.x & 63);
  const float* __restrict__ wmax = a.ws_max;
  const float* __restrict__ wsum = a.ws_sum;
  const float* __restrict__ wacc = a.ws_acc;
  float M = -INFINITY, den = 0.f, num0 = 0.f, num1 = 0.f;
  auto merge = [&](int64_t row) {
    const float m = wmax[row], l = wsum[row];
    const float2 acc = *reinterpret_cast<const float2*>(wacc + row * kD + dd);
    const float Mn = fmaxf(M, m);
    const float c_old = rescale(M, Mn), c_new = exp2_hw(m - Mn);
    den = den * c_old + l * c_new;
    num0 = num0 * c_old + acc.x * c_new;
    num1 = num1 * c_old + acc.y * c_new;
    M = Mn;
  };
  const int tf = d[1], tl = d[2], pst = d[3], pf = d[4], pl = d[5], cb = d[6];
#pragma unroll 2
  for (int s = tf; s <= tl; ++s)
    merge(sa.prefix_rows + ((int64_t)(b + s) * a.num_kv_heads + kvh) * G + hg);
  if (pst >= 0) {
#pragma unroll 2
    for (int s = pf; s <= pl; ++s)
      merge(((int64_t)(pst + s) * a.num_kv_heads + kvh) * kCols + cb + hg);
  }
  const int64_t o = ((int64_t)b * a.num_q_heads + h) * kD + dd;
  store_out(a, o, num0 / den);
  store_out(a, o + 1, num1 / den);
}

template <int G, bool F8>
hipError_t launch_shared_g(const SharedArgs& a, int block_size, int kh, hipStream_t s) {
  const dim3 grid(a.d.num_kv_heads / kh, a.d.slices);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: decode_shared_kernel<G, 8, F8><<<grid, block, 0, s>>>(a); break;
    case 16: decode_shared_kernel<G, 16, F8><<<grid, block, 0, s>>>(a); break;
    case 32: decode_shared_kernel<G, 32, F8><<<grid, block, 0, s>>>(a); break;
    case 64: decode_shared_kernel<G, 64, F8><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  shared_merge_kernel<G><<<dim3(a.d.num_seqs, (a.d.num_q_heads + 3) / 4), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_shared_decode(const SharedArgs& a, int block_size, int group, hipStream_t s,
                                bool fp8) {
  if (a.d.num_seqs < 1 || a.d.num_seqs > kMaxBalancedSeqs || a.num_groups < 0 ||
      a.num_groups > a.d.num_seqs)
    return hipErrorInvalidValue;
  const int kh = mfma_waves_per_group(a.d.num_kv_heads);
  switch (group) {
    case 1: return fp8 ? launch_shared_g<1, true>(a, block_size, kh, s)
                         : launch_shared_g<1, false>(a, block_size, kh, s);
    case 2: return fp8 ? launch_shared_g<2, true>(a, block_size, kh, s)
                         : launch_shared_g<2, false>(a, block_size, kh, s);
    case 4: return fp8 ? launch_shared_g<4, true>(a, block_size, kh, s)
                         : launch_shared_g<4, false>(a, block_size, kh, s);
    case 8: return fp8 ? launch_shared_g<8, true>(a, block_size, kh, s)
                         : launch_shared_g<8, false>(a, block_size, kh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
