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
// streams, are laid end to end and every workgroup takes an equal slice
// (at least one chunk), as in the balanced schedule of the
// plain decode.  Every workgroup derives the whole layout from the group
// description and seq_lens in LDS.
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

  // 5. Chunks of every stream: NPS prefix streams, then one tail per sequence.
  const int NST = NPS + B;
  const int total = block_scan(NST, s_cc, s_wsum, [&](int st) {
    if (st < NPS) return prefix_tokens(last_at_most(s_gsp, NG, st)) >> 4;
    const int b = st - NPS;
    return s_len[b] > s_tail[b] ? (s_len[b] - s_tail[b] + 15) >> 4 : 0;
  });
  const int per = max(1, (total + S - 1) / S);

  // 6. Merge descriptors, one workgroup: (merge needed, tail slices [tf, tl],
  //    prefix stream or -1, its slices [pf, pl], the member's first column).
  if (blockIdx.x == 0 && slice == 0) {
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
      const int cs = s_cc[NPS + b], ce = s_cc[NPS + b + 1];
      int tf = 0, tl = -1, pst = -1, pf = 0, pl = -1, cb = 0;
      if (ce > cs) {
        tf = cs / per;
        tl = (ce - 1) / per;
      }
      if (s_tail[b] > 0) {
        const int i = s_midx[b];
        const int g = last_at_most(s_goff, NG, i);
        const int k = i - s_goff[g];
        pst = s_gsp[g] + k / MPS;
        pf = s_cc[pst] / per;
        pl = (s_cc[pst + 1] - 1) / per;
        cb = (k % MPS) * G;
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

  // 7. This slice's chunks.
  const int c_lo = slice * per;
  const int c_hi = min(total, c_lo + per);
  if (c_lo >= c_hi) return;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  int st = last_at_most(s_cc, NST, c_lo);
  int c = c_lo;
  while (c < c_hi) {
    while (s_cc[st + 1] <= c) ++st;  // skip streams with no chunks
    const int cs = s_cc[st], ce = s_cc[st + 1];
    const int c_end = min(c_hi, ce);
    if (st < NPS) {
      // Prefix piece: members m0 .. m0 + nm - 1 of group g, through m0's table.
      const int g = last_at_most(s_gsp, NG, st);
      const int m0 = s_goff[g] + (st - s_gsp[g]) * MPS;
      const int nm = min(MPS, s_goff[g + 1] - m0);
      int lead = sa.group_seqs[m0];
      if (static_cast<unsigned>(lead) >= static_cast<unsigned>(B)) lead = 0;
      bf16x8_t qop[kSharedSets][4];
#pragma unroll
      for (int n = 0; n < kSharedSets; ++n) {
        const int mi = (16 * n + col) / G;
        int seq = mi < nm ? sa.group_seqs[m0 + mi] : lead;
        if (static_cast<unsigned>(seq) >= static_cast<unsigned>(B)) seq = lead;
        load_qop(q + ((int64_t)seq * a.num_q_heads + kvh * G + col % G) * kD, qr, qop[n]);
      }
      MfmaState<kSharedSets> ps;
      ps.reset();
      attend_table<BS, true, F8>(a, s_bt, k_lds, v_lds,
                                 a.block_tables + (int64_t)lead * a.max_blocks_per_seq, kvh,
                                 (c - cs) * 16, (c_end - cs) * 16, qop, ps,
                                 TableCheck{sa.group_seqs + m0, nm}, WindowTokens{}, prog);
      store_columns(a, ps, ((int64_t)(st + slice) * a.num_kv_heads + kvh) * kCols, nm * G);
    } else {
      // Tail piece of sequence b: tokens T + 16 (c - cs) .. of its own table.
      const int b = st - NPS;
      const int L = s_len[b];
      const int T = s_tail[b];
      bf16x8_t qop[1][4];
      load_query<G>(a, b, kvh, col, qr, qop);
      WaveState<G> ws;
      ws.reset();
      attend_range<G, BS, F8>(a, s_bt, k_lds, v_lds, b, kvh, T + (c - cs) * 16,
                                  min(T + (c_end - cs) * 16, L), qop, ws, prog);
      Sink sink{nullptr, nullptr, nullptr, 0, 0};
      if (!(T == 0 && c == cs && c_end == ce))
        sink = Sink{a.ws_acc, a.ws_max, a.ws_sum,
                    sa.prefix_rows + ((int64_t)(b + slice) * a.num_kv_heads + kvh) * G, 1};
      finish_wave<G>(a, ws, b, kvh, sink);
    }
    c = c_end;
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
