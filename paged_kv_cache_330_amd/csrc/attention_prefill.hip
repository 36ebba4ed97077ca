// Prefill attention over the paged pools: a chunk of new tokens per sequence
// (a whole prompt, or the next part of one after cached context) attends
// causally to the sequence's cached tokens.  bf16 or FP8 E4M3 pools (with a
// scale per block and kv head) with head_dim 128, on the matrix cores of
// gfx950.
//
// What is computed ("Paged KV" wiki, section "运行阶段": at prefill a sequence
// takes blocks in order and its K/V are filled in; section "Attention Kernel
// 的适配": K/V are read block by block through the block table): the new
// tokens' K/V are already in the cache (the slot-mapping write with N
// tokens), and the token at position p attends to the cached tokens 0 .. p.
// The decode step is the one-token case.
//
// Work split.  A work item is QT = 4 x 32 / G consecutive new tokens of one
// sequence and one kv head (grid x: work items, grid y: kv heads).  Its four
// waves each take 32 / G of the tokens: their 32 x G queries fill the 32
// columns of two 16-column MFMA sets (column 16 n + col: token
// (16 n + col) / G of the wave, head col % G), so Q.K^T and P.V are dense
// products of each K/V tile with 32 queries per wave.  The item streams its
// key range, tokens 0 .. (position of its last token), through the block
// table in 32-token tiles shared by the four waves: per 16-token chunk, every
// lane loads one 16-byte unit of a K row and of a V row into double-buffered
// LDS tiles (one barrier per tile; the next tile's loads are in flight while
// the current one is computed), and each wave reads its K and V operands
// from there (its Q operands stay in registers), masking the tokens after its
// own columns' positions on the tiles that reach them.  Sharing each tile between four
// waves cuts the K/V reads per query four times against one wave per tile.
// Items are numbered sequence by sequence from the per-sequence counts (a
// prefix scan in LDS) and dispatched from the last to the first, so the
// longest key ranges of each sequence start early.  The grid is
// one-dimensional and XCD-aware: workgroups are dealt round-robin over the
// eight XCDs, so the linear id is remapped to give each XCD a contiguous
// range of (kv head, item) pairs: the items of one sequence and kv head then
// run together on one XCD and re-read their K/V from its L2.
//
// Checks: a query range with query_start[b] < 0, query_start[b + 1] <
// query_start[b], query_start[b + 1] > num_tokens, or more new tokens than
// seq_lens[b] is flagged (kErrQuery) and that sequence is skipped.
#include "decode_mfma.h"

namespace pkv {
namespace {

constexpr int kCols = 16 * kSharedSets;  // query columns of a wave
constexpr int kItemWaves = 4;            // waves of a work item, sharing each K/V tile
constexpr int kItemThreads = kItemWaves * 64;
constexpr int kTC = 2;                   // 16-token chunks per shared K/V tile
constexpr int kTileRows = 16 * kTC;      // tokens per tile
static_assert(kItemThreads == 16 * 16, "one 16-byte unit of 16 rows per lane and chunk");

constexpr int kXcds = 8;  // XCDs of the device; workgroups go round-robin over them

constexpr float kStaleMax = 8.f;  // log2 headroom of the running max

// Sum of a lane's TC x 4 probabilities as a tree (a chain of adds would wait
// on the adder's latency at every step).
template <int TC>
__device__ __forceinline__ float tile_sum(const float (&x)[TC][4]) {
  float s[TC];
#pragma unroll
  for (int c = 0; c < TC; ++c) s[c] = (x[c][0] + x[c][1]) + (x[c][2] + x[c][3]);
#pragma unroll
  for (int w = 1; w < TC; w <<= 1)
#pragma unroll
    for (int c = 0; c + w < TC; c += 2 * w) s[c] += s[c + w];
  return s[0];
}

// Online-softmax step of one column that moves the running max m only when
// the tile's maximum exceeds it by more than 2^kStaleMax = 2^8.  Until
// then the probabilities exp2(x - m) stay below 2^8
// (far from the fp32 range, and split into bf16 hi + lo as before) and the
// accumulators need no rescaling.  The normalised result o / l does not
// depend on the m it was accumulated with, so only rounding changes; with a
// causal mask the running max of 32 query columns otherwise moves in most
// tiles of a prompt.  Returns the factor that rescales the state so far
// (exactly 1 when m stays).
template <int TC>
__device__ __forceinline__ float softmax_update_stale(float (&x)[TC][4], float mt, float& m,
                                                      float& l) {
  const float m_new = mt > m + kStaleMax ? mt : m;  // m = -inf: takes mt
  const float alpha = exp2_hw(m - m_new);
  m = m_new;
#pragma unroll
  for (int c = 0; c < TC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[c][i] = exp2_hw(x[c][i] - m_new);
  l = l * alpha + tile_sum<TC>(x);
  return alpha;
}

// softmax_update_stale for raw scores x (not yet multiplied by the positive
// factor sl = scale * log2(e)) and their raw tile maximum mt: since sl > 0,
// the maximum of the scaled scores is mt * sl, and the scaled score enters
// the exponent through one fused multiply-add, exp2(x * sl - m).
template <int TC>
__device__ __forceinline__ float softmax_update_stale_raw(float (&x)[TC][4], float mt, float sl,
                                                          float& m, float& l) {
  const float mts = mt * sl;
  const float m_new = mts > m + kStaleMax ? mts : m;  // m = -inf: takes mts
  const float alpha = exp2_hw(m - m_new);
  m = m_new;
#pragma unroll
  for (int c = 0; c < TC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[c][i] = exp2_hw(fmaf(x[c][i], sl, -m_new));
  l = l * alpha + tile_sum<TC>(x);
  return alpha;
}

// Bijection of [0, n): workgroup id p (on XCD p % kXcds) -> a logical id such
// that each XCD holds a contiguous range of logical ids.
__device__ __forceinline__ int xcd_contiguous(int p, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int xcd = p % kXcds, slot = p / kXcds;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// One lane's share of a 32-token K/V tile in registers, between its loads
// and its staging into LDS: per 16-token chunk, one 16-byte unit of bf16
// (8 dims) of a K row and of a V row, or for FP8 pools the 8 codes of those
// dims and the scales of the row's block.
template <bool F8>
struct TileUnits;
template <>
struct TileUnits<false> {
  u32x4_t k[kTC], v[kTC];
};
template <>
struct TileUnits<true> {
  u32x2_t k[kTC], v[kTC];
  float ks[kTC], vs[kTC];
};

template <int G, int BS, bool F8>
__global__ __launch_bounds__(kItemThreads, 2) void prefill_kernel(PrefillArgs pa, int items_ub) {
  static_assert(16 % G == 0, "group must divide 16");
  constexpr int QW = kCols / G;         // new tokens per wave
  constexpr int QT = kItemWaves * QW;   // new tokens per work item
  const DecodeArgs& a = pa.d;
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_k[2][kTileRows * kKRowPad];
  __shared__ u32x4_t s_v[2][kTileRows * kVRowPad];
  __shared__ float s_ks[2][F8 ? kTileRows : 1];  // FP8 pools: K and V scale of each row's block
  __shared__ float s_vs[2][F8 ? kTileRows : 1];
  __shared__ int s_item[kMaxBalancedSeqs + 1];  // first work item of each sequence
  __shared__ int s_wsum[kItemWaves];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
  const int logical = xcd_contiguous(blockIdx.x, gridDim.x);
  const int kvh = logical / items_ub;
  const int item_rev = logical - kvh * items_ub;  // 0: the last item
  const int B = a.num_seqs;
  const bool reporter = blockIdx.x == 0;
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
  const int item = W - 1 - item_rev;
  if (item < 0) return;
  const int b = last_at_most(s_item, B, item);
  const int n = new_tokens(b, false);  // > 0: b owns this item
  const int r0 = qs[b];
  const int pos0 = clamped_len(a, BS, b, false) - n;  // position of new token 0
  const int t0 = (item - s_item[b]) * QT;
  const int t1 = min(n, t0 + QT);          // the item's new tokens [t0, t1)
  const int wt0 = t0 + wave * QW;          // this wave's: [wt0, min(t1, wt0 + QW))
  const int wt1 = min(t1, wt0 + QW);

  // Columns: query rows and causal limits (a column past the item's last
  // token repeats it; its output is not stored).  The Q operands stay in
  // registers for the whole key range.
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  CausalTokens<kSharedSets> lim;
  bf16x8_t qop[kSharedSets][4];
#pragma unroll
  for (int s = 0; s < kSharedSets; ++s) {
    const int t = min(wt0 + (16 * s + col) / G, t1 - 1);
    load_qop(q + ((int64_t)(r0 + t) * a.num_q_heads + kvh * G + col % G) * kD, qr, qop[s]);
    lim.limit[s] = pos0 + t + 1;
  }
  // bf16 pools: the score factor sl = scale * log2(e) is applied inside the
  // exponent (softmax_update_stale_raw), which needs sl > 0.  A negative
  // scale negates the query operands instead (exact: a sign flip of every
  // bf16 value negates every product and sum), and sl = 0 is raised to the
  // smallest normal float, which leaves every exponent's rounding unchanged
  // (|score| * 2^-126 is far below half an ulp of the maximum's shift).
  constexpr bool kFold = !F8;
  float slf = a.scale_log2e;
  if constexpr (kFold) {
    if (slf < 0.f) {
#pragma unroll
      for (int s = 0; s < kSharedSets; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          qop[s][k] = __builtin_bit_cast(bf16x8_t, __builtin_bit_cast(u32x4_t, qop[s][k]) ^ 0x80008000u);
      slf = -slf;
    }
    slf = fmaxf(slf, 1.17549435e-38f);
  }
  MfmaState<kSharedSets> st;
  st.reset();

  // The lane's units of each tile: rows urow + 16 c, 16 bytes at dims 8 ucol ..
  const int urow = threadIdx.x >> 4, ucol = threadIdx.x & 15;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * kD;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * kD + 8 * ucol;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * kD + 8 * ucol;
  const uint8_t* kbase8 = static_cast<const uint8_t*>(a.k_cache) + (int64_t)kvh * kD + 8 * ucol;
  const uint8_t* vbase8 = static_cast<const uint8_t*>(a.v_cache) + (int64_t)kvh * kD + 8 * ucol;
  constexpr int es = F8 ? 1 : 2;  // bytes per stored element
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k_cache) + (int64_t)kvh * kD * es;
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v_cache) + (int64_t)kvh * kD * es;
  const uint32_t row_bytes = (uint32_t)(tok_stride * es);
  const uint32_t lane_bytes = (uint32_t)(8 * ucol * es);
  const uint32_t row_off = (uint32_t)urow * row_bytes + lane_bytes;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const int kend = pos0 + t1;  // key tokens of the item: 0 .. kend - 1
  // Every column attends to the keys before its first column's limit.
  const int first_limit = pos0 + min(wt0, t1 - 1) + 1;
  for (int w0 = 0; w0 < kend; w0 += kMaxPartitionTokens) {
    const int wend = min(kend, w0 + kMaxPartitionTokens);
    // tiles that end at or before this key need no mask
    const int mask_from = min(wend, first_limit);
    const int blk0 = w0 / BS;
    const int nblk = (wend - 1) / BS - blk0 + 1;
    __syncthreads();  // every wave is done with the previous window's ids and tiles
    for (int i = threadIdx.x; i < nblk; i += blockDim.x)
      s_bt[i] = checked_block(bt, blk0 + i, a.num_blocks, a.err);
    __syncthreads();
    // Rows past the window's end re-read its last token (masked).
    const int last_chunk = ((wend - 1) >> 4) << 4;  // start of the window's last 16-token chunk
    auto load_units = [&](int tt, TileUnits<F8>& u) {
#pragma unroll
      for (int c = 0; c < kTC; ++c) {
        if constexpr (BS >= 16) {
          // The chunk lies in one block: its address is wave-uniform and a
          // lane adds the 32-bit offset of its row, clamped to the window's
          // last token.  A chunk wholly past the end re-reads the last chunk
          // (never computed unmasked).
          const int tce = __builtin_amdgcn_readfirstlane(min(tt + 16 * c, last_chunk));
          const int lim = __builtin_amdgcn_readfirstlane(wend - 1 - tce);  // >= 0
          const int phys = __builtin_amdgcn_readfirstlane(s_bt[tce / BS - blk0]);
          const int64_t first = ((int64_t)phys * BS + (tce & (BS - 1))) * row_bytes;
          const uint32_t off = min(row_off, (uint32_t)lim * row_bytes + lane_bytes);
          if constexpr (F8) {
            u.k[c] = *reinterpret_cast<const u32x2_t*>(kpool + first + off);
            u.v[c] = *reinterpret_cast<const u32x2_t*>(vpool + first + off);
            u.ks[c] = a.k_scale[(int64_t)phys * a.num_kv_heads + kvh];
            u.vs[c] = a.v_scale[(int64_t)phys * a.num_kv_heads + kvh];
          } else {
            u.k[c] = *reinterpret_cast<const u32x4_t*>(kpool + first + off);
            u.v[c] = *reinterpret_cast<const u32x4_t*>(vpool + first + off);
          }
        } else {
          const int tok = min(tt + 16 * c + urow, wend - 1);
          const int phys = s_bt[tok / BS - blk0];
          const int64_t row = ((int64_t)phys * BS + (tok & (BS - 1))) * tok_stride;
          if constexpr (F8) {
            u.k[c] = *reinterpret_cast<const u32x2_t*>(kbase8 + row);
            u.v[c] = *reinterpret_cast<const u32x2_t*>(vbase8 + row);
            u.ks[c] = a.k_scale[(int64_t)phys * a.num_kv_heads + kvh];
            u.vs[c] = a.v_scale[(int64_t)phys * a.num_kv_heads + kvh];
          } else {
            u.k[c] = *reinterpret_cast<const u32x4_t*>(kbase + row);
            u.v[c] = *reinterpret_cast<const u32x4_t*>(vbase + row);
          }
        }
      }
    };
    // FP8 codes are widened to bf16 here (exactly), so the tile in LDS has
    // the layout of bf16 pools; the scales go beside it, one per row.
    auto stage = [&](int buf, const TileUnits<F8>& u) {
#pragma unroll
      for (int c = 0; c < kTC; ++c) {
        if constexpr (F8) {
          s_k[buf][(16 * c + urow) * kKRowPad + ucol] = widen_e4m3(u.k[c]);
          s_v[buf][(16 * c + urow) * kVRowPad + ucol] = widen_e4m3(u.v[c]);
          if (ucol == 0) {
            s_ks[buf][16 * c + urow] = u.ks[c];
            s_vs[buf][16 * c + urow] = u.vs[c];
          }
        } else {
          s_k[buf][(16 * c + urow) * kKRowPad + ucol] = u.k[c];
          s_v[buf][(16 * c + urow) * kVRowPad + ucol] = u.v[c];
        }
      }
    };
    auto compute = [&](int buf, int tt) {
      const u32x4_t* kt = s_k[buf];
      float x[kSharedSets][kTC][4], mt[kSharedSets], alpha[kSharedSets];
      __builtin_amdgcn_s_setprio(1);  // Q.K^T: this wave's products go first
      {
        // four independent accumulator chains (chunk, column set), k-step by
        // k-step, so that consecutive products never wait on each other
        u32x4_t kop[kTC][4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int c = 0; c < kTC; ++c) kop[c][s] = kt[(16 * c + col) * kKRowPad + 4 * s + qr];
        f32x4_t sacc[kTC][kSharedSets];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int c = 0; c < kTC; ++c)
#pragma unroll
            for (int m = 0; m < kSharedSets; ++m)
              sacc[c][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, kop[c][s]), qop[m][s],
                  s == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : sacc[c][m], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kTC; ++c) {
          // FP8: the lane's 4 rows (4 qr ..) lie in one block; its K scale
          // multiplies their scores
          const float sl = F8 ? a.scale_log2e * s_ks[buf][16 * c + 4 * qr] : a.scale_log2e;
#pragma unroll
          for (int m = 0; m < kSharedSets; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[m][c][i] = kFold ? sacc[c][m][i] : sacc[c][m][i] * sl;
        }
      }
      __builtin_amdgcn_s_setprio(0);  // softmax: the other wave's products may go first
      if (tt + kTileRows > mask_from) {  // the causal diagonal or the window's end
#pragma unroll
        for (int c = 0; c < kTC; ++c)
#pragma unroll
          for (int m = 0; m < kSharedSets; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (!lim.valid(m, tt + 16 * c + 4 * qr + i, wend)) x[m][c][i] = -INFINITY;
      }
#pragma unroll
      for (int m = 0; m < kSharedSets; ++m) {
        mt[m] = -INFINITY;
#pragma unroll
        for (int c = 0; c < kTC; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) mt[m] = fmaxf(mt[m], x[m][c][i]);
      }
      column_max<kSharedSets>(mt);
#pragma unroll
      for (int m = 0; m < kSharedSets; ++m)
        alpha[m] = kFold ? softmax_update_stale_raw<kTC>(x[m], mt[m], slf, st.m[m], st.l[m])
                         : softmax_update_stale<kTC>(x[m], mt[m], st.m[m], st.l[m]);
      if constexpr (F8) {  // dequantised V = scale * code: scale the probabilities (not l)
#pragma unroll
        for (int c = 0; c < kTC; ++c) {
          const float vsc = s_vs[buf][16 * c + 4 * qr];
#pragma unroll
          for (int m = 0; m < kSharedSets; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[m][c][i] *= vsc;
        }
      }
      rescale_lazy<kSharedSets>(alpha, st);
      __builtin_amdgcn_s_setprio(1);  // P.V
      const uint16_t* vt = reinterpret_cast<const uint16_t*>(s_v[buf]);
      static_assert(kTC % 2 == 0, "P.V takes the chunks of a tile in pairs");
#pragma unroll
      for (int c = 0; c < kTC; c += 2)
        pv_pair_from_lds<kTC, kSharedSets>(vt + 16 * c * kVRowPad * 8,
                                           vt + 16 * (c + 1) * kVRowPad * 8, c, c + 1, x, col,
                                           qr, st);
      __builtin_amdgcn_s_setprio(0);
    };
    // Two tiles in flight: registers a and b alternate, tile t is computed
    // from LDS buffer t & 1 while tiles t + 1 (staged next) and t + 2 load.
    // Pairs of tiles with a single loop exit (an exit per half makes the
    // compiler wait for every load at the loop head).
    constexpr int T = kTileRows;
    const int ntile = (wend - w0 + T - 1) / T;
    TileUnits<F8> ua, ub;
    load_units(w0, ua);
    load_units(w0 + T, ub);
    stage(0, ua);
    const int npair = ntile >> 1;
    for (int p = 0; p < npair; ++p) {
      const int tt = w0 + 2 * T * p;
      load_units(tt + 2 * T, ua);  // tile 2p + 2
      __syncthreads();                 // tile 2p is in buffer 0; tile 2p - 1 is done
      compute(0, tt);
      stage(1, ub);                // tile 2p + 1
      load_units(tt + 3 * T, ub);  // tile 2p + 3
      __syncthreads();
      compute(1, tt + T);
      stage(0, ua);                // tile 2p + 2
    }
    if (ntile & 1) {
      __syncthreads();
      compute(0, w0 + 2 * T * npair);
    }
  }

  // Normalised outputs of the wave's columns.
#pragma unroll
  for (int s = 0; s < kSharedSets; ++s) {
    st.l[s] += __shfl_xor(st.l[s], 16);
    st.l[s] += __shfl_xor(st.l[s], 32);
    const int t = wt0 + (16 * s + col) / G;
    if (t < wt1) {
      const int64_t o = ((int64_t)(r0 + t) * a.num_q_heads + kvh * G + col % G) * kD + 4 * qr;
      const float inv = 1.f / st.l[s];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(a, o + 16 * j + i, st.o[s][j][i] * inv);
    }
  }
}

template <int G, bool F8>
hipError_t launch_prefill_g(const PrefillArgs& a, int block_size, hipStream_t s) {
  constexpr int QT = kItemWaves * kCols / G;
  // Work items: at most ceil(T / QT) + B when the query ranges are consistent.
  const int64_t items = (a.num_tokens + QT - 1) / QT + a.d.num_seqs;
  const int64_t total = items * a.d.num_kv_heads;
  if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int ub = static_cast<int>(items);
  const dim3 grid(static_cast<unsigned>(total));
  const dim3 block(kItemThreads);
  switch (block_size) {
    case 8: prefill_kernel<G, 8, F8><<<grid, block, 0, s>>>(a, ub); break;
    case 16: prefill_kernel<G, 16, F8><<<grid, block, 0, s>>>(a, ub); break;
    case 32: prefill_kernel<G, 32, F8><<<grid, block, 0, s>>>(a, ub); break;
    case 64: prefill_kernel<G, 64, F8><<<grid, block, 0, s>>>(a, ub); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool F8>
hipError_t launch_prefill_typed(const PrefillArgs& a, int block_size, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_prefill_g<1, F8>(a, block_size, s);
    case 2: return launch_prefill_g<2, F8>(a, block_size, s);
    case 4: return launch_prefill_g<4, F8>(a, block_size, s);
    case 8: return launch_prefill_g<8, F8>(a, block_size, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int block_size, int group, hipStream_t s,
                          bool fp8) {
  if (a.d.num_seqs < 1 || a.d.num_seqs > kMaxBalancedSeqs || a.num_tokens < 1 ||
      a.num_tokens > 0x7FFFFFFF)
    return hipErrorInvalidValue;
  return fp8 ? launch_prefill_typed<true>(a, block_size, group, s)
             : launch_prefill_typed<false>(a, block_size, group, s);
}

}  // namespace pkv
