// Wave-level building blocks of the bf16 head_dim-128 decode kernels on the
// matrix cores of gfx950 (MI355X), shared by attention_mfma.hip (decode over
// independent sequences) and attention_shared.hip (decode with shared prefixes).
//
// What is computed ("Paged KV" wiki, section "Attention Kernel 的适配"): the
// kernel receives the block table and block_size, reaches each logical block
// of a sequence through the table and reads K/V block by block.  The result is
// ordinary softmax attention of one query token per head over the cached
// tokens (the explainer page: paging changes storage, not the attention
// algorithm).  Query head h reads kv head h / G, G = Hq / Hkv.  Token ranges
// are streamed with a running max / sum / unnormalised output in fp32 (the
// block-wise computation that the wiki's "与 FlashAttention 的关系" section
// says combines with block-wise storage) and split ranges are merged by
// max/sum rescaling.
//
// Work split: a workgroup has KH waves (KH = the largest of 8, 4, 2, 1 that
// divides Hkv) and wave w owns kv head kvg * KH + w of a token range.  All
// waves of a workgroup therefore read the same physical blocks at the same
// time, each its own 256-byte slice of every 2 KiB token row (Hkv = 8): the
// workgroup reads whole blocks, and the blocks' address translations are
// shared by its waves.  Each wave keeps its own kv head's softmax state, so
// no cross-wave merge is needed; the block ids of the range are read into LDS
// once for all waves.
//
// Inside a wave (lane = 16 * qr + col), per 16-token chunk:
//   Q.K^T  v_mfma_f32_16x16x32_bf16 with the K rows as the A operand (lane
//          holds 8 bf16 of token `col`, d-chunk 4 s + qr in k-step s) and the
//          query group as the B operand (column col = query head col % G,
//          replicated).  Result lane (col, qr), register i = score of head
//          col % G with token 4 qr + i.
//   softmax exp2 on the hardware unit, running max over the chunk(s) of a
//          tile with two cross-row shuffles.
//   P.V    for G >= 2 on the matrix cores (v_mfma_f32_16x16x16_bf16, fp32
//          accumulate): out^T = V^T P, B = P straight from the score registers
//          (lane (col, qr) holds head col % G, tokens 4 qr + i), split into a
//          bf16 high part and a bf16 remainder so that p keeps 16 significant
//          bits, never a single bf16 rounding; A = V^T read column-wise from the
//          V rows in LDS.  For G = 1 (15 of 16 MFMA columns would repeat the
//          head) on the vector ALUs in fp32: lane (col, qr) owns output dims
//          8 col .. 8 col + 7 of its tokens 4 qr + i, whose probabilities it
//          already holds (every column is the one head), and the four row
//          groups' sums are added at the end.
//   loads  every K/V load instruction reads 4 whole 256-byte rows (lane
//          (col, qr): 16 bytes of rows 4 qr + i); K reaches the A-operand
//          layout of Q.K^T through a padded wave-private LDS tile.
// FP8 pools: lane (col, qr) loads the K codes of its A operand straight from
// memory, bytes 16 qr .. 16 qr + 15 and 64 + 16 qr .. 64 + 16 qr + 15 of row
// col (each of the two load instructions reads 64 contiguous bytes of all 16
// rows), and widens them to bf16 in registers: no LDS tile for K.  The four
// k-steps of Q.K^T take dims 64 (s / 2) + 8 (s % 2) + 16 qr .. + 7, and the
// query operand follows that order.  V codes are widened to bf16 and P.V
// runs as above.
#pragma once

#include <type_traits>

#include "decode_common.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kMaxWaves = 8;

// Eight E4M3 codes widened to eight bf16 values, exactly (an E4M3 value has
// at most 4 significant bits); gfx950's conversions decode OCP E4M3.  The
// scaled conversion with scale 1 gives two bf16 per instruction.
__device__ __forceinline__ u32x4_t widen_e4m3(u32x2_t w) {
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    r[2 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.f, false));
    r[2 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], 1.f, true));
  }
  return r;
}

// Query operand of one set of 16 query columns; lane (col, qr) holds column
// col: the B operands of the four 32-deep k-steps of Q.K^T, 8 bf16 each.
// bf16 pools: dims 8 (4 s + qr) .. + 7 in step s (the K rows' order after
// the LDS transpose); FP8 pools: dims 64 (s / 2) + 8 (s % 2) + 16 qr .. + 7
// (the order in which a lane loads its K codes).
template <bool F8>
struct QueryOperand {
  bf16x8_t s[4];
};

// K and V rows of one 16-token tile of one wave: for bf16 pools 16 bytes
// (8 elements) of each of 4 rows per lane; for FP8 pools 8 bytes (the same
// 8 elements) of each V row, the 32 K codes of the lane's operand of the
// Q.K^T (row col), and the K and V scales of the block of rows 4 qr .. 4 qr + 3.
// krow/vrow give the rows as bf16.
template <bool F8 = false>
struct KVTile;

template <>
struct KVTile<false> {
  u32x4_t k[4];
  u32x4_t v[4];
  __device__ __forceinline__ u32x4_t krow(int i) const { return k[i]; }
  __device__ __forceinline__ u32x4_t vrow(int i) const { return v[i]; }
  // An empty asm on every loaded register (see stream_window).
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(k[s]), "+v"(v[s]));
  }
};

template <>
struct KVTile<true> {
  u32x4_t k[2];  // K codes of row col, dims 16 qr + j and 64 + 16 qr + j: the A operand of Q.K^T
  u32x2_t v[4];
  float ks, vs;  // scales of the block of this lane's rows 4 qr .. 4 qr + 3
  __device__ __forceinline__ u32x4_t vrow(int i) const { return widen_e4m3(v[i]); }
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(v[s]));
    asm volatile("" : "+v"(k[0]), "+v"(k[1]), "+v"(ks), "+v"(vs));
  }
};

// bf16 pools: the K rows are loaded like the V rows (each load instruction
// covers 4 whole 256-byte rows) and put into the MFMA operand layout through
// a wave-private LDS tile of 16 rows, each padded to 17 x 16 bytes so that
// both the row writes and the column reads are free of bank conflicts.
constexpr int kKRowPad = 17;  // 16-byte units per LDS row

// The V tile of P.V on the matrix cores is read back with gfx950's
// transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// 4 a + c receives, as element i, the c-th 16-bit value of the 8 bytes
// addressed by lane a + 4 i of the group.  Lane (col, qr) addresses row
// 4 qr + col / 4, dims 16 j + 4 (col % 4) .. + 3, so it receives
// V[4 qr + i][16 j + col], i = 0..3: the A operand of one 16x16x16 product in
// one instruction (instead of four 16-bit reads).  Rows are padded to 18
// 16-byte units, which puts the 8 rows a 32-lane half reads on 8 distinct
// 8-bank groups.
constexpr int kVRowPad = 18;  // 16-byte units per V row

__device__ __forceinline__ bf16x4_t lds_read_tr16(const uint16_t* p) {
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p)));
}

struct TileCtx {
  const uint16_t* kbase;  // K pool + kv head offset + this lane's dims
  const uint16_t* vbase;  // V pool + kv head offset + this lane's dims
  const uint8_t* vbase8;  // FP8 pools: V pool + kv head offset + this lane's dims
  const float* kscale;    // FP8 pools: scales [num_blocks][num_kv_heads] + kv head
  const float* vscale;
  int scale_stride;       // FP8 pools: num_kv_heads
  const uint8_t* kpool;   // K pool + kv head offset, in bytes (wave-uniform)
  const uint8_t* vpool;   // V pool + kv head offset, in bytes (wave-uniform)
  uint32_t row_bytes;     // bytes between consecutive slots
  uint32_t lane_bytes;    // this lane's byte offset inside a row (dims 8 col ..)
  uint32_t row_off[4];    // (4 qr + i) * row_bytes + lane_bytes: this lane's bytes of row i of a chunk
  uint32_t kcol_off;      // FP8 pools: col * row_bytes, the K row of this lane's Q.K^T operand
  uint32_t kq_bytes;      // FP8 pools: 16 * qr, its first byte inside the row (and 64 more)
  const uint8_t* kbase8q; // FP8 pools: K pool + kv head offset + kq_bytes
  u32x4_t* k_lds;         // this wave's K transpose tile (bf16 pools)
  u32x4_t* v_lds;         // this wave's V tile, read column-wise (P.V on the matrix cores)
  int64_t tok_stride;     // elements between consecutive slots
  const int* s_bt;        // physical block ids of the window (LDS)
  int blk0;               // logical block of s_bt[0]
  int end;                // one past the window's last token
  int last_chunk;         // start of the window's last 16-token chunk
  int col, qr;
  volatile int* prog;     // LDS tile counts of the workgroup's waves (issue balancing), or nullptr
  int wave;               // this wave's index in the workgroup
};

// Two waves share each SIMD (waves w and w + 4 of an 8-wave workgroup), and
// the older one wins the issue arbitration: left alone it streams well ahead
// of its partner, waits for it at the next barrier, and the workgroup's loads
// in flight halve meanwhile.  Each wave counts its tiles in LDS and, when it
// is behind its partner, raises its issue priority (and lowers it when ahead).
__device__ __forceinline__ void balance_issue(const TileCtx& c) {
  const int me = c.prog[c.wave] + 1;
  c.prog[c.wave] = me;
  const int other = c.prog[c.wave ^ 4];
  if (me > other) __builtin_amdgcn_s_setprio(0);
  else if (me < other) __builtin_amdgcn_s_setprio(2);
}

// 16 bytes of a K or V row; every K/V byte is read once per call, so the
// loads may carry the streaming (non-temporal) hint.
__device__ __forceinline__ u32x4_t load_kv(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// 8 bytes of an FP8 row, with the streaming hint like load_kv.
__device__ __forceinline__ u32x2_t load_kv8(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

// Issue the loads of the 16-token tile starting at token t0.  Tokens past
// the end of the window re-read its last token, so every address is a valid
// row (the scores of such tokens are masked to -inf), and a tile wholly past
// the end (the prefetch after a window's last tile, never computed) re-reads
// the window's last chunk.  (Skipping those loads behind a wave-uniform
// branch instead makes the compiler wait for all outstanding loads before
// the next tile's, which undoes the prefetch.)  A lane's 4 rows
// (4 qr .. 4 qr + 3, clamped to the window's last token) always lie in one
// block, whose FP8 scales it loads too.
template <int BS, bool F8 = false>
__device__ __forceinline__ void load_tile(KVTile<F8>& r, int t0, const TileCtx& c) {
  const int tce = min(t0, c.last_chunk);
  if constexpr (BS >= 16) {
    // The chunk lies in one block: its first row's address is wave-uniform
    // (scalar registers) and a lane adds only the 32-bit offset of its row,
    // row 4 qr + i clamped to the window's last token (tce is a multiple of
    // 16, so tce + r stays in the block).
    // min(r, lim) * row_bytes = min(r * row_bytes, lim * row_bytes).
    const int phys = __builtin_amdgcn_readfirstlane(c.s_bt[tce / BS - c.blk0]);
    const int tcu = __builtin_amdgcn_readfirstlane(tce);
    const int lim = __builtin_amdgcn_readfirstlane(c.end - 1 - tcu);  // >= 0: tce <= last_chunk
    const int64_t first = ((int64_t)phys * BS + (tcu & (BS - 1))) * c.row_bytes;
    const uint8_t* kb = c.kpool + first;
    const uint8_t* vb = c.vpool + first;
    const uint32_t lim_off = (uint32_t)lim * c.row_bytes + c.lane_bytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = min(c.row_off[i], lim_off);
      if constexpr (F8) {
        r.v[i] = load_kv8(vb + off);
      } else {
        r.k[i] = load_kv(reinterpret_cast<const uint16_t*>(kb + off));
        r.v[i] = load_kv(reinterpret_cast<const uint16_t*>(vb + off));
      }
    }
    if constexpr (F8) {
      // K row col (clamped like the others), 32 codes in two 16-byte loads.
      const uint32_t koff = min(c.kcol_off, (uint32_t)lim * c.row_bytes) + c.kq_bytes;
      r.k[0] = load_kv(reinterpret_cast<const uint16_t*>(kb + koff));
      r.k[1] = load_kv(reinterpret_cast<const uint16_t*>(kb + koff + 64));
      const int64_t si = (int64_t)phys * c.scale_stride;
      r.ks = c.kscale[si];
      r.vs = c.vscale[si];
    }
  } else {
    // 8-token blocks: a chunk spans two blocks, each row finds its own.
    int pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // row 4 qr + i, dims 8 col .. 8 col + 7
      const int tv = min(tce + 4 * c.qr + i, c.end - 1);
      pv[i] = c.s_bt[tv / BS - c.blk0];
      const int64_t row = ((int64_t)pv[i] * BS + (tv & (BS - 1))) * c.tok_stride;
      if constexpr (F8) {
        r.v[i] = load_kv8(c.vbase8 + row);
      } else {
        r.k[i] = load_kv(c.kbase + row);
        r.v[i] = load_kv(c.vbase + row);
      }
    }
    if constexpr (F8) {
      // K row col of the chunk (the Q.K^T operand), in its own block.
      const int tk = min(tce + c.col, c.end - 1);
      const int pk = c.s_bt[tk / BS - c.blk0];
      const uint16_t* kp = reinterpret_cast<const uint16_t*>(
          c.kbase8q + ((int64_t)pk * BS + (tk & (BS - 1))) * c.tok_stride);
      r.k[0] = load_kv(kp);
      r.k[1] = load_kv(kp + 32);
      const int64_t si = (int64_t)pv[0] * c.scale_stride;
      r.ks = c.kscale[si];
      r.vs = c.vscale[si];
    }
  }
}

// P.V runs on the matrix cores for query groups of at least 2 heads (p as
// bf16 hi + lo); a single head would use one MFMA column in 16, so it stays
// on the vector ALUs.
template <int G>
constexpr bool kPvOnMfma = G >= 2;

// Running softmax state of a wave whose P.V runs on the matrix cores, for NS
// sets of 16 query columns; lane (col, qr) keeps column col of every set.
template <int NS>
struct MfmaState {
  float m[NS], l[NS];  // max and (this lane's tokens') sum of column col
  f32x4_t o[NS][8];    // set n, tile j, register i: column col, dim 16 j + 4 qr + i
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      m[n] = -INFINITY;
      l[n] = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) o[n][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Running softmax state of a wave whose P.V runs on the vector ALUs (a
// single query head: every column holds it).
struct ValuState {
  float m[1], l[1];  // max and this lane's tokens' sum
  float acc[8];      // dims 8 col .. 8 col + 7, this lane's token rows
  __device__ __forceinline__ void reset() {
    m[0] = -INFINITY;
    l[0] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  }
};

// State of a wave over the G heads of its kv head (column col = head col % G).
template <int G>
using WaveState = std::conditional_t<kPvOnMfma<G>, MfmaState<1>, ValuState>;

// Which tokens of a window a query column attends to.  WindowTokens: all of
// them (decode).  CausalTokens: column set n of this lane stops below
// limit[n] (prefill: a token sees the tokens up to its own position).
// whole(tok0, end): every column attends to all 16 tokens from tok0 (a
// wave-uniform test that lets the per-token test be skipped).
struct WindowTokens {
  __device__ __forceinline__ bool valid(int, int tok, int end) const { return tok < end; }
  __device__ __forceinline__ bool whole(int tok0, int end) const { return tok0 + 16 <= end; }
};
template <int NS>
struct CausalTokens {
  int limit[NS];
  __device__ __forceinline__ bool valid(int n, int tok, int end) const {
    return tok < end && tok < limit[n];
  }
  __device__ __forceinline__ bool whole(int, int) const { return false; }
};

// Scores of one chunk (tokens tok0 .. tok0 + 15) from the raw products
// sacc of NS sets of query columns times sl[n]; tokens a column does not
// attend to score -inf.  mt[n] takes the maximum of set n over this lane's
// rows (lane (col, qr), register i: token 4 qr + i).
template <int NS, class Lim>
__device__ __forceinline__ void scores_of_chunk(const f32x4_t (&sacc)[NS], const float (&sl)[NS],
                                                int tok0, int end, int qr, float (&x)[NS][1][4],
                                                float (&mt)[NS], const Lim& lim) {
#pragma unroll
  for (int n = 0; n < NS; ++n) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[n][0][i] = sacc[n][i] * sl[n];
    if (!lim.whole(tok0, end)) {  // only a window's last chunk holds tokens past its end
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!lim.valid(n, tok0 + 4 * qr + i, end)) x[n][0][i] = -INFINITY;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) mt[n] = fmaxf(mt[n], x[n][0][i]);
  }
}

// Maximum of x over lanes l and l ^ 16, then l ^ 32: the four row groups of
// a column.  The gfx950 lane swaps exchange 16-lane rows (row 2k + 1 of the
// first operand with row 2k of the second) and 32-lane halves without going
// through LDS; the maximum of the two results is symmetric in the pair.
__device__ __forceinline__ float rowgroup_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Column maxima over the four row groups of a wave.
template <int NS>
__device__ __forceinline__ void column_max(float (&mt)[NS]) {
#pragma unroll
  for (int n = 0; n < NS; ++n) mt[n] = rowgroup_max(mt[n]);
}

// Q.K^T of one loaded tile for NS sets of query columns, scaled by
// scale * log2(e); tokens the columns do not attend to (at or past `end`, or
// past a column's limit) score -inf.  mt[n] is the tile's maximum of set n
// over each column (all four row groups).
template <int NS, bool F8, class Lim = WindowTokens>
__device__ __forceinline__ void tile_scores(const KVTile<F8>& r, int t0, int end,
                                            const QueryOperand<F8> (&qop)[NS], float scale_log2e,
                                            const TileCtx& ctx, float (&x)[NS][1][4],
                                            float (&mt)[NS], const Lim& lim = Lim{}) {
  const int qr = ctx.qr;
  f32x4_t sacc[NS];
  float sl[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    mt[n] = -INFINITY;
    sacc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if constexpr (F8) {
    // A = the K codes as loaded, widened (exactly) to bf16: k-step s takes
    // codes 8 s .. 8 s + 7 of this lane.  Dequantised K = scale * code value.
    u32x4_t kop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      kop[s] = widen_e4m3(u32x2_t{r.k[s >> 1][2 * (s & 1)], r.k[s >> 1][2 * (s & 1) + 1]});
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[s]),
                                                          qop[n].s[s], sacc[n], 0, 0, 0);
      sl[n] = scale_log2e * r.ks;
    }
  } else {
    // rows as loaded -> LDS -> lane (col, qr) takes d-chunk 4 s + qr of row col
    u32x4_t kop[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ctx.k_lds[(4 * qr + i) * kKRowPad + ctx.col] = r.krow(i);
#pragma unroll
    for (int s = 0; s < 4; ++s) kop[s] = ctx.k_lds[ctx.col * kKRowPad + 4 * s + qr];
#pragma unroll
    for (int n = 0; n < NS; ++n) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[s]),
                                                          qop[n].s[s], sacc[n], 0, 0, 0);
      sl[n] = scale_log2e;
    }
  }
  scores_of_chunk<NS>(sacc, sl, t0, end, qr, x, mt, lim);
  column_max<NS>(mt);
}

// Online-softmax step of one column: the running max takes the tile's max,
// the scores become exp2(x - max) and the sum is rescaled and extended.
// Returns the factor that rescales the state accumulated so far.
template <int TC>
__device__ __forceinline__ float softmax_update(float (&x)[TC][4], float mt, float& m, float& l) {
  const float m_new = fmaxf(m, mt);  // finite: the tile holds a valid token
  const float alpha = exp2_hw(m - m_new);
  m = m_new;
  float psum = 0.f;
#pragma unroll
  for (int c = 0; c < TC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[c][i] = exp2_hw(x[c][i] - m_new);
      psum += x[c][i];
    }
  l = l * alpha + psum;
  return alpha;
}

// Rescales the P.V accumulators by alpha, only when some column's running
// max moved (alpha == 1 exactly otherwise, so skipping changes no bit); past
// the first few hundred tokens most tiles skip it.
template <int NS>
__device__ __forceinline__ void rescale_lazy(const float (&alpha)[NS], MfmaState<NS>& st) {
  bool moved = false;
#pragma unroll
  for (int n = 0; n < NS; ++n) moved |= alpha[n] != 1.f;
  if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int j = 0; j < 8; ++j) st.o[n][j] *= alpha[n];
  }
}

// out^T[d][col] += sum_t V[t][d] P[t][col] for chunk c with
// v_mfma_f32_16x16x16_bf16, 16 dims per product.  B = P: lane (col, qr)
// already holds P[4 qr + i][col].  p is split into bf16 hi + lo (the top 8
// and the next 8 mantissa bits), two products each, so p keeps 16 bits.
// A = V^T from the chunk's 16 V rows in LDS (`vcol`, rows kVRowPad units
// apart): lane (col, qr) takes V[4 qr + i][16 j + col]; every column set uses
// the same A operand.
template <int TC, int NS>
__device__ __forceinline__ void pv_from_lds(const uint16_t* vcol, int c,
                                            const float (&x)[NS][TC][4], int col, int qr,
                                            MfmaState<NS>& st) {
  bf16x4_t phi[NS], plo[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    uint32_t hb[4], lb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      hb[i] = __float_as_uint(x[n][c][i]) & 0xFFFF0000u;
      lb[i] = __float_as_uint(x[n][c][i] - __uint_as_float(hb[i]));
    }
    const uint32_t hi[2] = {__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                            __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)};
    const uint32_t lo[2] = {__builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                            __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u)};
    phi[n] = __builtin_bit_cast(bf16x4_t, hi);
    plo[n] = __builtin_bit_cast(bf16x4_t, lo);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const bf16x4_t vt =
        lds_read_tr16(vcol + (4 * qr + col / 4) * (kVRowPad * 8) + 16 * j + 4 * (col % 4));
#pragma unroll
    for (int n = 0; n < NS; ++n) {
      st.o[n][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi[n], st.o[n][j], 0, 0, 0);
      st.o[n][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo[n], st.o[n][j], 0, 0, 0);
    }
  }
}

// pv_from_lds for two chunks c0, c1 at once with v_mfma_f32_16x16x32_bf16
// (twice the rate of the 16-deep product): lane (col, qr)'s eight k-slots are
// its four tokens of chunk c0 (4 qr + i) followed by its four of chunk c1, in
// both operands, so the sum over k is unchanged.  The A operand joins two
// transposing reads, one per chunk (`vcol0`, `vcol1`).
template <int TC, int NS>
__device__ __forceinline__ void pv_pair_from_lds(const uint16_t* vcol0, const uint16_t* vcol1,
                                                 int c0, int c1, const float (&x)[NS][TC][4],
                                                 int col, int qr, MfmaState<NS>& st) {
  bf16x8_t phi[NS], plo[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = i < 4 ? x[n][c0][i] : x[n][c1][i - 4];
      hb[i] = __float_as_uint(v) & 0xFFFF0000u;
      lb[i] = __float_as_uint(v - __uint_as_float(hb[i]));
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      hi[k] = __builtin_amdgcn_perm(hb[2 * k + 1], hb[2 * k], 0x07060302u);
      lo[k] = __builtin_amdgcn_perm(lb[2 * k + 1], lb[2 * k], 0x07060302u);
    }
    phi[n] = __builtin_bit_cast(bf16x8_t, hi);
    plo[n] = __builtin_bit_cast(bf16x8_t, lo);
  }
  const int off = (4 * qr + col / 4) * (kVRowPad * 8) + 4 * (col % 4);
  auto read_v = [&](int j) {
    const bf16x4_t va = lds_read_tr16(vcol0 + off + 16 * j);
    const bf16x4_t vb = lds_read_tr16(vcol1 + off + 16 * j);
    return __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // The high parts of 16-dim block j go in with the low parts of block
  // j - 1, so that the two products on one accumulator are 2 NS products
  // apart; the operand of block j + 1 is read meanwhile.
  bf16x8_t vt[3];  // blocks j - 1, j, j + 1
  vt[0] = read_v(0);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j + 1 < 8) vt[(j + 1) % 3] = read_v(j + 1);
#pragma unroll
    for (int n = 0; n < NS; ++n)
      st.o[n][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[j % 3], phi[n], st.o[n][j], 0, 0, 0);
    if (j > 0) {
#pragma unroll
      for (int n = 0; n < NS; ++n)
        st.o[n][j - 1] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[(j - 1) % 3], plo[n], st.o[n][j - 1], 0, 0, 0);
    }
  }
#pragma unroll
  for (int n = 0; n < NS; ++n)
    st.o[n][7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt[7 % 3], plo[n], st.o[n][7], 0, 0, 0);
}

// Scores, online-softmax update and P.V accumulation for one loaded tile,
// P.V on the matrix cores.
template <int NS, bool F8, class Lim = WindowTokens>
__device__ __forceinline__ void compute_tile(const KVTile<F8>& r, int t0, int end,
                                             const QueryOperand<F8> (&qop)[NS], float scale_log2e,
                                             const TileCtx& ctx, MfmaState<NS>& st,
                                             const Lim& lim = Lim{}) {
  const int qr = ctx.qr;
  float x[NS][1][4], mt[NS], alpha[NS];
  tile_scores<NS>(r, t0, end, qop, scale_log2e, ctx, x, mt, lim);
#pragma unroll
  for (int n = 0; n < NS; ++n) alpha[n] = softmax_update<1>(x[n], mt[n], st.m[n], st.l[n]);
  if constexpr (F8) {  // dequantised V = scale * code value: scale the probabilities (not l)
#pragma unroll
    for (int n = 0; n < NS; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[n][0][i] *= r.vs;
  }
  rescale_lazy<NS>(alpha, st);
#pragma unroll
  for (int i = 0; i < 4; ++i) ctx.v_lds[(4 * qr + i) * kVRowPad + ctx.col] = r.vrow(i);
  pv_from_lds<1, NS>(reinterpret_cast<const uint16_t*>(ctx.v_lds), 0, x, ctx.col, qr, st);
}

// The same with P.V on the vector ALUs in fp32 (one query head).
template <bool F8>
__device__ __forceinline__ void compute_tile(const KVTile<F8>& r, int t0, int end,
                                             const QueryOperand<F8> (&qop)[1], float scale_log2e,
                                             const TileCtx& ctx, ValuState& st,
                                             const WindowTokens& = WindowTokens{}) {
  float x[1][1][4], mt[1];
  tile_scores<1>(r, t0, end, qop, scale_log2e, ctx, x, mt);
  const float alpha = softmax_update<1>(x[0], mt[0], st.m[0], st.l[0]);
  if constexpr (F8) {  // dequantised V = scale * code value: scale the probabilities (not l)
#pragma unroll
    for (int i = 0; i < 4; ++i) x[0][0][i] *= r.vs;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) st.acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float vf[8];
    unpack_bf16x8(r.vrow(i), vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[e] = fmaf(x[0][0][i], vf[e], st.acc[e]);
  }
}

// B operand of one set of query columns: this lane's column reads the
// 128-element query row `qrow`.
__device__ __forceinline__ void load_qop(const uint16_t* qrow, int qr, bf16x8_t (&qop)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qop[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * qr));
}

__device__ __forceinline__ void load_qop(const uint16_t* qrow, int qr, QueryOperand<false>& op) {
  load_qop(qrow, qr, op.s);
}

// The FP8 pools' order: k-step s reads dims 64 (s / 2) + 8 (s % 2) + 16 qr .. + 7.
__device__ __forceinline__ void load_qop(const uint16_t* qrow, int qr, QueryOperand<true>& op) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    op.s[s] = __builtin_bit_cast(
        bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 64 * (s >> 1) + 8 * (s & 1) + 16 * qr));
}

// Query operand of the group of kv head kvh, sequence b (column col = head col % G).
template <int G, bool F8>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int kvh, int col, int qr,
                                           QueryOperand<F8> (&qop)[1]) {
  load_qop(static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + kvh * G + col % G) * kD,
           qr, qop[0]);
}

// Streams tokens [begin, end) of one window through this wave's state, tile
// by tile.  Two register buffers alternate (the loop is unrolled by two), so
// that the loads of the next tile are issued before the current tile is
// computed and stay in flight during the whole compute: with a single
// loop-carried buffer the back edge copies the just-loaded registers, which
// makes the wave wait for those loads at the end of every iteration.  The
// scheduling barriers keep the loads ahead of the compute.  Past the window's
// end the loads re-read its last chunk and are never used.
template <int BS, bool F8, int NS, class State, class Lim = WindowTokens>
__device__ __forceinline__ void stream_window(const DecodeArgs& a, const TileCtx& c, int begin,
                                              const QueryOperand<F8> (&qop)[NS], State& st,
                                              const Lim& lim = Lim{}) {
  constexpr int TILE = 16;
  int t0 = begin;
  KVTile<F8> ta, tb;
  load_tile<BS>(ta, t0, c);
  // The first tile passes through an empty asm so that ta is not a load on
  // both incoming edges of the loop: otherwise the optimiser merges the two
  // loads of ta into one at the loop top, which undoes the prefetch.
  ta.pin();
  // Pairs of tiles with a single exit: with an exit after each half the
  // compiler joins both exits in one block with an edge back to the loop
  // head, and must then wait for every load at the head.
  const int n = (c.end - begin + TILE - 1) / TILE;  // tiles of the window (uniform)
  for (int i = 0; i + 1 < n; i += 2) {
    load_tile<BS>(tb, t0 + TILE, c);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(ta, t0, c.end, qop, a.scale_log2e, c, st, lim);
    load_tile<BS>(ta, t0 + 2 * TILE, c);
    __builtin_amdgcn_sched_barrier(0);
    compute_tile(tb, t0 + TILE, c.end, qop, a.scale_log2e, c, st, lim);
    t0 += 2 * TILE;
    if (c.prog != nullptr) balance_issue(c);
  }
  if (n & 1) compute_tile(ta, t0, c.end, qop, a.scale_log2e, c, st, lim);
  // Wait here for the prefetch past the end (vmcnt 0; expcnt and lgkmcnt
  // left free).  Otherwise it is still in flight when the caller streams its
  // next window, whose loop head is the same code, and the compiler puts a
  // full wait at that head, in front of every other tile's loads.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Sequences whose block tables must agree with the streamed table over every
// window (the members of a shared prefix); each disagreement is flagged in the
// error word.  Entries of `seqs` outside [0, num_seqs) are skipped.
struct TableCheck {
  const int32_t* seqs;
  int count;
};

// Streams tokens [begin, end) (begin a multiple of 16) through the block-table
// row `bt` into the state of each wave, wave w for kv head kvh0 + w.  The
// block ids of a window of up to kMaxPartitionTokens tokens go to LDS once for
// all waves.  Every thread of the workgroup calls this with the same range.
template <int BS, bool kCheck, bool F8 = false, int NS, class State, class Lim = WindowTokens>
__device__ __forceinline__ void attend_table(const DecodeArgs& a, int* s_bt, u32x4_t* k_lds,
                                             u32x4_t* v_lds, const int32_t* bt, int kvh,
                                             int begin, int end,
                                             const QueryOperand<F8> (&qop)[NS], State& st,
                                             TableCheck chk = TableCheck{nullptr, 0},
                                             const Lim& lim = Lim{}, int* prog = nullptr) {
  const int lane = threadIdx.x & 63;
  TileCtx c;
  c.prog = prog;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  c.tok_stride = (int64_t)a.num_kv_heads * kD;
  c.col = lane & 15;
  c.qr = lane >> 4;
  c.kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * kD + 8 * c.col;
  c.k_lds = k_lds;
  c.vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * kD + 8 * c.col;
  c.v_lds = v_lds;
  c.s_bt = s_bt;
  {
    constexpr int es = F8 ? 1 : 2;  // bytes per stored element
    c.kpool = static_cast<const uint8_t*>(a.k_cache) + (int64_t)kvh * kD * es;
    c.vpool = static_cast<const uint8_t*>(a.v_cache) + (int64_t)kvh * kD * es;
    c.row_bytes = (uint32_t)(c.tok_stride * es);
    c.lane_bytes = (uint32_t)(8 * c.col * es);
#pragma unroll
    for (int i = 0; i < 4; ++i) c.row_off[i] = (uint32_t)(4 * c.qr + i) * c.row_bytes + c.lane_bytes;
  }
  if constexpr (F8) {
    c.kcol_off = (uint32_t)c.col * c.row_bytes;
    c.kq_bytes = 16u * c.qr;
    c.kbase8q = static_cast<const uint8_t*>(a.k_cache) + (int64_t)kvh * kD + c.kq_bytes;
    c.vbase8 = static_cast<const uint8_t*>(a.v_cache) + (int64_t)kvh * kD + 8 * c.col;
    c.kscale = a.k_scale + kvh;
    c.vscale = a.v_scale + kvh;
    c.scale_stride = a.num_kv_heads;
  }
  for (int w0 = begin; w0 < end; w0 += kMaxPartitionTokens) {
    const int wend = min(end, w0 + kMaxPartitionTokens);
    const int blk0 = w0 / BS;
    const int nblk = (wend - 1) / BS - blk0 + 1;  // <= kMaxPartitionTokens / BS + 1
    __syncthreads();  // every wave is done with the previous window's ids
    for (int i = threadIdx.x; i < nblk; i += blockDim.x)
      s_bt[i] = checked_block(bt, blk0 + i, a.num_blocks, a.err);
    if constexpr (kCheck) {
      const int n = chk.count * nblk;
      for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int m = i / nblk, j = i - m * nblk;
        const int seq = chk.seqs[m];
        if (static_cast<unsigned>(seq) < static_cast<unsigned>(a.num_seqs) &&
            a.block_tables[(int64_t)seq * a.max_blocks_per_seq + blk0 + j] != bt[blk0 + j])
          atomicOr(a.err, kErrShared);
      }
    }
    __syncthreads();
    c.blk0 = blk0;
    c.end = wend;
    c.last_chunk = ((wend - 1) >> 4) << 4;
    stream_window<BS, F8>(a, c, w0, qop, st, lim);
  }
}

// attend_table over sequence b's own block table and queries.
template <int G, int BS, bool F8 = false>
__device__ __forceinline__ void attend_range(const DecodeArgs& a, int* s_bt, u32x4_t* k_lds,
                                             u32x4_t* v_lds, int b, int kvh, int begin, int end,
                                             const QueryOperand<F8> (&qop)[1], WaveState<G>& st,
                                             int* prog = nullptr) {
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  attend_table<BS, false, F8>(a, s_bt, k_lds, v_lds, bt, kvh, begin, end, qop, st,
                              TableCheck{nullptr, 0}, WindowTokens{}, prog);
}

// Slices of a work stream of `total` units, in pairs: slice 2k takes `even`
// units of each pair's q, slice 2k + 1 the rest.  Workgroups are dealt
// round-robin over the eight XCDs, so with one kv-head group per grid row
// slice 2k runs on an even XCD and slice 2k + 1 on an odd one.  Timestamps of
// the bf16 decode (a least-squares fit of each workgroup's time over its
// chunks and pieces) leave a residual set by XCD parity alone: under a
// full-bandwidth load the odd XCDs finish 17-24 us after the even ones over
// about 250 us.  bf16 pools therefore give the even slice of a pair 51.5% of
// its units; FP8 pools, which showed no such split, give both halves.  With an
// even number of kv-head groups per row a slice's XCD parity is that of its
// group, and with fewer than kXcdSplitMin units per slice (a small,
// cache-resident call, where the share's rounding would outweigh it) the
// slices stay equal.
template <bool F8>
constexpr int kXcdEvenPermille = F8 ? 500 : 515;
constexpr int kXcdSplitMin = 48;

struct SliceSplit {
  int q;     // units per pair of slices
  int even;  // units of its even slice
  template <bool F8>
  __device__ static SliceSplit make(int total, int slices, int groups) {
    if (slices >= 2 && (groups & 1) && total >= kXcdSplitMin * slices) {
      const int q = max(2, (total + slices / 2 - 1) / (slices / 2));
      const int even = min(q - 1, max(1, (q * kXcdEvenPermille<F8> + 500) / 1000));
      return {q, even};
    }
    const int per = max(1, (total + slices - 1) / slices);
    return {2 * per, per};
  }
  __device__ int begin(int s) const { return (s >> 1) * q + ((s & 1) ? even : 0); }
  __device__ int end(int s) const { return (s >> 1) * q + ((s & 1) ? q : even); }
  __device__ int slice_of(int c) const {  // slice of unit c
    const int p = c / q;
    return 2 * p + (c - p * q >= even ? 1 : 0);
  }
};

// Where a wave's finished range goes.
struct Sink {
  float* acc;      // unnormalised output rows (D floats each), or nullptr: final output
  float* max;
  float* sum;
  int64_t row0;    // row of head 0 of the kv head's group
  int64_t stride;  // rows between consecutive heads
};

// Completes the wave's sums over its token rows, then writes either the
// normalised output rows of the G heads (sink.acc == nullptr) or their
// partial results.
template <int G>
__device__ __forceinline__ void finish_wave(const DecodeArgs& a, WaveState<G>& st, int b, int kvh,
                                            const Sink& sink) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
  if constexpr (kPvOnMfma<G>) {
    // The matrix cores already summed over the tokens; only l needs the rows.
    st.l[0] += __shfl_xor(st.l[0], 16);
    st.l[0] += __shfl_xor(st.l[0], 32);
    if (col >= G) return;  // columns >= G repeat heads 0 .. G-1
    const int h = col;
    if (sink.acc == nullptr) {
      const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G + h) * kD + 4 * qr;
      const float inv = 1.f / st.l[0];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(a, o + 16 * j + i, st.o[0][j][i] * inv);
    } else {
      const int64_t row = sink.row0 + h * sink.stride;
      float* dst = sink.acc + row * kD + 4 * qr;
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = st.o[0][j];
      if (qr == 0) {
        sink.max[row] = st.m[0];
        sink.sum[row] = st.l[0];
      }
    }
  } else {
    // One query head (G = 1): add the four row groups' sums of the lane's
    // dims; lanes of row group 0 write dims 8 col .. 8 col + 7.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      st.acc[e] += __shfl_xor(st.acc[e], 16);
      st.acc[e] += __shfl_xor(st.acc[e], 32);
    }
    st.l[0] += __shfl_xor(st.l[0], 16);
    st.l[0] += __shfl_xor(st.l[0], 32);
    if (qr != 0) return;
    const int h = kvh * G;
    if (sink.acc == nullptr) {
      const int64_t o = ((int64_t)b * a.num_q_heads + h) * kD + 8 * col;
      const float inv = 1.f / st.l[0];
#pragma unroll
      for (int e = 0; e < 8; ++e) store_out(a, o + e, st.acc[e] * inv);
    } else {
      const int64_t row = sink.row0;
      float* dst = sink.acc + row * kD + 8 * col;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = st.acc[e];
      if (col == 0) {
        sink.max[row] = st.m[0];
        sink.sum[row] = st.l[0];
      }
    }
  }
}

// Zero output rows of the G heads of kv head kvh, sequence b (one wave).
template <int G>
__device__ __forceinline__ void zero_rows(const DecodeArgs& a, int b, int kvh) {
  const int lane = threadIdx.x & 63;
  const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G) * kD;
  for (int i = lane; i < G * kD; i += 64) store_out(a, o + i, 0.f);
}

// Zero output rows (kv head kvh, one wave) of every sequence b < B for which
// empty(b) holds.  The wave tests 64 sequences at a time and walks the ballot,
// so the cost grows with the number of empty sequences, not with B.
template <int G, class F>
__device__ __forceinline__ void zero_rows_where(const DecodeArgs& a, int B, int kvh, F&& empty) {
  const int lane = threadIdx.x & 63;
  for (int base = 0; base < B; base += 64) {
    const int j = base + lane;
    unsigned long long m = __ballot(j < B && empty(j));
    while (m) {
      const int k = __builtin_ctzll(m);
      m &= m - 1;
      zero_rows<G>(a, base + k, kvh);
    }
  }
}

// Exclusive prefix sums out[i] = count(0) + ... + count(i - 1) for i <= n of a
// count that every thread can evaluate; returns out[n].  All threads of the
// workgroup call it; it ends with a barrier.
template <class F>
__device__ __forceinline__ int block_scan(int n, int* out, int* s_wsum, F&& count) {
  const int nw = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int j = base + threadIdx.x;
    const int cnt = j < n ? count(j) : 0;
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
    if (j < n) out[j] = before + x - cnt;
    carry += total;
    __syncthreads();  // s_wsum is rewritten by the next round
  }
  if (threadIdx.x == 0) out[n] = carry;
  __syncthreads();
  return carry;
}

// Largest i in [0, n) with arr[i] <= v, for a nondecreasing arr with arr[0] <= v.
__device__ __forceinline__ int last_at_most(const int* arr, int n, int v) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (arr[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace
}  // namespace pkv
