// Decode-step attention, bf16 pools with head_dim 128, on the matrix cores
// of gfx950 (MI355X).
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
//          head) on the vector ALUs in fp32: lane owns output dims
//          8 col .. 8 col + 7 and tokens 4 qr + i; accumulator slot R holds query
//          head gsel[R], the head of the lane that DPP row rotation R reaches,
//          so that head's probabilities and rescale factors arrive by the same
//          rotation.
//   loads  every K/V load instruction reads 4 whole 256-byte rows (lane
//          (col, qr): 16 bytes of rows 4 qr + i); K reaches the A-operand
//          layout of Q.K^T through a padded wave-private LDS tile.
//
// Two schedules:
//  * decode_mfma_kernel, partition grid: workgroup (kv-head group, sequence,
//    partition of part_tokens tokens), highest partition dispatched first;
//    splitk_reduce_kernel merges the partitions of a sequence.
//  * decode_balanced_kernel: the sequences' 16-token chunks are laid end to
//    end and every workgroup takes an equal slice of that stream (see the
//    kernel), so the work per workgroup does not depend on the length mix;
//    balanced_reduce_kernel merges the sequences that slices cut.
#include "decode_common.h"

namespace pkv {
namespace {

constexpr int kD = 128;
constexpr int kMaxWaves = 8;

#if PKV_BALANCED_WAVES_PER_EU > 0
#define PKV_BALANCED_OCCUPANCY \
  __attribute__((amdgpu_waves_per_eu(PKV_BALANCED_WAVES_PER_EU, PKV_BALANCED_WAVES_PER_EU)))
#else
#define PKV_BALANCED_OCCUPANCY
#endif

// K and V rows of one tile (TC chunks of 16 tokens) of one wave.
template <int TC>
struct KVTile {
  u32x4_t k[TC][4];
  u32x4_t v[TC][4];
};

// With PKV_K_VIA_LDS the K rows are loaded like the V rows (each load
// instruction covers 4 whole 256-byte rows instead of 64 bytes of 16 rows)
// and put into the MFMA operand layout through a wave-private LDS tile of
// 16 rows, each padded to 17 x 16 bytes so that both the row writes and the
// column reads are free of bank conflicts.
constexpr int kKRowPad = 17;  // 16-byte units per LDS row

struct TileCtx {
  const uint16_t* kbase;  // K pool + kv head offset + this lane's d-chunk (or dims)
  const uint16_t* vbase;  // V pool + kv head offset + this lane's dims
  const uint16_t* kdead;  // this wave's query row + this lane's offset (see load_tile)
  const uint16_t* vdead;  // this wave's query row + this lane's dims
  u32x4_t* k_lds;         // this wave's K transpose tile (PKV_K_VIA_LDS)
  u32x4_t* v_lds;         // this wave's V tile, read column-wise (P.V on the matrix cores)
  int64_t tok_stride;     // elements between consecutive slots
  const int* s_bt;        // physical block ids of the window (LDS)
  int blk0;               // logical block of s_bt[0]
  int end;                // one past the window's last token
  int last_chunk;         // start of the window's last 16-token chunk
  int col, qr;
};

// 16 bytes of a K or V row; every K/V byte is read once per call, so the
// loads may carry the streaming (non-temporal) hint.
__device__ __forceinline__ u32x4_t load_kv(const uint16_t* p) {
#if PKV_KV_NONTEMPORAL
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
#else
  return *reinterpret_cast<const u32x4_t*>(p);
#endif
}

// Issue the loads of the tile starting at token t0.  Tokens past the end of
// the window re-read its last token, so every address is a valid row (the
// scores of such tokens are masked to -inf).  A chunk wholly past the end
// (the prefetch after a window's last tile, never computed) reads this
// wave's 256-byte query row instead, which is in cache, so it costs no HBM
// traffic.
template <int BS, int TC>
__device__ __forceinline__ void load_tile(KVTile<TC>& r, int t0, const TileCtx& c) {
#pragma unroll
  for (int ch = 0; ch < TC; ++ch) {
    const bool dead = t0 + 16 * ch > c.last_chunk;
    const int tce = min(t0 + 16 * ch, c.last_chunk);
    const int tk = min(tce + c.col, c.end - 1);
    int pk, pv[4];
    if constexpr (BS >= 16) {
      const int phys = __builtin_amdgcn_readfirstlane(c.s_bt[tce / BS - c.blk0]);
      pk = phys;
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = phys;
    } else {
      pk = c.s_bt[tk / BS - c.blk0];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = c.s_bt[min(tce + 4 * c.qr + i, c.end - 1) / BS - c.blk0];
    }
#if PKV_K_VIA_LDS
    (void)pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // row 4 qr + i, dims 8 col .. 8 col + 7
      const int tv = min(tce + 4 * c.qr + i, c.end - 1);
      const int64_t row = ((int64_t)pv[i] * BS + (tv & (BS - 1))) * c.tok_stride;
      r.k[ch][i] = load_kv(dead ? c.kdead : c.kbase + row);
      r.v[ch][i] = load_kv(dead ? c.vdead : c.vbase + row);
    }
#else
    const uint16_t* kp =
        dead ? c.kdead : c.kbase + ((int64_t)pk * BS + (tk & (BS - 1))) * c.tok_stride;
#pragma unroll
    for (int s = 0; s < 4; ++s) r.k[ch][s] = load_kv(kp + 32 * s);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tv = min(tce + 4 * c.qr + i, c.end - 1);
      const uint16_t* vp =
          dead ? c.vdead : c.vbase + ((int64_t)pv[i] * BS + (tv & (BS - 1))) * c.tok_stride;
      r.v[ch][i] = load_kv(vp);
    }
#endif
  }
}

// P.V runs on the matrix cores for query groups of at least
// PKV_PV_MFMA_MIN_GROUP heads; a single head would use one MFMA column in 16,
// so it stays on the vector ALUs.
template <int G>
constexpr bool kPvOnMfma = G >= PKV_PV_MFMA_MIN_GROUP;

// Running softmax state of one wave for the G heads of its kv head.
template <int G, bool kMfma = kPvOnMfma<G>>
struct WaveState;

template <int G>
struct WaveState<G, true> {
  float m, l;   // max and (this lane's tokens') sum of head col % G
  f32x4_t o[8]; // tile j, register i: output of head col % G, dim 16 j + 4 qr + i
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
};

template <int G>
struct WaveState<G, false> {
  float m, l;        // max and sum of head col % G (copies in every column with that head)
  float acc[G][8];   // slot R: head gsel[R], dims 8 col .. 8 col + 7, this lane's token rows
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  }
};

// Scores, online-softmax update and P.V accumulation for one loaded tile.
template <int G, int TC>
__device__ __forceinline__ void compute_tile(const KVTile<TC>& r, int t0, int end,
                                             const bf16x8_t (&qop)[4], float scale_log2e,
                                             const TileCtx& ctx, WaveState<G>& st) {
  const int qr = ctx.qr;
  float x[TC][4];
  float mt = -INFINITY;
#pragma unroll
  for (int c = 0; c < TC; ++c) {
    u32x4_t kop[4];
#if PKV_K_VIA_LDS
    // rows as loaded -> LDS -> lane (col, qr) takes d-chunk 4 s + qr of row col
#pragma unroll
    for (int i = 0; i < 4; ++i) ctx.k_lds[(4 * qr + i) * kKRowPad + ctx.col] = r.k[c][i];
#pragma unroll
    for (int s = 0; s < 4; ++s) kop[s] = ctx.k_lds[ctx.col * kKRowPad + 4 * s + qr];
#else
#pragma unroll
    for (int s = 0; s < 4; ++s) kop[s] = r.k[c][s];
#endif
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kop[s]),
                                                      qop[s], sacc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = t0 + 16 * c + 4 * qr + i;
      x[c][i] = tok < end ? sacc[i] * scale_log2e : -INFINITY;
      mt = fmaxf(mt, x[c][i]);
    }
  }
  mt = fmaxf(mt, __shfl_xor(mt, 16));
  mt = fmaxf(mt, __shfl_xor(mt, 32));
  const float m_new = fmaxf(st.m, mt);  // finite: the tile holds a valid token
  const float alpha = exp2_hw(st.m - m_new);
  st.m = m_new;
  float psum = 0.f;
#pragma unroll
  for (int c = 0; c < TC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[c][i] = exp2_hw(x[c][i] - m_new);
      psum += x[c][i];
    }
  st.l = st.l * alpha + psum;
  if constexpr (kPvOnMfma<G>) {
    // P.V on the matrix cores: out^T[d][h] += sum_t V[t][d] P[t][h] with
    // v_mfma_f32_16x16x16_bf16, 16 dims per tile.  B = P: lane (col, qr) already
    // holds P[4 qr + i][head col % G].  p is split into bf16 hi + lo (the top 8
    // and the next 8 mantissa bits), two products each, so p keeps 16 bits.
    // A = V^T: lane (col, qr) takes V[4 qr + i][16 j + col], read column-wise
    // from the V rows this wave wrote to LDS.
#pragma unroll
    for (int j = 0; j < 8; ++j) st.o[j] *= alpha;
    const uint16_t* vcol = reinterpret_cast<const uint16_t*>(ctx.v_lds);
#pragma unroll
    for (int c = 0; c < TC; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ctx.v_lds[(4 * qr + i) * kKRowPad + ctx.col] = r.v[c][i];
      uint32_t hb[4], lb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hb[i] = __float_as_uint(x[c][i]) & 0xFFFF0000u;
        lb[i] = __float_as_uint(x[c][i] - __uint_as_float(hb[i]));
      }
      const uint32_t hi[2] = {__builtin_amdgcn_perm(hb[1], hb[0], 0x07060302u),
                              __builtin_amdgcn_perm(hb[3], hb[2], 0x07060302u)};
      const uint32_t lo[2] = {__builtin_amdgcn_perm(lb[1], lb[0], 0x07060302u),
                              __builtin_amdgcn_perm(lb[3], lb[2], 0x07060302u)};
      const bf16x4_t phi = __builtin_bit_cast(bf16x4_t, hi);
      const bf16x4_t plo = __builtin_bit_cast(bf16x4_t, lo);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint16_t e[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) e[t] = vcol[(4 * qr + t) * (kKRowPad * 8) + 16 * j + ctx.col];
        const uint32_t va[2] = {e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16)};
        const bf16x4_t vt = __builtin_bit_cast(bf16x4_t, va);
        st.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, phi, st.o[j], 0, 0, 0);
        st.o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vt, plo, st.o[j], 0, 0, 0);
      }
    }
  } else {
    static_for<G>([&](auto rr) {
      constexpr int R = decltype(rr)::value;
      const float ar = row_ror<R>(alpha);
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[R][e] *= ar;
    });
#pragma unroll
    for (int c = 0; c < TC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float vf[8];
        unpack_bf16x8(r.v[c][i], vf);
        static_for<G>([&](auto rr) {
          constexpr int R = decltype(rr)::value;
          const float pr = row_ror<R>(x[c][i]);
#pragma unroll
          for (int e = 0; e < 8; ++e) st.acc[R][e] = fmaf(pr, vf[e], st.acc[R][e]);
        });
      }
  }
}

// Query operand of the group of kv head kvh, sequence b.
template <int G>
__device__ __forceinline__ void load_query(const DecodeArgs& a, int b, int kvh, int col, int qr,
                                           bf16x8_t (&qop)[4]) {
  const uint16_t* qrow =
      static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + kvh * G + col % G) * kD;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qop[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * qr));
}

// Streams tokens [begin, end) of one window through this wave's state, tile
// by tile.  The loads of the next tile are issued before the current tile is
// computed and reach the next iteration through `cur`, so a tile's loads are
// always in flight during the compute.  Past the window's end they re-read its
// last chunk and are never used.
template <int G, int BS, int TC>
__device__ __forceinline__ void stream_window(const DecodeArgs& a, const TileCtx& c, int begin,
                                              const bf16x8_t (&qop)[4], WaveState<G>& st) {
  constexpr int TILE = 16 * TC;
  int t0 = begin;
  KVTile<TC> cur;
  load_tile<BS, TC>(cur, t0, c);
#if PKV_PREFETCH_TILES >= 2
  KVTile<TC> n1;
  load_tile<BS, TC>(n1, t0 + TILE, c);
#endif
  // The first tile(s) pass through an empty asm so that the loop-carried
  // buffers are not loads on every incoming edge: otherwise the optimiser
  // merges the loads into one at the loop top, which undoes the prefetch.
  // (It waits for the first tile(s), which are needed next anyway.)
#pragma unroll
  for (int ch = 0; ch < TC; ++ch)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      asm volatile("" : "+v"(cur.k[ch][s]), "+v"(cur.v[ch][s]));
#if PKV_PREFETCH_TILES >= 2
      asm volatile("" : "+v"(n1.k[ch][s]), "+v"(n1.v[ch][s]));
#endif
    }
  while (true) {
    KVTile<TC> nxt;
    load_tile<BS, TC>(nxt, t0 + PKV_PREFETCH_TILES * TILE, c);
    compute_tile<G, TC>(cur, t0, c.end, qop, a.scale_log2e, c, st);
    t0 += TILE;
    if (t0 >= c.end) break;
#if PKV_PREFETCH_TILES >= 2
    cur = n1;
    n1 = nxt;
#else
    cur = nxt;
#endif
  }
}

// Streams tokens [begin, end) (begin a multiple of 16) of sequence b into the
// state of each wave, wave w for kv head kvh0 + w.  The block ids of a window
// of up to kMaxPartitionTokens tokens go to LDS once for all waves.  Every
// thread of the workgroup calls this with the same range.
template <int G, int BS, int TC>
__device__ __forceinline__ void attend_range(const DecodeArgs& a, int* s_bt, u32x4_t* k_lds,
                                             u32x4_t* v_lds, int b, int kvh, int begin, int end,
                                             const bf16x8_t (&qop)[4], WaveState<G>& st) {
  const int lane = threadIdx.x & 63;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;
  const uint16_t* qrow =
      static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + kvh * G) * kD;
  TileCtx c;
  c.tok_stride = (int64_t)a.num_kv_heads * kD;
  c.col = lane & 15;
  c.qr = lane >> 4;
#if PKV_K_VIA_LDS
  c.kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * kD + 8 * c.col;
  c.kdead = qrow + 8 * c.col;
  c.k_lds = k_lds;
#else
  c.kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * kD + 8 * c.qr;
  c.kdead = qrow + 8 * c.qr;  // + 32 s: 16 bytes inside the 128-element row
  c.k_lds = nullptr;
#endif
  c.vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * kD + 8 * c.col;
  c.vdead = qrow + 8 * c.col;
  c.v_lds = v_lds;
  c.s_bt = s_bt;
  for (int w0 = begin; w0 < end; w0 += kMaxPartitionTokens) {
    const int wend = min(end, w0 + kMaxPartitionTokens);
    const int blk0 = w0 / BS;
    const int nblk = (wend - 1) / BS - blk0 + 1;  // <= kMaxPartitionTokens / BS + 1
    __syncthreads();  // every wave is done with the previous window's ids
    for (int i = threadIdx.x; i < nblk; i += blockDim.x)
      s_bt[i] = checked_block(bt, blk0 + i, a.num_blocks, a.err);
    __syncthreads();
    c.blk0 = blk0;
    c.end = wend;
    c.last_chunk = ((wend - 1) >> 4) << 4;
    stream_window<G, BS, TC>(a, c, w0, qop, st);
  }
}

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
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    if (col >= G) return;  // columns >= G repeat heads 0 .. G-1
    const int h = col;
    if (sink.acc == nullptr) {
      const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G + h) * kD + 4 * qr;
      const float inv = 1.f / st.l;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) store_out(a, o + 16 * j + i, st.o[j][i] * inv);
    } else {
      const int64_t row = sink.row0 + h * sink.stride;
      float* dst = sink.acc + row * kD + 4 * qr;
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<f32x4_t*>(dst + 16 * j) = st.o[j];
      if (qr == 0) {
        sink.max[row] = st.m;
        sink.sum[row] = st.l;
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        st.acc[r][e] += __shfl_xor(st.acc[r][e], 16);
        st.acc[r][e] += __shfl_xor(st.acc[r][e], 32);
      }
    st.l += __shfl_xor(st.l, 16);
    st.l += __shfl_xor(st.l, 32);
    // Head, max and sum of every slot, by the same rotation as the accumulation
    // (computed by all lanes: DPP reads neighbouring lanes).
    int hsel[G];
    float msel[G], lsel[G];
    static_for<G>([&](auto rr) {
      constexpr int R = decltype(rr)::value;
      hsel[R] = row_ror<R>(col % G);
      msel[R] = row_ror<R>(st.m);
      lsel[R] = row_ror<R>(st.l);
    });
    if (qr != 0) return;
#pragma unroll
    for (int r = 0; r < G; ++r) {
      if (sink.acc == nullptr) {
        const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G + hsel[r]) * kD + 8 * col;
        const float inv = 1.f / lsel[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) store_out(a, o + e, st.acc[r][e] * inv);
      } else {
        const int64_t row = sink.row0 + hsel[r] * sink.stride;
        float* dst = sink.acc + row * kD + 8 * col;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = st.acc[r][e];
        if (col == 0) {
          sink.max[row] = msel[r];
          sink.sum[row] = lsel[r];
        }
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

// ----------------------------------------------------------------------------
// Partition grid: workgroup (kv-head group, sequence, partition), partitions
// dispatched from the last to the first so that the full partitions of long
// sequences start early and the short tails of short ones fill the end.
// ----------------------------------------------------------------------------
template <int G, int BS, int TC>
__global__ __launch_bounds__(kMaxWaves * 64) void decode_mfma_kernel(DecodeArgs a) {
  static_assert(16 % G == 0, "group must divide 16");
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[PKV_K_VIA_LDS ? kMaxWaves * 16 * kKRowPad : 1];
  __shared__ u32x4_t s_vt[kPvOnMfma<G> ? kMaxWaves * 16 * kKRowPad : 1];
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
  bf16x8_t qop[4];
  load_query<G>(a, b, kvh, lane & 15, lane >> 4, qop);
  WaveState<G> st;
  st.reset();
  attend_range<G, BS, TC>(a, s_bt, s_kt + (PKV_K_VIA_LDS ? wave * 16 * kKRowPad : 0),
                          s_vt + (kPvOnMfma<G> ? wave * 16 * kKRowPad : 0), b, kvh, pt.begin,
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
// are laid end to end (sequence 0's, then sequence 1's, ...).  For each
// kv-head group, gridDim.y workgroups take equal consecutive slices of that
// chunk stream, so every workgroup streams the same number of K/V bytes
// whatever the length mix; a slice may cover the end of one sequence, several
// whole sequences and the start of another.  Each workgroup computes the chunk
// prefix sums of seq_lens in LDS.  A sequence that lies inside one slice is
// written to `out` directly; a sequence cut by slice boundaries leaves one
// partial (max, sum, unnormalised output) per piece and balanced_reduce_kernel
// merges them.  Partial slot of a piece in slice s: 1 if the piece starts its
// sequence (it then ends the slice), else 0 (it then starts the slice), so
// each slot of a slice holds at most one piece.  Partial rows:
// [slice][Hkv][slot][G].  A slice holds the final piece of at most one cut
// sequence (its first piece); its merge descriptor ws_desc[slice] names that
// sequence and the slice of its first piece, or -1.
// ----------------------------------------------------------------------------
template <int G, int BS, int TC>
__global__ __launch_bounds__(kMaxWaves * 64) PKV_BALANCED_OCCUPANCY void decode_balanced_kernel(
    DecodeArgs a) {
  static_assert(16 % G == 0, "group must divide 16");
  __shared__ int s_bt[kMaxPartitionTokens / BS + 1];
  __shared__ u32x4_t s_kt[PKV_K_VIA_LDS ? kMaxWaves * 16 * kKRowPad : 1];
  __shared__ u32x4_t s_vt[kPvOnMfma<G> ? kMaxWaves * 16 * kKRowPad : 1];
  __shared__ int s_cc[kMaxBalancedSeqs + 1];
  __shared__ int s_wsum[kMaxWaves];

  const int nt = blockDim.x, nw = nt >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int kvh = blockIdx.x * nw + wave;
  const int slice = blockIdx.y, S = gridDim.y;
  const int B = a.num_seqs;
  const bool reporter = blockIdx.x == 0 && slice == 0;
  // Merge descriptor of this slice: no split sequence ends here (yet).
  int* desc = a.ws_desc + 2 * slice;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    desc[0] = -1;
    desc[1] = 0;
  }

  // Exclusive prefix sums of the chunk counts: s_cc[b] = chunks before b.
  int carry = 0;
  for (int base = 0; base < B; base += nt) {
    const int j = base + threadIdx.x;
    const int cnt = j < B ? (clamped_len(a, BS, j, reporter) + 15) >> 4 : 0;
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
  const int per = max(1, (total + S - 1) / S);

  if (slice == 0)  // sequences of length 0 get zero rows
    for (int j = 0; j < B; ++j)
      if (s_cc[j + 1] == s_cc[j]) zero_rows<G>(a, j, kvh);

  const int c_lo = slice * per;
  const int c_hi = min(total, c_lo + per);
  if (c_lo >= c_hi) return;
  // first sequence of the slice: the largest b < B with s_cc[b] <= c_lo
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_cc[mid] <= c_lo) lo = mid; else hi = mid;
  }
  int b = lo;
  int c = c_lo;
  while (c < c_hi) {
    while (s_cc[b + 1] <= c) ++b;  // skip sequences with no chunks
    const int cb = s_cc[b], ce = s_cc[b + 1];
    const int c_end = min(c_hi, ce);
    const int L = clamped_len(a, BS, b, false);
    const int tok_begin = (c - cb) * 16;
    const int tok_end = min((c_end - cb) * 16, L);
    const bool first = c == cb, last = c_end == ce;

    bf16x8_t qop[4];
    load_query<G>(a, b, kvh, lane & 15, lane >> 4, qop);
    WaveState<G> st;
    st.reset();
    attend_range<G, BS, TC>(a, s_bt, s_kt + (PKV_K_VIA_LDS ? wave * 16 * kKRowPad : 0),
                            s_vt + (kPvOnMfma<G> ? wave * 16 * kKRowPad : 0), b, kvh, tok_begin,
                            tok_end, qop, st);
    Sink sink{nullptr, nullptr, nullptr, 0, 0};
    if (!(first && last))
      sink = Sink{a.ws_acc, a.ws_max, a.ws_sum,
                  ((int64_t)(slice * a.num_kv_heads + kvh) * 2 + (first ? 1 : 0)) * G, 1};
    finish_wave<G>(a, st, b, kvh, sink);
    if (last && !first && blockIdx.x == 0 && threadIdx.x == 0) {
      // the final piece of a cut sequence: the reduce of this slice merges it
      desc[0] = b;
      desc[1] = cb / per;  // slice of its first piece
    }
    c = c_end;
  }
}

// Merges the pieces of the sequence whose final piece lies in slice
// blockIdx.x (if any): workgroup (slice, kv-head group), wave w for kv head
// kvg * KH + w, lane for output dims 2 lane and 2 lane + 1.  The pieces are
// merged with a running maximum, so the loads of all pieces are independent
// and issued together: out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p.
template <int G>
__global__ __launch_bounds__(kMaxWaves * 64) void balanced_reduce_kernel(DecodeArgs a) {
  const int slice = blockIdx.x;
  const int b = a.ws_desc[2 * slice];
  if (b < 0) return;
  const int s0 = a.ws_desc[2 * slice + 1], s1 = slice;
  const int kvh = blockIdx.y * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int d = 2 * (threadIdx.x & 63);
  const float* __restrict__ wmax = a.ws_max;
  const float* __restrict__ wsum = a.ws_sum;
  const float* __restrict__ wacc = a.ws_acc;
  float M[G], den[G], num0[G], num1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = -INFINITY;
    den[g] = num0[g] = num1[g] = 0.f;
  }
  // All loads first (no store in between), merged with a running maximum.
#pragma unroll 2
  for (int s = s0; s <= s1; ++s) {
    const int64_t r0 = ((int64_t)(s * a.num_kv_heads + kvh) * 2 + (s == s0 ? 1 : 0)) * G;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m = wmax[r0 + g], l = wsum[r0 + g];
      const float2 acc = *reinterpret_cast<const float2*>(wacc + (r0 + g) * kD + d);
      const float Mn = fmaxf(M[g], m);
      const float c_old = rescale(M[g], Mn), c_new = exp2_hw(m - Mn);
      den[g] = den[g] * c_old + l * c_new;
      num0[g] = num0[g] * c_old + acc.x * c_new;
      num1[g] = num1[g] * c_old + acc.y * c_new;
      M[g] = Mn;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t o = ((int64_t)b * a.num_q_heads + kvh * G + g) * kD + d;
    store_out(a, o, num0[g] / den[g]);
    store_out(a, o + 1, num1[g] / den[g]);
  }
}

template <int G>
hipError_t launch_partitions_g(const DecodeArgs& a, int block_size, int kh, hipStream_t s) {
  constexpr int TC = PKV_MFMA_TILE_CHUNKS;
  const dim3 grid(a.num_kv_heads / kh, a.num_seqs, a.max_parts);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: decode_mfma_kernel<G, 8, TC><<<grid, block, 0, s>>>(a); break;
    case 16: decode_mfma_kernel<G, 16, TC><<<grid, block, 0, s>>>(a); break;
    case 32: decode_mfma_kernel<G, 32, TC><<<grid, block, 0, s>>>(a); break;
    case 64: decode_mfma_kernel<G, 64, TC><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G>
hipError_t launch_balanced_g(const DecodeArgs& a, int block_size, int kh, hipStream_t s) {
  constexpr int TC = PKV_MFMA_TILE_CHUNKS;
  const dim3 grid(a.num_kv_heads / kh, a.slices);
  const dim3 block(kh * 64);
  switch (block_size) {
    case 8: decode_balanced_kernel<G, 8, TC><<<grid, block, 0, s>>>(a); break;
    case 16: decode_balanced_kernel<G, 16, TC><<<grid, block, 0, s>>>(a); break;
    case 32: decode_balanced_kernel<G, 32, TC><<<grid, block, 0, s>>>(a); break;
    case 64: decode_balanced_kernel<G, 64, TC><<<grid, block, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  balanced_reduce_kernel<G><<<dim3(a.slices, a.num_kv_heads / kh), block, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int mfma_waves_per_group(int num_kv_heads) {
  for (int kh = kMaxWaves; kh > 1; kh >>= 1)
    if (num_kv_heads % kh == 0) return kh;
  return 1;
}

hipError_t launch_mfma_decode(const DecodeArgs& a, int block_size, int group, hipStream_t s) {
  const int kh = mfma_waves_per_group(a.num_kv_heads);
  if (a.slices > 0) {
    if (a.num_seqs > kMaxBalancedSeqs) return hipErrorInvalidValue;
    switch (group) {
      case 1: return launch_balanced_g<1>(a, block_size, kh, s);
      case 2: return launch_balanced_g<2>(a, block_size, kh, s);
      case 4: return launch_balanced_g<4>(a, block_size, kh, s);
      case 8: return launch_balanced_g<8>(a, block_size, kh, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (group) {
    case 1: return launch_partitions_g<1>(a, block_size, kh, s);
    case 2: return launch_partitions_g<2>(a, block_size, kh, s);
    case 4: return launch_partitions_g<4>(a, block_size, kh, s);
    case 8: return launch_partitions_g<8>(a, block_size, kh, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv
