// Decode-step attention over a paged KV pool, for gfx950 (MI355X).
//
// What is computed ("Paged KV" wiki, section "Attention Kernel 的适配"): the
// kernel receives the block table and block_size, reaches each logical block
// of a sequence through the table and reads K/V block by block.  The result is
// ordinary softmax attention of one query token per head over the cached
// tokens (the explainer page: paging changes storage, not the attention
// algorithm).  Query head h reads KV head h / G, G = Hq / Hkv.
//
// Work decomposition: one workgroup per (kv head, token partition, sequence),
// grid (Hkv, max_parts, B), so the Hkv workgroups that read the same physical
// blocks are adjacent in dispatch order.  Each partition of part_tokens
// tokens keeps a running max / sum / unnormalised output in fp32 (the
// block-wise computation the wiki's "与 FlashAttention 的关系" section says can
// be combined with block-wise storage).  A sequence with one partition writes
// `out` directly; otherwise the partition writes its partial result and
// splitk_reduce_kernel merges the partitions with max/sum rescaling.
//
// Two main kernels:
//  * decode_mfma_kernel (bf16, head_dim 128, G in {1,2,4,8}): Q.K^T of the
//    whole query group against 16 tokens at a time on the matrix cores
//    (v_mfma_f32_16x16x32_bf16, K rows as the A operand straight from HBM,
//    the query group replicated across the 16 B columns), exp2-based online
//    softmax per tile, P.V on the vector ALUs in fp32 (p is never rounded to
//    bf16), with the probabilities of the other query heads fetched by DPP
//    row rotations instead of LDS round trips.
//  * decode_valu_kernel (fp32 any shape, bf16 head_dim 64): a plain vector
//    kernel where each group of lanes owns one token row at a time and keeps an
//    independent online softmax, merged at the end.
#include <type_traits>
#include <utility>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;  // waves per workgroup (256 threads)

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
  }(std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(m_old - m_new) with an empty side (-inf) weighted 0 even when both are -inf.
__device__ __forceinline__ float rescale(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : exp2_hw(m_old - m_new);
}

// Value of lane (row base + (i +/- R) mod 16) within this lane's 16-lane DPP row.
template <int R>
__device__ __forceinline__ int row_ror(int x) {
  if constexpr (R == 0) {
    return x;
  } else {
    return __builtin_amdgcn_update_dpp(0, x, 0x120 + R, 0xF, 0xF, false);
  }
}
template <int R>
__device__ __forceinline__ float row_ror(float x) {
  return __int_as_float(row_ror<R>(__float_as_int(x)));
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& w, float (&f)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[2 * j] = __uint_as_float(u[j] << 16);
    f[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;  // keep NaN a NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t i, float x) {
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[i] = f32_to_bf16_rne(x);
  else
    static_cast<float*>(a.out)[i] = x;
}

__device__ __forceinline__ int checked_block(const int32_t* bt, int bi, int64_t num_blocks,
                                             unsigned* err) {
  int phys = bt[bi];
  if (static_cast<uint64_t>(static_cast<int64_t>(phys)) >= static_cast<uint64_t>(num_blocks)) {
    atomicOr(err, kErrBlockId);
    phys = 0;  // never dereference an out-of-range id; the result is flagged
  }
  return phys;
}

struct Partition {
  int begin, end, count;  // token range [begin, end) and partitions of the sequence
};

// Returns false when this workgroup has nothing to do.  A sequence of length
// 0 gets a zero row from partition 0.
template <int G, int D>
__device__ __forceinline__ bool setup_partition(const DecodeArgs& a, int block_size, int b,
                                                int kvh, int part, Partition& p) {
  int L = a.seq_lens[b];
  const int cap = a.max_blocks_per_seq * block_size;
  if (L < 0 || L > cap) {
    if (threadIdx.x == 0 && kvh == 0 && part == 0) atomicOr(a.err, kErrSeqLen);
    L = L < 0 ? 0 : cap;
  }
  if (L == 0) {
    if (part == 0)
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        store_out(a, ((int64_t)b * a.num_q_heads + kvh * G) * D + i, 0.f);
    return false;
  }
  p.begin = part * a.part_tokens;
  if (p.begin >= L) return false;
  p.end = min(L, p.begin + a.part_tokens);
  p.count = (L + a.part_tokens - 1) / a.part_tokens;
  return true;
}

// Merge the per-wave (max, sum, acc) in LDS and write the partition's result:
// the final normalised row when the sequence has one partition, otherwise the
// partial (max, sum, unnormalised acc) for splitk_reduce_kernel.
template <int G, int D>
__device__ __forceinline__ void finish_partition(const DecodeArgs& a, int b, int kvh, int part,
                                                 int nparts, const float* s_max,
                                                 const float* s_sum, const float* s_acc) {
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int g = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_max[w * G + g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = rescale(s_max[w * G + g], M);
      num += sc * s_acc[(w * G + g) * D + d];
      den += sc * s_sum[w * G + g];
    }
    const int64_t row = (int64_t)b * a.num_q_heads + kvh * G + g;
    if (nparts == 1) {
      store_out(a, row * D + d, num / den);
    } else {
      const int64_t pr = row * a.max_parts + part;
      a.ws_acc[pr * D + d] = num;
      if (d == 0) {
        a.ws_max[pr] = M;
        a.ws_sum[pr] = den;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// MFMA kernel: bf16, head_dim 128.
//
// Lane layout inside a wave (lane = 16 * qr + col):
//   Q.K^T  A operand = K rows: lane holds 8 bf16 of token `col` of the chunk,
//          d-chunk (4 s + qr) in k-step s (64 contiguous bytes of 16 rows per
//          load instruction);
//          B operand = query group: column col is query head (col % G), same
//          d-chunks; result lane (col, qr), register i = score of query head
//          (col % G) with token 4 qr + i.
//   P.V    lane owns output dims 8 col .. 8 col + 7 and tokens 4 qr + i of
//          each chunk (each V load instruction reads 4 whole 256-byte rows);
//          slot r of its accumulator holds query head gsel[r] = the head of
//          the lane reached by DPP row rotation r, so the probabilities and
//          the rescale factors of that head arrive by the same rotation.
// Each wave takes tiles of TC * 16 tokens, wave w tiles w, w + 4, ...
// ----------------------------------------------------------------------------
template <int G, int BS, int TC>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int TILE = 16 * TC;
  static_assert(16 % G == 0, "group must divide 16");
  __shared__ float s_acc[kWaves * G * D];
  __shared__ float s_max[kWaves * G];
  __shared__ float s_sum[kWaves * G];

  const int kvh = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  Partition pt;
  if (!setup_partition<G, D>(a, BS, b, kvh, part, pt)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, qr = lane >> 4;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;  // elements between slots
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * D;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  bf16x8_t qop[4];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + ((int64_t)b * a.num_q_heads + kvh * G + col % G) * D;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qop[s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qrow + 32 * s + 8 * qr));
  }
  int gsel[G];
  static_for<G>([&](auto r) {
    constexpr int R = decltype(r)::value;
    gsel[R] = row_ror<R>(col % G);
  });

  float m_run = -INFINITY, l_run = 0.f;
  float acc[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;

  const int last_chunk = ((pt.end - 1) >> 4) << 4;
  for (int t0 = pt.begin + wave * TILE; t0 < pt.end; t0 += kWaves * TILE) {
    uint4 kr[TC][4], vr[TC][4];
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      const int tce = min(t0 + 16 * c, last_chunk);  // chunks past the end re-read the last one
      const int tk = min(tce + col, pt.end - 1);
      int pk, pv[4];
      if constexpr (BS >= 16) {
        const int phys = checked_block(bt, tce / BS, a.num_blocks, a.err);
        pk = phys;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = phys;
      } else {
        const int blk0 = tce / BS;
        const int blk1 = min(blk0 + 1, (pt.end - 1) / BS);
        const int p0 = checked_block(bt, blk0, a.num_blocks, a.err);
        const int p1 = checked_block(bt, blk1, a.num_blocks, a.err);
        pk = (tk / BS == blk0) ? p0 : p1;
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = (min(tce + 4 * qr + i, pt.end - 1) / BS == blk0) ? p0 : p1;
      }
      const uint16_t* kp = kbase + ((int64_t)pk * BS + (tk & (BS - 1))) * tok_stride + 8 * qr;
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[c][s] = *reinterpret_cast<const uint4*>(kp + 32 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tv = min(tce + 4 * qr + i, pt.end - 1);
        const uint16_t* vp = vbase + ((int64_t)pv[i] * BS + (tv & (BS - 1))) * tok_stride + 8 * col;
        vr[c][i] = *reinterpret_cast<const uint4*>(vp);
      }
    }

    float x[TC][4];
    float mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[c][s]),
                                                        qop[s], sacc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * c + 4 * qr + i;
        x[c][i] = tok < pt.end ? sacc[i] * a.scale_log2e : -INFINITY;
        mt = fmaxf(mt, x[c][i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);  // finite: the tile holds a valid token
    const float alpha = exp2_hw(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int c = 0; c < TC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[c][i] = exp2_hw(x[c][i] - m_new);
        psum += x[c][i];
      }
    l_run = l_run * alpha + psum;
    static_for<G>([&](auto r) {
      constexpr int R = decltype(r)::value;
      const float ar = row_ror<R>(alpha);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[R][e] *= ar;
    });
#pragma unroll
    for (int c = 0; c < TC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float vf[8];
        unpack_bf16x8(vr[c][i], vf);
        static_for<G>([&](auto r) {
          constexpr int R = decltype(r)::value;
          const float pr = row_ror<R>(x[c][i]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[R][e] = fmaf(pr, vf[e], acc[R][e]);
        });
      }
  }

  // Sum the four token rows (qr) of the wave, then merge the waves in LDS.
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[r][e] += __shfl_xor(acc[r][e], 16);
      acc[r][e] += __shfl_xor(acc[r][e], 32);
    }
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (qr == 0) {
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float* dst = s_acc + (wave * G + gsel[r]) * D + 8 * col;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = acc[r][e];
    }
  }
  if (lane < G) {
    s_max[wave * G + lane] = m_run;
    s_sum[wave * G + lane] = l_run;
  }
  __syncthreads();
  finish_partition<G, D>(a, b, kvh, part, pt.count, s_max, s_sum, s_acc);
}

// ----------------------------------------------------------------------------
// Generic vector kernel: T = float (fp32 pool) or uint16_t (bf16 pool).
// A row of D elements is read by LPT lanes, 16 bytes each; the workgroup holds
// NS = 256 / LPT token slots, slot j visiting tokens begin + j, begin + j + NS...
// Every slot keeps its own running max / sum / output for the G query heads of
// the group; slots are merged inside the wave with shuffles, then across waves.
// ----------------------------------------------------------------------------
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a, int block_size,
                                                          int block_shift) {
  constexpr int EPL = 16 / sizeof(T);
  constexpr int LPT = D / EPL;
  constexpr int NS = 256 / LPT;
  static_assert(LPT <= 64 && 64 % LPT == 0, "a row must fit in a wave");
  __shared__ float s_acc[kWaves * G * D];
  __shared__ float s_max[kWaves * G];
  __shared__ float s_sum[kWaves * G];

  const int kvh = blockIdx.x, part = blockIdx.y, b = blockIdx.z;
  Partition pt;
  if (!setup_partition<G, D>(a, block_size, b, kvh, part, pt)) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = threadIdx.x / LPT, c = threadIdx.x % LPT;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
  const T* kbase = static_cast<const T*>(a.k_cache) + (int64_t)kvh * D + c * EPL;
  const T* vbase = static_cast<const T*>(a.v_cache) + (int64_t)kvh * D + c * EPL;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  auto load_f = [](const T* p, float (&f)[EPL]) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    if constexpr (std::is_same_v<T, float>) {
      f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y);
      f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
    } else {
      unpack_bf16x8(w, f);
    }
  };

  float qv[G][EPL];
  const T* qrow = static_cast<const T*>(a.q) + ((int64_t)b * a.num_q_heads + kvh * G) * D + c * EPL;
#pragma unroll
  for (int g = 0; g < G; ++g) load_f(qrow + g * D, qv[g]);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  for (int t = pt.begin + slot; t < pt.end; t += NS) {
    const int phys = checked_block(bt, t >> block_shift, a.num_blocks, a.err);
    const int64_t row = ((int64_t)phys * block_size + (t & (block_size - 1))) * tok_stride;
    float kf[EPL], vf[EPL];
    load_f(kbase + row, kf);
    load_f(vbase + row, vf);
    float s[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qv[g][e], kf[e], d);
      s[g] = d;
    }
#pragma unroll
    for (int off = LPT / 2; off >= 1; off >>= 1)
#pragma unroll
      for (int g = 0; g < G; ++g) s[g] += __shfl_xor(s[g], off);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float x = s[g] * a.scale_log2e;
      const float mn = fmaxf(m[g], x);
      const float al = exp2_hw(m[g] - mn);
      const float p = exp2_hw(x - mn);
      l[g] = l[g] * al + p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, vf[e], acc[g][e] * al);
      m[g] = mn;
    }
  }

  // Merge the token slots of this wave (lanes LPT, 2 LPT, ... apart).
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a1 = rescale(m[g], mn), a2 = rescale(mo, mn);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] = acc[g][e] * a1 + __shfl_xor(acc[g][e], off) * a2;
      m[g] = mn;
    }
  }
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[(wave * G + g) * D + c * EPL + e] = acc[g][e];
      if (c == 0) {
        s_max[wave * G + g] = m[g];
        s_sum[wave * G + g] = l[g];
      }
    }
  }
  __syncthreads();
  finish_partition<G, D>(a, b, kvh, part, pt.count, s_max, s_sum, s_acc);
}

// ----------------------------------------------------------------------------
// Split-K reduce: one workgroup per (query head, sequence), one thread per
// output dimension.  out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(D) void splitk_reduce_kernel(DecodeArgs a, int block_size) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int L = a.seq_lens[b];
  const int cap = a.max_blocks_per_seq * block_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int64_t row = (int64_t)b * a.num_q_heads + h;
  const float* mx = a.ws_max + row * a.max_parts;
  const float* sm = a.ws_sum + row * a.max_parts;
  const float* ac = a.ws_acc + row * a.max_parts * D;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, mx[p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float sc = exp2_hw(mx[p] - M);
    num = fmaf(sc, ac[(int64_t)p * D + d], num);
    den = fmaf(sc, sm[p], den);
  }
  store_out(a, row * D + d, num / den);
}

template <int G>
hipError_t launch_mfma(const DecodeArgs& a, int block_size, dim3 grid, hipStream_t s) {
  constexpr int TC = 2;
  switch (block_size) {
    case 8: decode_mfma_kernel<G, 8, TC><<<grid, 256, 0, s>>>(a); break;
    case 16: decode_mfma_kernel<G, 16, TC><<<grid, 256, 0, s>>>(a); break;
    case 32: decode_mfma_kernel<G, 32, TC><<<grid, 256, 0, s>>>(a); break;
    case 64: decode_mfma_kernel<G, 64, TC><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_valu(const DecodeArgs& a, int block_size, int group, dim3 grid, hipStream_t s) {
  const int shift = __builtin_ctz(static_cast<unsigned>(block_size));
  switch (group) {
    case 1: decode_valu_kernel<T, D, 1><<<grid, 256, 0, s>>>(a, block_size, shift); break;
    case 2: decode_valu_kernel<T, D, 2><<<grid, 256, 0, s>>>(a, block_size, shift); break;
    case 4: decode_valu_kernel<T, D, 4><<<grid, 256, 0, s>>>(a, block_size, shift); break;
    case 8: decode_valu_kernel<T, D, 8><<<grid, 256, 0, s>>>(a, block_size, shift); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int bf16, int head_dim, int block_size, int group,
                         hipStream_t stream) {
  const dim3 grid(a.num_kv_heads, a.max_parts, a.num_seqs);
  hipError_t e = hipErrorInvalidValue;
  if (bf16 && head_dim == 128) {
    switch (group) {
      case 1: e = launch_mfma<1>(a, block_size, grid, stream); break;
      case 2: e = launch_mfma<2>(a, block_size, grid, stream); break;
      case 4: e = launch_mfma<4>(a, block_size, grid, stream); break;
      case 8: e = launch_mfma<8>(a, block_size, grid, stream); break;
      default: return hipErrorInvalidValue;
    }
  } else if (bf16 && head_dim == 64) {
    e = launch_valu<uint16_t, 64>(a, block_size, group, grid, stream);
  } else if (!bf16 && head_dim == 64) {
    e = launch_valu<float, 64>(a, block_size, group, grid, stream);
  } else if (!bf16 && head_dim == 128) {
    e = launch_valu<float, 128>(a, block_size, group, grid, stream);
  }
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const dim3 rgrid(a.num_q_heads, a.num_seqs);
  if (head_dim == 128)
    splitk_reduce_kernel<128><<<rgrid, 128, 0, stream>>>(a, block_size);
  else
    splitk_reduce_kernel<64><<<rgrid, 64, 0, stream>>>(a, block_size);
  return hipGetLastError();
}

}  // namespace pkv
