// Decode-step attention on the vector ALUs (fp32 pools, and bf16 pools with
// head_dim 64), the split-K reduce of the partition grid, and the dispatch
// between these and the matrix-core kernels of attention_mfma.hip.
//
// What is computed ("Paged KV" wiki, section "Attention Kernel 的适配"): the
// kernel receives the block table and block_size, reaches each logical block
// of a sequence through the table and reads K/V block by block; the result is
// ordinary softmax attention of one query token per head over the cached
// tokens.  Query head h reads kv head h / G, G = Hq / Hkv.
//
// Partition grid: workgroup (kv head, sequence, partition of part_tokens
// tokens), highest partition dispatched first.  A row of D elements is read by
// LPT lanes, 16 bytes each; the workgroup holds NS = 256 / LPT token slots,
// slot j visiting tokens begin + j, begin + j + NS, ...; every slot keeps its
// own running max / sum / output for the G query heads of the group (fp32
// throughout: no bf16 matrix instruction touches fp32 data), and the slots
// are merged inside the wave with shuffles, then across waves in LDS.
#include <type_traits>

#include "decode_common.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;  // waves per workgroup (256 threads)

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

  const int kvh = blockIdx.x, b = blockIdx.y, part = gridDim.z - 1 - blockIdx.z;
  Partition pt;
  if (!setup_partition(a, block_size, b, part, kvh == 0 && threadIdx.x == 0, pt)) {
    if (pt.len == 0 && part == 0)
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        store_out(a, ((int64_t)b * a.num_q_heads + kvh * G) * D + i, 0.f);
    return;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slot = threadIdx.x / LPT, c = threadIdx.x % LPT;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;
  const T* kbase = static_cast<const T*>(a.k_cache) + (int64_t)kvh * D + c * EPL;
  const T* vbase = static_cast<const T*>(a.v_cache) + (int64_t)kvh * D + c * EPL;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks_per_seq;

  auto load_f = [](const T* p, float (&f)[EPL]) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
    if constexpr (std::is_same_v<T, float>) {
#pragma unroll
      for (int j = 0; j < 4; ++j) f[j] = __uint_as_float(w[j]);
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

  // Merge the waves; write the normalised row (one partition) or the partial.
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
    if (pt.count == 1) {
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

// Split-K reduce of the partition grid: one workgroup per (query head,
// sequence), one thread per output dimension:
// out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p,  M = max_p m_p.
// Both loops are unrolled so that the loads of eight partitions are in
// flight together (a long sequence has 64 partitions of 512 tokens).
template <int D>
__global__ __launch_bounds__(D) void splitk_reduce_kernel(DecodeArgs a, int block_size) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = clamped_len(a, block_size, b, false);
  const int nparts = (L + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;  // written by the main kernel
  const int64_t row = (int64_t)b * a.num_q_heads + h;
  const float* __restrict__ mx = a.ws_max + row * a.max_parts;
  const float* __restrict__ sm = a.ws_sum + row * a.max_parts;
  const float* __restrict__ ac = a.ws_acc + row * a.max_parts * D;
  float M = -INFINITY;
#pragma unroll 8
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, mx[p]);
  float num = 0.f, den = 0.f;
#pragma unroll 8
  for (int p = 0; p < nparts; ++p) {
    const float sc = exp2_hw(mx[p] - M);
    num = fmaf(sc, ac[(int64_t)p * D + d], num);
    den = fmaf(sc, sm[p], den);
  }
  store_out(a, row * D + d, num / den);
}

template <typename T, int D>
hipError_t launch_valu(const DecodeArgs& a, int block_size, int group, hipStream_t s) {
  const int shift = __builtin_ctz(static_cast<unsigned>(block_size));
  const dim3 grid(a.num_kv_heads, a.num_seqs, a.max_parts);
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
                         hipStream_t stream, bool fp8) {
  hipError_t e = hipErrorInvalidValue;
  if (fp8 && head_dim != 128) return hipErrorInvalidValue;
  if ((bf16 || fp8) && head_dim == 128) {
    e = launch_mfma_decode(a, block_size, group, stream, fp8);
    if (e != hipSuccess || a.slices > 0) return e;  // the balanced schedule has its own reduce
  } else if (a.slices > 0) {
    return hipErrorInvalidValue;
  } else if (bf16 && head_dim == 64) {
    e = launch_valu<uint16_t, 64>(a, block_size, group, stream);
  } else if (!bf16 && head_dim == 64) {
    e = launch_valu<float, 64>(a, block_size, group, stream);
  } else if (!bf16 && head_dim == 128) {
    e = launch_valu<float, 128>(a, block_size, group, stream);
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
