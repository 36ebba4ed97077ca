// Measurement support, not part of libpagedkv: the practical HBM read rates
// the decode kernels are compared with.  A plain streaming read of a large
// device buffer, and a paged read of K/V blocks in a given order with the
// decode kernels' wave layout and no compute.  Built into its own
// libpkv_probe.so and used only by the benchmark (bench.py --read-probe).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte vectors, 4 grid strides per iteration, with the
// streaming hint, and folds them into a value that is stored only if it
// equals a constant that practically never occurs (so no load is dead).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ p,
                                                          int64_t n_vec, unsigned* out) {
  unsigned acc = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(p + i);
    const u32x4_t b = __builtin_nontemporal_load(p + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n_vec; i += stride) acc ^= p[i].x;
  if (acc == 0x9E3779B9u) out[0] = acc;
}

// K and V rows of physical blocks blocks[0 .. nblocks) (bf16, head_dim 128,
// block size a multiple of 16), read as the decode kernels read them: a
// workgroup of 8 waves, wave w for kv head 8 blockIdx.y + w, lane
// (col, qr) loading 16 bytes of rows 4 qr .. 4 qr + 3 of each 16-token tile
// with the streaming hint; every workgroup takes an equal consecutive share of
// the block list.  Nothing is computed: the loaded words are folded into a
// value stored only if it equals a constant that practically never occurs.
__global__ __launch_bounds__(512) void paged_read_kernel(const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ blocks,
                                                         int nblocks, int bs, int hkv,
                                                         unsigned* out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, qr = lane >> 4;
  const int kvh = blockIdx.y * 8 + wave;
  const int per = (nblocks + gridDim.x - 1) / gridDim.x;
  const int b0 = blockIdx.x * per, b1 = min(nblocks, b0 + per);
  const int tiles = bs / 16;
  const int64_t stride = (int64_t)hkv * 128;
  u32x4_t acc = {0, 0, 0, 0};
  for (int t = 0; t < (b1 - b0) * tiles; ++t) {
    const int blk = blocks[b0 + t / tiles];
    const int tok0 = (t % tiles) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = ((int64_t)blk * bs + tok0 + 4 * qr + i) * stride + kvh * 128 + 8 * col;
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k + row));
      acc ^= __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v + row));
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9E3779B9u) out[0] = acc.x;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from `p` with `blocks` workgroups of 256
// threads on `stream`; `out` is a 4-byte device word.  Returns 0, or -1 on a
// bad argument or launch failure.
extern "C" int pkv_probe_stream_read(const void* p, int64_t bytes, void* out, int blocks,
                                     void* stream) {
  if (!p || !out || bytes <= 0 || bytes % 16 != 0 || blocks <= 0) return -1;
  stream_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4_t*>(p), bytes / 16, static_cast<unsigned*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Reads the K and V blocks listed in `blocks` (device int32, `nblocks` ids,
// each in [0, pool blocks)) of bf16 pools with head_dim 128, block_size a
// multiple of 16 and num_kv_heads a multiple of 8, with `workgroups`
// workgroups per 8 kv heads on `stream`; `out` is a 4-byte device word.
// Returns 0, or -1 on a bad argument or launch failure.
extern "C" int pkv_probe_paged_read(const void* k, const void* v, const int32_t* blocks,
                                    int nblocks, int block_size, int num_kv_heads, void* out,
                                    int workgroups, void* stream) {
  if (!k || !v || !blocks || !out || nblocks <= 0 || block_size < 16 || block_size % 16 != 0 ||
      num_kv_heads < 8 || num_kv_heads % 8 != 0 || workgroups <= 0)
    return -1;
  paged_read_kernel<<<dim3(workgroups, num_kv_heads / 8), 512, 0,
                      static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), blocks, nblocks,
      block_size, num_kv_heads, static_cast<unsigned*>(out));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
