// Measurement support, not part of libpagedkv: a plain streaming read of a
// large device buffer, the practical HBM read rate the decode kernels are
// compared with.  Built into its own libpkv_probe.so and used only by the
// benchmark (bench.py --read-probe).
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
