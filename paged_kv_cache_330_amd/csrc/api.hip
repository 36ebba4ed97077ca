// C ABI of libpagedkv: argument validation, kernel choice and launch.
// Declarations and contracts: include/pagedkv.h.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace pkv {

WorkspaceLayout workspace_layout(int64_t rows, int64_t head_dim, int64_t desc_ints) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  WorkspaceLayout l;
  l.desc_off = 0;
  l.max_off = up(static_cast<size_t>(desc_ints) * sizeof(int));
  l.sum_off = l.max_off + up(static_cast<size_t>(rows) * sizeof(float));
  l.acc_off = l.sum_off + up(static_cast<size_t>(rows) * sizeof(float));
  l.total = l.acc_off + up(static_cast<size_t>(rows) * head_dim * sizeof(float));
  return l;
}

}  // namespace pkv

namespace {

// One error word per device; kernels OR range-check failures into it.
__device__ unsigned g_device_error;

constexpr int kMaxDevices = 64;
unsigned* g_error_word[kMaxDevices];
std::mutex g_error_mutex;

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Address of the current device's error word (looked up once per device).
int error_word(unsigned** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_HIP, "device ordinal %d too large", dev);
  std::lock_guard<std::mutex> lock(g_error_mutex);
  if (!g_error_word[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_device_error));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(error word)");
    g_error_word[dev] = static_cast<unsigned*>(p);
  }
  *out = g_error_word[dev];
  return PKV_OK;
}

// Workspace of pkv_attention_decode_noalloc: one array per device, for
// callers that cannot allocate.  In host code `scratch` names a host-side
// stand-in, not device memory: host code uses only the device address that
// hipGetSymbolAddress returns for the current device (g_scratch_ptr).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;  // 32 MiB
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
void* g_scratch_ptr[kMaxDevices];  // guarded by g_error_mutex

// Device address of the current device's `scratch` (looked up once per device).
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_HIP, "device ordinal %d too large", dev);
  std::lock_guard<std::mutex> lock(g_error_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : 1; }

int check_cache(const pkv_cache_desc* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "cache descriptor is NULL");
  if (c->num_blocks < 0 || c->num_blocks > (int64_t(1) << 40))
    return fail(PKV_ERR_INVALID_ARG, "num_blocks %lld out of range", (long long)c->num_blocks);
  if (c->dtype != PKV_F32 && c->dtype != PKV_BF16 && c->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "cache dtype %d is not PKV_F32, PKV_BF16 or PKV_FP8_E4M3",
                c->dtype);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", c->head_dim);
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32 && c->block_size != 64)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d is not 8, 16, 32 or 64", c->block_size);
  if (c->num_kv_heads < 1 || c->num_kv_heads > 1024)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads %d out of range", c->num_kv_heads);
  return PKV_OK;
}

// FP8 pools go through the *_fp8 calls, which also take their scales.
int check_not_fp8(const pkv_cache_desc* c, const char* call) {
  if (c->dtype == PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "%s does not take PKV_FP8_E4M3 pools; use %s_fp8", call, call);
  return PKV_OK;
}

int check_fp8(const pkv_cache_desc* c, const char* call) {
  if (c->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "%s takes PKV_FP8_E4M3 pools only", call);
  return PKV_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (!p) return fail(PKV_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(PKV_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return PKV_OK;
}

#define PKV_TRY(x)             \
  do {                         \
    int _s = (x);              \
    if (_s != PKV_OK) return _s; \
  } while (0)

int resolve_partition(int32_t partition_tokens, int32_t block_size, int32_t* part) {
  const int32_t p = partition_tokens == 0 ? pkv::kDefaultPartitionTokens : partition_tokens;
  if (p < 64 || p % 64 != 0 || p % block_size != 0 || p > pkv::kMaxPartitionTokens)
    return fail(PKV_ERR_INVALID_ARG,
                "partition_tokens %d must be 0 or a multiple of 64 and of block_size %d, at most %d",
                partition_tokens, block_size, pkv::kMaxPartitionTokens);
  *part = p;
  return PKV_OK;
}

// Device-side address of `p`: device memory as is, pinned host memory
// through its mapping; pageable host memory and unknown pointers fail.
int device_address(const void* p, const char* name, void** out) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    return fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory (%s)",
                name, hipGetErrorString(e));
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(p);
    return PKV_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr &&
      attr.hostPointer != nullptr) {
    // hostPointer/devicePointer may name the allocation or `p` itself; the
    // offset of `p` from hostPointer covers both.
    *out = static_cast<char*>(attr.devicePointer) +
           (static_cast<const char*>(p) - static_cast<const char*>(attr.hostPointer));
    return PKV_OK;
  }
  return fail(PKV_ERR_INVALID_ARG, "%s is neither device memory nor pinned host memory", name);
}

// Schedule and workspace of one decode call, from host-known sizes only.
struct Plan {
  int32_t part;       // partition grid: tokens per partition
  int64_t max_parts;  // partition grid: partitions of the longest possible sequence
  int32_t slices;     // > 0: balanced schedule, slices per kv head
  pkv::WorkspaceLayout layout;
  size_t workspace;   // bytes (0: none needed)
};

int make_plan(const pkv_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
              int32_t max_blocks_per_seq, int32_t partition_tokens, Plan* p) {
  PKV_TRY(check_cache(cache));
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs %d < 0", num_seqs);
  if (num_seqs > 65535) return fail(PKV_ERR_INVALID_ARG, "num_seqs %d > 65535", num_seqs);
  if (num_q_heads < 1 || num_q_heads % cache->num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, cache->num_kv_heads);
  if (max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  const int64_t max_tokens = static_cast<int64_t>(max_blocks_per_seq) * cache->block_size;
  if (max_tokens > 0x7FFFFFFF)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq * block_size exceeds 2^31 - 1");
  PKV_TRY(resolve_partition(partition_tokens, cache->block_size, &p->part));
  p->max_parts = (max_tokens + p->part - 1) / p->part;
  if (p->max_parts > 65535)
    return fail(PKV_ERR_INVALID_ARG, "%lld partitions per sequence exceed 65535",
                (long long)p->max_parts);
  // The balanced schedule serves the automatic choice for the head_dim 128
  // matrix-core kernels (bf16 and FP8 pools); an explicit partition size asks
  // for the partition grid.
  const bool balanced = partition_tokens == 0 &&
                        (cache->dtype == PKV_BF16 || cache->dtype == PKV_FP8_E4M3) &&
                        cache->head_dim == 128 && num_seqs <= pkv::kMaxBalancedSeqs &&
                        num_seqs > 0;
  p->slices = balanced ? pkv::balanced_slices(cache->num_kv_heads) : 0;
  p->workspace = 0;
  if (balanced) {
    p->layout = pkv::workspace_layout(static_cast<int64_t>(p->slices) * 2 * num_q_heads,
                                      cache->head_dim, 2 * static_cast<int64_t>(p->slices));
    p->workspace = p->layout.total;
  } else if (p->max_parts > 1 && num_seqs > 0) {
    p->layout = pkv::workspace_layout(static_cast<int64_t>(num_seqs) * num_q_heads * p->max_parts,
                                      cache->head_dim, 0);
    p->workspace = p->layout.total;
  }
  return PKV_OK;
}

// Schedule and workspace of one shared-prefix decode call.
struct SharedPlan {
  int32_t slices;       // slices per kv-head group
  int64_t prefix_rows;  // partial rows of prefix pieces
  pkv::WorkspaceLayout layout;
  size_t workspace;
};

int make_shared_plan(const pkv_cache_desc* cache, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_blocks_per_seq, int32_t num_groups, SharedPlan* p) {
  Plan base;
  PKV_TRY(make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, &base));
  if ((cache->dtype != PKV_BF16 && cache->dtype != PKV_FP8_E4M3) || cache->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED,
                "shared-prefix decode needs bf16 or FP8 pools with head_dim 128");
  const int group = num_q_heads / cache->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PKV_ERR_UNSUPPORTED, "query group %d is not 1, 2, 4 or 8", group);
  if (num_seqs > pkv::kMaxBalancedSeqs)
    return fail(PKV_ERR_UNSUPPORTED, "shared-prefix decode takes at most %d sequences, got %d",
                pkv::kMaxBalancedSeqs, num_seqs);
  if (num_groups < 0 || num_groups > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "num_groups %d is not in [0, num_seqs = %d]", num_groups,
                num_seqs);
  p->slices = pkv::balanced_slices(cache->num_kv_heads);
  p->prefix_rows = pkv::shared_prefix_rows(num_seqs, num_groups, cache->num_kv_heads, group,
                                           p->slices);
  const int64_t rows = p->prefix_rows + pkv::shared_tail_rows(num_seqs, num_q_heads, p->slices);
  p->layout = pkv::workspace_layout(rows, cache->head_dim,
                                    static_cast<int64_t>(pkv::kSharedDescInts) * num_seqs);
  p->workspace = num_seqs > 0 ? p->layout.total : 0;
  return PKV_OK;
}

// Query group, output type and scale of a decode call.
int check_decode_scalars(const pkv_cache_desc* cache, int32_t num_q_heads, int32_t out_dtype,
                         float scale) {
  const int group = num_q_heads / cache->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PKV_ERR_UNSUPPORTED, "query group %d is not 1, 2, 4 or 8", group);
  if (out_dtype != PKV_F32 && out_dtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "out_dtype %d is neither PKV_F32 nor PKV_BF16", out_dtype);
  if (!(scale == scale) || scale == INFINITY || scale == -INFINITY)
    return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  return PKV_OK;
}

// Checks shared by both decode calls; fills everything but the workspace
// and the error word (no HIP call here).
int fill_decode_args(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                     const void* v_cache, const pkv_cache_desc* cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                     pkv::DecodeArgs* a) {
  PKV_TRY(check_ptr(out, 16, "out"));
  PKV_TRY(check_ptr(q, 16, "q"));
  PKV_TRY(check_ptr(k_cache, 16, "k_cache"));
  PKV_TRY(check_ptr(v_cache, 16, "v_cache"));
  PKV_TRY(check_ptr(block_tables, 4, "block_tables"));
  PKV_TRY(check_ptr(seq_lens, 4, "seq_lens"));
  if (cache->num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  a->out = out;
  a->q = q;
  a->k_cache = k_cache;
  a->v_cache = v_cache;
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->num_blocks = cache->num_blocks;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = cache->num_kv_heads;
  a->out_bf16 = out_dtype == PKV_BF16;
  a->scale_log2e = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  return PKV_OK;
}

// Points the partial-result arrays of `a` into a checked workspace.
int attach_workspace(void* workspace, size_t workspace_bytes, size_t need,
                     const pkv::WorkspaceLayout& layout, pkv::DecodeArgs* a) {
  if (need == 0) return PKV_OK;
  if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(workspace, 16)) return fail(PKV_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required, got %zu", need,
                workspace_bytes);
  char* w = static_cast<char*>(workspace);
  a->ws_desc = reinterpret_cast<int*>(w + layout.desc_off);
  a->ws_max = reinterpret_cast<float*>(w + layout.max_off);
  a->ws_sum = reinterpret_cast<float*>(w + layout.sum_off);
  a->ws_acc = reinterpret_cast<float*>(w + layout.acc_off);
  return PKV_OK;
}

// Both bf16/fp32 decode calls.  no_alloc: the workspace is this device's
// `scratch` array (workspace/workspace_bytes unused); sizes past it are
// rejected before any HIP call.
int decode_common(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                  const void* v_cache, const pkv_cache_desc* cache, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                  int32_t num_q_heads, float scale, int32_t partition_tokens, void* workspace,
                  size_t workspace_bytes, bool no_alloc, void* stream) {
  Plan plan;
  PKV_TRY(make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan));
  PKV_TRY(check_not_fp8(cache, no_alloc ? "pkv_attention_decode_noalloc" : "pkv_attention_decode"));
  PKV_TRY(check_decode_scalars(cache, num_q_heads, out_dtype, scale));
  if (no_alloc && plan.workspace > kNoAllocScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "pkv_attention_decode_noalloc: these sizes need %zu bytes of scratch, more than "
                "the %zu bytes the library holds per device",
                plan.workspace, kNoAllocScratchBytes);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  PKV_TRY(fill_decode_args(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, &a));
  if (no_alloc && plan.workspace > 0) {
    PKV_TRY(scratch_address(&workspace));
    workspace_bytes = kNoAllocScratchBytes;
  }
  PKV_TRY(attach_workspace(workspace, workspace_bytes, plan.workspace, plan.layout, &a));
  PKV_TRY(error_word(&a.err));
  a.part_tokens = plan.part;
  a.max_parts = static_cast<int32_t>(plan.max_parts);
  a.slices = plan.slices;
  hipError_t e = pkv::launch_decode(a, cache->dtype == PKV_BF16, cache->head_dim,
                                    cache->block_size, num_q_heads / cache->num_kv_heads,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attention_decode launch");
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_kv_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                 void* k_cache, void* v_cache, const pkv_cache_desc* cache, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(cache));
  PKV_TRY(check_not_fp8(cache, "pkv_kv_write"));
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens == 0) return PKV_OK;
  PKV_TRY(check_ptr(k, 16, "k"));
  PKV_TRY(check_ptr(v, 16, "v"));
  PKV_TRY(check_ptr(slot_mapping, 8, "slot_mapping"));
  PKV_TRY(check_ptr(k_cache, 16, "k_cache"));
  PKV_TRY(check_ptr(v_cache, 16, "v_cache"));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  const int64_t row_bytes =
      static_cast<int64_t>(cache->num_kv_heads) * cache->head_dim * elem_bytes(cache->dtype);
  hipError_t e = pkv::launch_kv_write(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                      cache->num_blocks * cache->block_size, row_bytes, err,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_write launch");
}

int pkv_block_copy(void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                   const int64_t* src_dst_pairs, int64_t num_pairs, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(cache));
  PKV_TRY(check_not_fp8(cache, "pkv_block_copy"));
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs %lld < 0", (long long)num_pairs);
  if (num_pairs == 0) return PKV_OK;
  PKV_TRY(check_ptr(src_dst_pairs, 8, "src_dst_pairs"));
  PKV_TRY(check_ptr(k_cache, 16, "k_cache"));
  PKV_TRY(check_ptr(v_cache, 16, "v_cache"));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  const int64_t block_bytes = static_cast<int64_t>(cache->block_size) * cache->num_kv_heads *
                              cache->head_dim * elem_bytes(cache->dtype);
  hipError_t e = pkv::launch_block_copy(k_cache, v_cache, k_cache, v_cache, src_dst_pairs,
                                        num_pairs, cache->num_blocks, cache->num_blocks,
                                        block_bytes, err, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "block_copy launch");
}

int pkv_block_transfer(void* dst_k, void* dst_v, const pkv_cache_desc* dst_cache,
                       const void* src_k, const void* src_v, const pkv_cache_desc* src_cache,
                       const int64_t* src_dst_pairs, int64_t num_pairs, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(dst_cache));
  PKV_TRY(check_cache(src_cache));
  PKV_TRY(check_not_fp8(src_cache, "pkv_block_transfer"));
  if (dst_cache->block_size != src_cache->block_size ||
      dst_cache->num_kv_heads != src_cache->num_kv_heads ||
      dst_cache->head_dim != src_cache->head_dim || dst_cache->dtype != src_cache->dtype)
    return fail(PKV_ERR_INVALID_ARG, "source and destination pools differ in block shape or dtype");
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs %lld < 0", (long long)num_pairs);
  if (num_pairs == 0) return PKV_OK;
  PKV_TRY(check_ptr(src_dst_pairs, 8, "src_dst_pairs"));
  PKV_TRY(check_ptr(dst_k, 16, "dst_k"));
  PKV_TRY(check_ptr(dst_v, 16, "dst_v"));
  PKV_TRY(check_ptr(src_k, 16, "src_k"));
  PKV_TRY(check_ptr(src_v, 16, "src_v"));
  // Every pool must be memory the device can address: device memory, or
  // pinned host memory mapped for the device (its device-side address is
  // used).  Anything else is rejected here instead of faulting in the kernel.
  void* dk = nullptr;
  void* dv = nullptr;
  const void* sk = nullptr;
  const void* sv = nullptr;
  PKV_TRY(device_address(dst_k, "dst_k", &dk));
  PKV_TRY(device_address(dst_v, "dst_v", &dv));
  PKV_TRY(device_address(src_k, "src_k", const_cast<void**>(&sk)));
  PKV_TRY(device_address(src_v, "src_v", const_cast<void**>(&sv)));
  void* pairs_dev = nullptr;
  PKV_TRY(device_address(src_dst_pairs, "src_dst_pairs", &pairs_dev));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  const int64_t block_bytes = static_cast<int64_t>(src_cache->block_size) *
                              src_cache->num_kv_heads * src_cache->head_dim *
                              elem_bytes(src_cache->dtype);
  hipError_t e = pkv::launch_block_copy(dk, dv, sk, sv, static_cast<const int64_t*>(pairs_dev),
                                        num_pairs, src_cache->num_blocks, dst_cache->num_blocks,
                                        block_bytes, err, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "block_transfer launch");
}

size_t pkv_attention_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_blocks_per_seq,
                                     int32_t partition_tokens) {
  Plan p;
  if (make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &p) != PKV_OK)
    return 0;
  return p.workspace;
}

int pkv_attention_decode(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                         const void* v_cache, const pkv_cache_desc* cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return decode_common(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                       partition_tokens, workspace, workspace_bytes, false, stream);
}

int pkv_attention_decode_noalloc(void* out, int32_t out_dtype, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const pkv_cache_desc* cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t num_q_heads, float scale,
                                 int32_t partition_tokens, void* stream) {
  g_last_error.clear();
  return decode_common(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale,
                       partition_tokens, nullptr, 0, true, stream);
}

size_t pkv_attention_shared_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t num_groups) {
  SharedPlan p;
  if (make_shared_plan(cache, num_seqs, num_q_heads, 1, num_groups, &p) != PKV_OK) return 0;
  return p.workspace;
}

}  // extern "C"

namespace {

// Both prefill calls: FP8 pools bring their scales.
int prefill_common(void* out, int32_t out_dtype, const void* q, int64_t num_tokens,
                   const int32_t* query_start, const void* k_cache, const void* v_cache,
                   const float* k_scale, const float* v_scale, const pkv_cache_desc* cache,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                   void* stream, bool fp8) {
  Plan base;
  PKV_TRY(make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, 0, &base));
  PKV_TRY(check_decode_scalars(cache, num_q_heads, out_dtype, scale));
  if (fp8) {
    PKV_TRY(check_fp8(cache, "pkv_attention_prefill_fp8"));
  } else {
    PKV_TRY(check_not_fp8(cache, "pkv_attention_prefill"));
  }
  if (cache->head_dim != 128 || (!fp8 && cache->dtype != PKV_BF16))
    return fail(PKV_ERR_UNSUPPORTED, "prefill attention needs %s pools with head_dim 128",
                fp8 ? "FP8" : "bf16");
  if (num_seqs > pkv::kMaxBalancedSeqs)
    return fail(PKV_ERR_UNSUPPORTED, "prefill attention takes at most %d sequences, got %d",
                pkv::kMaxBalancedSeqs, num_seqs);
  if (num_tokens < 0 || num_tokens > 0x7FFFFFFF)
    return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld out of range", (long long)num_tokens);
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  pkv::PrefillArgs pa{};
  PKV_TRY(fill_decode_args(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, &pa.d));
  PKV_TRY(check_ptr(query_start, 4, "query_start"));
  if (fp8) {
    PKV_TRY(check_ptr(k_scale, 4, "k_scale"));
    PKV_TRY(check_ptr(v_scale, 4, "v_scale"));
    pa.d.k_scale = k_scale;
    pa.d.v_scale = v_scale;
  }
  PKV_TRY(error_word(&pa.d.err));
  pa.query_start = query_start;
  pa.num_tokens = num_tokens;
  hipError_t e = pkv::launch_prefill(pa, cache->block_size, num_q_heads / cache->num_kv_heads,
                                     static_cast<hipStream_t>(stream), fp8);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attention_prefill launch");
}

// Both shared-prefix decode calls: FP8 pools bring their scales.
int shared_common(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                  const void* v_cache, const float* k_scale, const float* v_scale,
                  const pkv_cache_desc* cache, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                  int32_t num_q_heads, float scale, const int32_t* group_offsets,
                  const int32_t* group_seqs, const int32_t* group_lens, int32_t num_groups,
                  void* workspace, size_t workspace_bytes, void* stream, bool fp8) {
  SharedPlan plan;
  PKV_TRY(make_shared_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, num_groups, &plan));
  if (fp8) {
    PKV_TRY(check_fp8(cache, "pkv_attention_decode_shared_fp8"));
  } else {
    PKV_TRY(check_not_fp8(cache, "pkv_attention_decode_shared"));
  }
  PKV_TRY(check_decode_scalars(cache, num_q_heads, out_dtype, scale));
  if (num_seqs == 0) return PKV_OK;
  pkv::SharedArgs sa{};
  PKV_TRY(fill_decode_args(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, &sa.d));
  if (fp8) {
    PKV_TRY(check_ptr(k_scale, 4, "k_scale"));
    PKV_TRY(check_ptr(v_scale, 4, "v_scale"));
    sa.d.k_scale = k_scale;
    sa.d.v_scale = v_scale;
  }
  if (num_groups > 0) {
    PKV_TRY(check_ptr(group_offsets, 4, "group_offsets"));
    PKV_TRY(check_ptr(group_seqs, 4, "group_seqs"));
    PKV_TRY(check_ptr(group_lens, 4, "group_lens"));
  }
  PKV_TRY(attach_workspace(workspace, workspace_bytes, plan.workspace, plan.layout, &sa.d));
  PKV_TRY(error_word(&sa.d.err));
  sa.d.slices = plan.slices;
  sa.group_offsets = group_offsets;
  sa.group_seqs = group_seqs;
  sa.group_lens = group_lens;
  sa.num_groups = num_groups;
  sa.prefix_rows = plan.prefix_rows;
  hipError_t e = pkv::launch_shared_decode(sa, cache->block_size,
                                           num_q_heads / cache->num_kv_heads,
                                           static_cast<hipStream_t>(stream), fp8);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attention_decode_shared launch");
}

}  // namespace

extern "C" {

int pkv_attention_decode_shared(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                                const void* v_cache, const pkv_cache_desc* cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                float scale, const int32_t* group_offsets,
                                const int32_t* group_seqs, const int32_t* group_lens,
                                int32_t num_groups, void* workspace, size_t workspace_bytes,
                                void* stream) {
  g_last_error.clear();
  return shared_common(out, out_dtype, q, k_cache, v_cache, nullptr, nullptr, cache, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, group_offsets,
                       group_seqs, group_lens, num_groups, workspace, workspace_bytes, stream,
                       false);
}

int pkv_attention_decode_shared_fp8(void* out, int32_t out_dtype, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const pkv_cache_desc* cache, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    const int32_t* group_offsets, const int32_t* group_seqs,
                                    const int32_t* group_lens, int32_t num_groups,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return shared_common(out, out_dtype, q, k_cache, v_cache, k_scale, v_scale, cache, block_tables,
                       max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, group_offsets,
                       group_seqs, group_lens, num_groups, workspace, workspace_bytes, stream,
                       true);
}

int pkv_attention_prefill(void* out, int32_t out_dtype, const void* q, int64_t num_tokens,
                          const int32_t* query_start, const void* k_cache, const void* v_cache,
                          const pkv_cache_desc* cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, void* stream) {
  g_last_error.clear();
  return prefill_common(out, out_dtype, q, num_tokens, query_start, k_cache, v_cache, nullptr,
                        nullptr, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                        num_q_heads, scale, stream, false);
}

int pkv_attention_prefill_fp8(void* out, int32_t out_dtype, const void* q, int64_t num_tokens,
                              const int32_t* query_start, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              const pkv_cache_desc* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, float scale, void* stream) {
  g_last_error.clear();
  return prefill_common(out, out_dtype, q, num_tokens, query_start, k_cache, v_cache, k_scale,
                        v_scale, cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                        num_q_heads, scale, stream, true);
}

int pkv_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                     int64_t num_tokens, void* k_cache, void* v_cache, const float* k_scale,
                     const float* v_scale, const pkv_cache_desc* cache, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(cache));
  PKV_TRY(check_fp8(cache, "pkv_kv_write_fp8"));
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens %lld < 0", (long long)num_tokens);
  if (num_tokens == 0) return PKV_OK;
  PKV_TRY(check_ptr(k, 16, "k"));
  PKV_TRY(check_ptr(v, 16, "v"));
  PKV_TRY(check_ptr(slot_mapping, 8, "slot_mapping"));
  PKV_TRY(check_ptr(k_cache, 16, "k_cache"));
  PKV_TRY(check_ptr(v_cache, 16, "v_cache"));
  PKV_TRY(check_ptr(k_scale, 4, "k_scale"));
  PKV_TRY(check_ptr(v_scale, 4, "v_scale"));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  hipError_t e = pkv::launch_kv_write_fp8(k, v, slot_mapping, num_tokens, k_cache, v_cache,
                                          k_scale, v_scale, cache->num_blocks * cache->block_size,
                                          cache->block_size, cache->num_kv_heads, cache->head_dim,
                                          err, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : hip_fail(e, "kv_write_fp8 launch");
}

int pkv_attention_decode_fp8(void* out, int32_t out_dtype, const void* q, const void* k_cache,
                             const void* v_cache, const float* k_scale, const float* v_scale,
                             const pkv_cache_desc* cache, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t num_q_heads, float scale,
                             int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_last_error.clear();
  Plan plan;
  PKV_TRY(make_plan(cache, num_seqs, num_q_heads, max_blocks_per_seq, partition_tokens, &plan));
  PKV_TRY(check_fp8(cache, "pkv_attention_decode_fp8"));
  if (cache->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "FP8 decode needs head_dim 128, got %d", cache->head_dim);
  PKV_TRY(check_decode_scalars(cache, num_q_heads, out_dtype, scale));
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  PKV_TRY(fill_decode_args(out, out_dtype, q, k_cache, v_cache, cache, block_tables,
                           max_blocks_per_seq, seq_lens, num_seqs, num_q_heads, scale, &a));
  PKV_TRY(check_ptr(k_scale, 4, "k_scale"));
  PKV_TRY(check_ptr(v_scale, 4, "v_scale"));
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  PKV_TRY(attach_workspace(workspace, workspace_bytes, plan.workspace, plan.layout, &a));
  PKV_TRY(error_word(&a.err));
  a.part_tokens = plan.part;
  a.max_parts = static_cast<int32_t>(plan.max_parts);
  a.slices = plan.slices;
  hipError_t e = pkv::launch_decode(a, 0, cache->head_dim, cache->block_size,
                                    num_q_heads / cache->num_kv_heads,
                                    static_cast<hipStream_t>(stream), true);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "attention_decode_fp8 launch");
}

int pkv_block_copy_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pkv_cache_desc* cache, const int64_t* src_dst_pairs,
                       int64_t num_pairs, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(cache));
  PKV_TRY(check_fp8(cache, "pkv_block_copy_fp8"));
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs %lld < 0", (long long)num_pairs);
  if (num_pairs == 0) return PKV_OK;
  PKV_TRY(check_ptr(src_dst_pairs, 8, "src_dst_pairs"));
  PKV_TRY(check_ptr(k_cache, 16, "k_cache"));
  PKV_TRY(check_ptr(v_cache, 16, "v_cache"));
  PKV_TRY(check_ptr(k_scale, 4, "k_scale"));
  PKV_TRY(check_ptr(v_scale, 4, "v_scale"));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  const int64_t block_bytes = static_cast<int64_t>(cache->block_size) * cache->num_kv_heads *
                              cache->head_dim * elem_bytes(cache->dtype);
  pkv::BlockScales sc;
  sc.dst_ks = k_scale;
  sc.dst_vs = v_scale;
  sc.src_ks = k_scale;
  sc.src_vs = v_scale;
  sc.scales = cache->num_kv_heads;
  hipError_t e = pkv::launch_block_copy(k_cache, v_cache, k_cache, v_cache, src_dst_pairs,
                                        num_pairs, cache->num_blocks, cache->num_blocks,
                                        block_bytes, err, static_cast<hipStream_t>(stream), sc);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "block_copy_fp8 launch");
}

int pkv_block_transfer_fp8(void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                           const pkv_cache_desc* dst_cache, const void* src_k, const void* src_v,
                           const float* src_k_scale, const float* src_v_scale,
                           const pkv_cache_desc* src_cache, const int64_t* src_dst_pairs,
                           int64_t num_pairs, void* stream) {
  g_last_error.clear();
  PKV_TRY(check_cache(dst_cache));
  PKV_TRY(check_cache(src_cache));
  PKV_TRY(check_fp8(src_cache, "pkv_block_transfer_fp8"));
  if (dst_cache->block_size != src_cache->block_size ||
      dst_cache->num_kv_heads != src_cache->num_kv_heads ||
      dst_cache->head_dim != src_cache->head_dim || dst_cache->dtype != src_cache->dtype)
    return fail(PKV_ERR_INVALID_ARG, "source and destination pools differ in block shape or dtype");
  if (num_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "num_pairs %lld < 0", (long long)num_pairs);
  if (num_pairs == 0) return PKV_OK;
  PKV_TRY(check_ptr(src_dst_pairs, 8, "src_dst_pairs"));
  PKV_TRY(check_ptr(dst_k, 16, "dst_k"));
  PKV_TRY(check_ptr(dst_v, 16, "dst_v"));
  PKV_TRY(check_ptr(src_k, 16, "src_k"));
  PKV_TRY(check_ptr(src_v, 16, "src_v"));
  PKV_TRY(check_ptr(dst_k_scale, 4, "dst_k_scale"));
  PKV_TRY(check_ptr(dst_v_scale, 4, "dst_v_scale"));
  PKV_TRY(check_ptr(src_k_scale, 4, "src_k_scale"));
  PKV_TRY(check_ptr(src_v_scale, 4, "src_v_scale"));
  void* dk = nullptr;
  void* dv = nullptr;
  const void* sk = nullptr;
  const void* sv = nullptr;
  void* dks = nullptr;
  void* dvs = nullptr;
  const void* sks = nullptr;
  const void* svs = nullptr;
  PKV_TRY(device_address(dst_k, "dst_k", &dk));
  PKV_TRY(device_address(dst_v, "dst_v", &dv));
  PKV_TRY(device_address(src_k, "src_k", const_cast<void**>(&sk)));
  PKV_TRY(device_address(src_v, "src_v", const_cast<void**>(&sv)));
  PKV_TRY(device_address(dst_k_scale, "dst_k_scale", &dks));
  PKV_TRY(device_address(dst_v_scale, "dst_v_scale", &dvs));
  PKV_TRY(device_address(src_k_scale, "src_k_scale", const_cast<void**>(&sks)));
  PKV_TRY(device_address(src_v_scale, "src_v_scale", const_cast<void**>(&svs)));
  void* pairs_dev = nullptr;
  PKV_TRY(device_address(src_dst_pairs, "src_dst_pairs", &pairs_dev));
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  const int64_t block_bytes = static_cast<int64_t>(src_cache->block_size) *
                              src_cache->num_kv_heads * src_cache->head_dim *
                              elem_bytes(src_cache->dtype);
  pkv::BlockScales sc;
  sc.dst_ks = static_cast<float*>(dks);
  sc.dst_vs = static_cast<float*>(dvs);
  sc.src_ks = static_cast<const float*>(sks);
  sc.src_vs = static_cast<const float*>(svs);
  sc.scales = src_cache->num_kv_heads;
  hipError_t e = pkv::launch_block_copy(dk, dv, sk, sv, static_cast<const int64_t*>(pairs_dev),
                                        num_pairs, src_cache->num_blocks, dst_cache->num_blocks,
                                        block_bytes, err, static_cast<hipStream_t>(stream), sc);
  return e == hipSuccess ? PKV_OK : hip_fail(e, "block_transfer_fp8 launch");
}

int pkv_check_device_errors(void* stream) {
  g_last_error.clear();
  unsigned* err = nullptr;
  PKV_TRY(error_word(&err));
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  unsigned word = 0;
  e = hipMemcpy(&word, err, sizeof(word), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
  if (word == 0) return PKV_OK;
  const unsigned zero = 0;
  e = hipMemcpy(err, &zero, sizeof(zero), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clear error word)");
  return fail(PKV_ERR_INVALID_ARG, "device range checks failed:%s%s%s%s%s%s%s",
              (word & pkv::kErrSlot) ? " slot>=num_blocks*block_size" : "",
              (word & pkv::kErrBlockId) ? " block_id_out_of_range" : "",
              (word & pkv::kErrSeqLen) ? " seq_len_out_of_range" : "",
              (word & pkv::kErrCopyPair) ? " copy_pair_out_of_range" : "",
              (word & pkv::kErrShared) ? " shared_prefix_inconsistent" : "",
              (word & pkv::kErrQuery) ? " prefill_query_range_inconsistent" : "",
              (word & pkv::kErrScale) ? " fp8_scale_not_positive_finite" : "");
}

}  // extern "C"
