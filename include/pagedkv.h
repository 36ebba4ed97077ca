/*
 * pagedkv.h - C ABI of the MI355X (gfx950) paged KV-cache decode path.
 *
 * The KV cache of one attention layer is a pool of equal physical blocks,
 * one pool for K and one for V, each laid out as
 *     [num_blocks][block_size][num_kv_heads][head_dim]
 * ("Paged KV" wiki, section "初始化阶段": the KV memory is cut into N equal
 * physical blocks of shape [block_size, num_kv_heads, head_dim]; the
 * K/V pair and the per-layer factor of that formula are kept as separate
 * per-layer pools here).  A sequence reaches its tokens through a block
 * table: entry j is the physical block that holds its logical block j
 * ("Paged KV", section "运行阶段").  A slot number names one token row of the
 * pool: slot = physical_block * block_size + offset_in_block.
 *
 * Conventions common to every call:
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library allocates no memory and keeps no pointer after the call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns as soon as its kernels are queued.
 *   - Host-checkable mistakes return a negative pkv_status before anything is
 *     launched; pkv_last_error() then describes the mistake.  Launch failures
 *     return PKV_ERR_HIP.
 *   - Device data (slots, block ids, sequence lengths, copy pairs) are checked
 *     in the kernels: an out-of-range value is skipped (never dereferenced) and
 *     recorded in a per-device error word that pkv_check_device_errors() reads.
 *   - Base pointers of caches, K/V rows, q, out and workspace must be 16-byte
 *     aligned; int32/int64 arrays must be naturally aligned.
 *   - Supported: dtype PKV_F32 or PKV_BF16; head_dim 64 or 128; block_size
 *     8, 16, 32 or 64; num_q_heads / num_kv_heads in {1, 2, 4, 8}.  Pools of
 *     PKV_FP8_E4M3 codes have calls of their own (the *_fp8 calls below);
 *     every other call rejects them with PKV_ERR_UNSUPPORTED.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * PKV_FP8_E4M3: one byte per element, the OCP 8-bit E4M3 format (1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; largest finite magnitude 448), with one fp32 scale per (physical
 * block, kv head) for K and one for V: a cached element is
 * scale * value(code).
 */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null/misaligned pointer, negative size, bad shape */
  PKV_ERR_UNSUPPORTED = -2, /* dtype, head_dim, block_size or group not built */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} pkv_status;

/* Shape and element type of one K (and the matching V) block pool. */
typedef struct {
  int64_t num_blocks;   /* physical blocks in each pool */
  int32_t block_size;   /* tokens per block */
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype;        /* pkv_dtype of the stored elements */
} pkv_cache_desc;

/*
 * Slot-mapping scatter ("Paged KV", "运行阶段": each new token's K/V go into the
 * next slot of the sequence's active block; prefill fills blocks in order).
 *
 *   k, v          [num_tokens][num_kv_heads][head_dim], cache->dtype, read.
 *   slot_mapping  [num_tokens] int64; token i is copied bitwise to row
 *                 slot_mapping[i] of both pools; -1 skips the token.  Slots
 *                 must be distinct within one call (else which token lands is
 *                 unspecified); a slot >= num_blocks*block_size is skipped and
 *                 flagged in the device error word.
 *   k_cache, v_cache  the pools, written only at the named slots.
 * num_tokens == 0 is a no-op.
 */
int pkv_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                 int64_t num_tokens, void* k_cache, void* v_cache,
                 const pkv_cache_desc* cache, void* stream);

/*
 * Whole-block copies for copy-on-write of shared blocks ("PagedAttention
 * 动态内存分页", section "写时复制与内存共享": sharers reference the same
 * physical block until one must write, which copies it first).
 *
 *   src_dst_pairs  [num_pairs][2] int64 (src, dst).  For every pair the whole
 *                  K block and the whole V block (all block_size slots) of
 *                  src are copied to dst.  The dsts must be distinct and no
 *                  dst may be a src in the same call, so that every read sees
 *                  the pre-call pool.  Out-of-range ids are skipped and
 *                  flagged in the device error word.
 * num_pairs == 0 is a no-op.
 */
int pkv_block_copy(void* k_cache, void* v_cache, const pkv_cache_desc* cache,
                   const int64_t* src_dst_pairs, int64_t num_pairs, void* stream);

/*
 * Whole-block transfers between two pools of the same block shape, for
 * swapping blocks out of the device pool into host memory and back
 * ("PagedAttention 动态内存分页", section "动态块分配与回收": when device memory
 * runs short, inactive KV blocks are moved to CPU memory and loaded back when
 * they are needed).
 *
 *   dst_k, dst_v  destination pools, laid out as dst_cache describes.
 *   src_k, src_v  source pools, laid out as src_cache describes; read only.
 *                 The two descriptors must agree on block_size, num_kv_heads,
 *                 head_dim and dtype (num_blocks may differ).  Each of the four
 *                 pools is device memory or pinned host memory mapped for the
 *                 device (hipHostMalloc); pageable host memory is rejected with
 *                 PKV_ERR_INVALID_ARG before anything is launched.  Source and
 *                 destination pools must not overlap.
 *   src_dst_pairs [num_pairs][2] int64 (block in the source pools, block in
 *                 the destination pools), device or pinned host memory.  For
 *                 every pair the whole K block and the whole V block are
 *                 copied.  Destinations must be distinct.  Out-of-range ids
 *                 are skipped and flagged in the device error word.
 * num_pairs == 0 is a no-op.  Same-pool copies use pkv_block_copy.
 */
int pkv_block_transfer(void* dst_k, void* dst_v, const pkv_cache_desc* dst_cache,
                       const void* src_k, const void* src_v, const pkv_cache_desc* src_cache,
                       const int64_t* src_dst_pairs, int64_t num_pairs, void* stream);

/*
 * Bytes of device workspace pkv_attention_decode needs for these sizes (0 when
 * none is needed); the arguments mean what they mean for that call.  Returns
 * 0 as well for arguments the call would reject (pkv_last_error() then says
 * why).  Depends on host-known sizes only, so it can size a buffer before any
 * sequence length is known.
 */
size_t pkv_attention_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                     int32_t num_q_heads, int32_t max_blocks_per_seq,
                                     int32_t partition_tokens);

/*
 * Decode-step attention over the paged pools ("Paged KV", section
 * "Attention Kernel 的适配": the kernel takes the block table and block_size
 * in addition, and reads K/V block by block through the table).  For query
 * head h of sequence b, with G = num_q_heads / num_kv_heads and
 * kv = h / G (consecutive grouping):
 *     out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) * V_t
 * over the t < seq_lens[b] tokens reached through block_tables[b].
 * The tokens are split into pieces whose partial results (running max, sum
 * of exponentials, unnormalised output) are merged by max/sum rescaling; the
 * split changes the result only by fp32 rounding.
 *
 *   out           [num_seqs][num_q_heads][head_dim], out_dtype (PKV_F32 or
 *                 PKV_BF16, round to nearest even), written.  A sequence of
 *                 length 0 gets a zero row.
 *   q             [num_seqs][num_q_heads][head_dim], cache->dtype, read.
 *   block_tables  [num_seqs][max_blocks_per_seq] int32, read; only the first
 *                 ceil(seq_lens[b] / block_size) entries of a row are read.
 *   seq_lens      [num_seqs] int32, tokens cached for each sequence (the
 *                 newest included); must be <= max_blocks_per_seq*block_size.
 *   scale         softmax scale applied to the fp32 dot products.
 *   partition_tokens  0 chooses the split: for bf16 pools with head_dim 128
 *                 and at most 2048 sequences, a balanced schedule that gives
 *                 every workgroup about the same share of all the sequences'
 *                 tokens; otherwise partitions of 512 tokens.  A positive value asks
 *                 for partitions of that many tokens: a multiple of 64 and of
 *                 block_size, at most 4096.
 *   workspace     pkv_attention_workspace_bytes(...) bytes of scratch (may be
 *                 NULL when that is 0), overwritten; calls that share a
 *                 workspace must not overlap in time.
 * Pools, q, tables and lengths are only read.  num_seqs == 0 is a no-op.
 */
int pkv_attention_decode(void* out, int32_t out_dtype, const void* q,
                         const void* k_cache, const void* v_cache,
                         const pkv_cache_desc* cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t partition_tokens,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_attention_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, result and errors are those
 * of pkv_attention_decode, whose kernels it runs; the partial results go to
 * a scratch array the library holds per device: 32 MiB (33554432 bytes),
 * placed when the library is loaded on that device and held until the
 * process ends.  The call allocates nothing and calls no allocating routine.
 * Sizes whose pkv_attention_workspace_bytes(...) exceeds 33554432 return
 * PKV_ERR_WORKSPACE before any launch (the batch-256 GQA decode with 32 query
 * heads needs 8.1 MiB, 8 sequences of 32768 tokens with 64 query heads
 * 16.3 MiB with either schedule).
 * The scratch array keeps the last call's contents; nothing in it has to
 * start at zero.  Every call on one device shares that device's array:
 * calls that overlap in time on one device (on different streams, or from
 * different threads without ordering) race and must not be issued.
 */
int pkv_attention_decode_noalloc(void* out, int32_t out_dtype, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const pkv_cache_desc* cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, int32_t num_seqs,
                                 int32_t num_q_heads, float scale, int32_t partition_tokens,
                                 void* stream);

/*
 * Bytes of device workspace pkv_attention_decode_shared (bf16 descriptor) or
 * pkv_attention_decode_shared_fp8 (FP8 descriptor) needs: 0 for arguments
 * that call would reject, with pkv_last_error() saying why, and for
 * num_seqs == 0.  Host-known sizes only.
 */
size_t pkv_attention_shared_workspace_bytes(const pkv_cache_desc* cache, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t num_groups);

/*
 * Decode-step attention for batches in which groups of sequences share a
 * prefix of their cache ("PagedAttention 动态内存分页", section "写时复制与内存
 * 共享": samples or beams forked from one prompt reference the prompt's
 * physical blocks; "Paged KV", section "支持 Prefix Cache": several sequences
 * may hold read-only references to one physical block).  The output is the
 * one pkv_attention_decode computes for the same arguments (up to fp32
 * rounding); the description of the groups only lets the kernels read each
 * shared block once for the whole group instead of once per member.
 *
 * All arguments shared with pkv_attention_decode mean the same; the pools
 * must be PKV_BF16 with head_dim 128 (FP8 pools: the _fp8 variant), and
 * num_seqs <= 2048.
 *   group_offsets [num_groups + 1] int32: the members of group g are
 *                 group_seqs[group_offsets[g] .. group_offsets[g + 1]);
 *                 group_offsets[0] == 0, nondecreasing, last <= num_seqs.
 *   group_seqs    int32 sequence indices in [0, num_seqs); a sequence is a
 *                 member of at most one group, and sequences in no group are
 *                 attended on their own.
 *   group_lens    [num_groups] int32: shared tokens P_g of group g.  Every
 *                 member must map each token t < P_g to the same slot, i.e.
 *                 the first ceil(P_g / block_size) entries of the members'
 *                 block tables are equal, and P_g <= seq_lens of every member.
 *   num_groups    0 <= num_groups <= num_seqs (0: no sharing; the three
 *                 group arrays are then not read and may be NULL).
 *   workspace     pkv_attention_shared_workspace_bytes(...) bytes of scratch,
 *                 overwritten; calls that share a workspace must not overlap.
 * The group description lives in device memory and is checked there: offsets
 * that do not start at 0, decrease or exceed num_seqs make the call ignore
 * the sharing; member ids out of range, a sequence listed twice, a P_g outside
 * [0, seq_len] of a member, or block tables that differ over the shared
 * tokens leave the output unspecified.  Each of these is recorded in the
 * device error word (reported by pkv_check_device_errors); no access leaves
 * the buffers in any case.  num_seqs == 0 is a no-op.
 */
int pkv_attention_decode_shared(void* out, int32_t out_dtype, const void* q,
                                const void* k_cache, const void* v_cache,
                                const pkv_cache_desc* cache,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                                float scale, const int32_t* group_offsets,
                                const int32_t* group_seqs, const int32_t* group_lens,
                                int32_t num_groups, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Prefill attention over the paged pools ("Paged KV", section "运行阶段": at
 * prefill a sequence takes blocks in order and its K/V are filled in, here by
 * pkv_kv_write with one slot per prompt token; section "Attention Kernel 的
 * 适配": K/V are read block by block through the block table).  Sequence b
 * brings n_b = query_start[b + 1] - query_start[b] new tokens, its newest:
 * positions seq_lens[b] - n_b .. seq_lens[b] - 1 (earlier tokens, if any, are
 * cached context, so a long prompt can be processed in chunks).  For query
 * head h of the new token at position p, kv = h / G:
 *     out[row][h] = sum_{t <= p} softmax_t(scale * <q[row][h], K_t>) * V_t
 * over the tokens t = 0 .. p reached through block_tables[b]; with n_b = 1
 * this is the decode step.
 *
 *   out           [num_tokens][num_q_heads][head_dim], out_dtype, written;
 *                 rows outside every sequence's range are not written.
 *   q             [num_tokens][num_q_heads][head_dim], cache->dtype, read.
 *   query_start   [num_seqs + 1] int32, nondecreasing, query_start[0] == 0,
 *                 query_start[num_seqs] <= num_tokens; n_b <= seq_lens[b].
 *                 A sequence whose range breaks this is skipped and flagged in
 *                 the device error word.
 *   block_tables, seq_lens, scale: as for pkv_attention_decode (seq_lens
 *                 counts the new tokens too).
 * The pools must be PKV_BF16 with head_dim 128, and num_seqs <= 2048.  No
 * workspace.  num_seqs == 0 or num_tokens == 0 is a no-op.
 */
int pkv_attention_prefill(void* out, int32_t out_dtype, const void* q, int64_t num_tokens,
                          const int32_t* query_start, const void* k_cache, const void* v_cache,
                          const pkv_cache_desc* cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, void* stream);

/*
 * FP8 KV cache with a scale per block ("Paged KV" wiki, section "局限性": the
 * page names an FP8 KV cache whose scaling factor is kept per block, and notes
 * that such schemes tie the block size to the scale granularity; here the
 * block is the scale group, so every supported block_size works).
 *
 * FP8 pools: k_cache, v_cache laid out as every pool, elements PKV_FP8_E4M3
 * codes (cache->dtype must be PKV_FP8_E4M3; head_dim 64 or 128 for the
 * write and the block moves, 128 for attention).  Scales: k_scale, v_scale
 * [num_blocks][num_kv_heads] fp32, 4-byte aligned, owned by the caller, who
 * sets a block's scales before its first token is written and keeps them
 * while the block holds tokens (a scale is a property of the block, not of
 * the token).
 */

/*
 * Slot-mapping write into FP8 pools.  As pkv_kv_write, except that k and v are
 * [num_tokens][num_kv_heads][head_dim] bf16 and element x of kv head h of a
 * token whose slot lies in block blk is stored as the E4M3 code nearest to
 * the binary32 quotient fl(x / scale[blk][h]) (ties to the even code,
 * magnitudes beyond 448 saturate to 448, NaN stays NaN, -0 keeps its sign).
 * A token row whose scale is not a positive finite number is not written and
 * is flagged in the device error word.  Scales are only read.
 */
int pkv_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping,
                     int64_t num_tokens, void* k_cache, void* v_cache, const float* k_scale,
                     const float* v_scale, const pkv_cache_desc* cache, void* stream);

/*
 * Decode attention over FP8 pools: the result pkv_attention_decode gives for
 * pools holding the dequantized values scale * value(code) (fp32 arithmetic;
 * q is bf16).  All other arguments, the workspace included, mean what they
 * mean for pkv_attention_decode, whose pkv_attention_workspace_bytes sizes
 * the workspace here too (with the FP8 descriptor).  Scales are used as
 * given.
 */
int pkv_attention_decode_fp8(void* out, int32_t out_dtype, const void* q,
                             const void* k_cache, const void* v_cache, const float* k_scale,
                             const float* v_scale, const pkv_cache_desc* cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                             float scale, int32_t partition_tokens, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Prefill attention over FP8 pools: the result pkv_attention_prefill gives
 * for pools holding the dequantized values scale * value(code) (q is bf16).
 * All other arguments mean what they mean for pkv_attention_prefill; the
 * prompt's K/V are written first with pkv_kv_write_fp8.  Scales are used as
 * given.
 */
int pkv_attention_prefill_fp8(void* out, int32_t out_dtype, const void* q, int64_t num_tokens,
                              const int32_t* query_start, const void* k_cache,
                              const void* v_cache, const float* k_scale, const float* v_scale,
                              const pkv_cache_desc* cache, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* seq_lens,
                              int32_t num_seqs, int32_t num_q_heads, float scale, void* stream);

/*
 * Shared-prefix decode over FP8 pools: the result pkv_attention_decode_shared
 * gives for pools holding the dequantized values scale * value(code) (q is
 * bf16), which is also what pkv_attention_decode_fp8 gives on the same
 * arguments.  Every other argument, the group description and the workspace
 * (sized by pkv_attention_shared_workspace_bytes with the FP8 descriptor)
 * included, means what it means for pkv_attention_decode_shared, and is
 * checked the same way.  Blocks shared by a group share their scales too,
 * since a scale belongs to a physical block.  Scales are used as given.
 */
int pkv_attention_decode_shared_fp8(void* out, int32_t out_dtype, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const float* k_scale, const float* v_scale,
                                    const pkv_cache_desc* cache, const int32_t* block_tables,
                                    int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                    int32_t num_seqs, int32_t num_q_heads, float scale,
                                    const int32_t* group_offsets, const int32_t* group_seqs,
                                    const int32_t* group_lens, int32_t num_groups,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_block_copy for FP8 pools: each pair copies the K and V codes of the
 * block and its num_kv_heads K and V scales, so that a copied block decodes
 * to the same values.
 */
int pkv_block_copy_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                       const pkv_cache_desc* cache, const int64_t* src_dst_pairs,
                       int64_t num_pairs, void* stream);

/*
 * pkv_block_transfer for FP8 pools: codes and scales of each pair move
 * together.  The scale arrays follow the rules of their pools (device or
 * pinned host memory, [num_blocks][num_kv_heads] fp32 of their own pool).
 */
int pkv_block_transfer_fp8(void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                           const pkv_cache_desc* dst_cache, const void* src_k, const void* src_v,
                           const float* src_k_scale, const float* src_v_scale,
                           const pkv_cache_desc* src_cache, const int64_t* src_dst_pairs,
                           int64_t num_pairs, void* stream);

/* Message for the last non-OK return on this thread ("" if none). */
const char* pkv_last_error(void);

/*
 * Synchronises `stream`, then reads and clears the current device's error
 * word.  Returns PKV_OK if no kernel recorded a bad slot, block id, sequence
 * length, copy pair, shared-prefix description, prefill query range or FP8
 * scale since the last check;
 * otherwise PKV_ERR_INVALID_ARG with the offending kinds in pkv_last_error().
 */
int pkv_check_device_errors(void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
