"""fp64 CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
this module imports nothing from the product package.

What it computes, and where that is defined
-------------------------------------------
Sources are cited by page title and section:

* "Paged KV" (miraclefarms wiki), sections "初始化阶段", "运行阶段",
  "Attention Kernel 的适配", "与 FlashAttention 的关系".
* "PagedAttention 动态内存分页：vLLM 高吞吐推理的 KV Cache 调度实践"
  (hotdry blog), sections "块粒度与块表", "写时复制与内存共享".
* "一文读懂vLLM的“酒店拼房”神技 PagedAttention" (explainer), opening
  paragraphs and "核心原理".

The explainer states that PagedAttention is a KV-cache management scheme and
not a new attention algorithm, so paged decode attention must give exactly the
result of ordinary softmax attention over the same cached tokens.  The oracle
therefore writes that plain definition out in fp64 on the exact input values.

Storage conventions (shared with the callers, not with any GPU code):

* caches are ``[num_blocks, block_size, num_kv_heads, head_dim]`` arrays, one
  for K and one for V (the per-layer reading of the wiki's block shape);
* ``dtype="f32"`` arrays are ``numpy.float32``; ``dtype="bf16"`` arrays are
  ``numpy.uint16`` holding the raw bfloat16 bit patterns; ``dtype="f64"``
  takes values that are already exact binary64 (hand-worked fixtures);
* a slot number is ``physical_block * block_size + offset`` and ``-1`` means
  "skip this token";
* ``block_tables[b, j]`` is the physical block holding logical block ``j`` of
  sequence ``b``; ``seq_lens[b]`` counts the cached tokens, the newest included.

Every function here is pinned against closed forms, brute force and the
pages' definitions by ``tests/test_oracle.py``; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "widen",
    "write_ref",
    "copy_ref",
    "transfer_ref",
    "gather_sequence",
    "softmax_attention",
    "decode_ref",
    "prefill_ref",
    "e4m3_value",
    "e4m3_encode",
    "write_fp8_ref",
    "dequantize_fp8",
    "contiguous_ref",
    "brute_ref",
    "splitk_ref",
]


def widen(x, dtype: str) -> np.ndarray:
    """Exact conversion of stored values to float64.

    bfloat16 is the top half of an IEEE binary32 word, so shifting the 16
    stored bits up by 16 gives the binary32 value exactly; binary32 -> binary64
    is exact as well.
    """
    x = np.asarray(x)
    if dtype == "f64":
        return x.astype(np.float64)
    if dtype == "f32":
        return x.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "bf16":
        if x.dtype != np.uint16:
            raise TypeError("bf16 data must be given as uint16 bit patterns")
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def write_ref(k, v, slot_mapping, k_cache, v_cache) -> None:
    """Slot-mapping scatter, in place on ``k_cache`` / ``v_cache``.

    "Paged KV", "运行阶段": each new token's K and V go into the next slot of
    the sequence's active block.  Token ``i`` is stored at slot
    ``slot_mapping[i]`` = block * block_size + offset; a negative slot skips the
    token.  The copy is bitwise: ``k``/``v`` already have the cache's storage
    type, and no value is converted.
    """
    slots = np.asarray(slot_mapping, dtype=np.int64)
    bs = k_cache.shape[1]
    for i, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        blk, off = divmod(s, bs)
        k_cache[blk, off] = k[i]
        v_cache[blk, off] = v[i]


def copy_ref(k_cache, v_cache, pairs) -> None:
    """Whole-block copy-on-write copies, in place.

    "PagedAttention 动态内存分页", "写时复制与内存共享": sequences that share a
    prefix reference the same physical blocks, and a block is copied only when
    one of the sharers has to write into it.  For every ``(src, dst)`` pair the
    whole K block and the whole V block (all ``block_size`` slots, filled or
    not) are copied.  All reads see the cache as it was before the call.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    snap_k = {int(s): k_cache[int(s)].copy() for s, _ in pairs}
    snap_v = {int(s): v_cache[int(s)].copy() for s, _ in pairs}
    for s, d in pairs.tolist():
        k_cache[d] = snap_k[s]
        v_cache[d] = snap_v[s]


def transfer_ref(dst_k, dst_v, src_k, src_v, pairs) -> None:
    """Whole-block transfers between two pools, in place on ``dst_k`` / ``dst_v``.

    "PagedAttention 动态内存分页", "动态块分配与回收": under memory pressure,
    inactive blocks are swapped out to CPU memory and loaded back when needed.
    For every ``(src, dst)`` pair, block ``src`` of the source pools (all
    ``block_size`` slots, K and V) becomes block ``dst`` of the destination
    pools; nothing else changes.  The pools are distinct, so no read sees a
    write of the same call.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    for s, d in pairs.tolist():
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]


def gather_sequence(cache, table_row, seq_len: int) -> np.ndarray:
    """Logical view of one sequence's cached rows, ``[seq_len, Hkv, D]``.

    "Paged KV", "运行阶段" / "Attention Kernel 的适配": logical block ``j`` of a
    sequence lives in physical block ``table_row[j]``; token ``t`` is slot
    ``t % block_size`` of logical block ``t // block_size``.
    """
    bs = cache.shape[1]
    t = np.arange(seq_len)
    phys = np.asarray(table_row, dtype=np.int64)[t // bs]
    return cache[phys, t % bs]


def softmax_attention(q_vec, keys, values, scale: float) -> np.ndarray:
    """Textbook scaled dot-product attention for one query vector, fp64.

    s_t = scale * <q, k_t>;  out = sum_t exp(s_t - max s) v_t / sum_t exp(s_t - max s).
    With no keys the result is the zero vector.
    """
    if keys.shape[0] == 0:
        return np.zeros(values.shape[-1], dtype=np.float64)
    s = float(scale) * (keys @ q_vec)
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


def decode_ref(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype: str) -> np.ndarray:
    """Paged decode attention, fp64 ``[B, Hq, D]``.

    For query head ``h`` of sequence ``b`` the keys and values are the
    ``seq_lens[b]`` rows reached through ``block_tables[b]`` ("Paged KV",
    "Attention Kernel 的适配": the kernel takes the block table and block size
    and reads K/V block by block).  Query heads map to KV heads in consecutive
    groups, ``kv_head = h // (Hq // Hkv)``.  ``scale`` is used as given (the
    binary32 value the GPU receives, widened).
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        K = widen(gather_sequence(k_cache, block_tables[b], L), dtype)
        V = widen(gather_sequence(v_cache, block_tables[b], L), dtype)
        for h in range(Hq):
            kvh = h // group
            out[b, h] = softmax_attention(qf[b, h], K[:, kvh], V[:, kvh], scale)
    return out


def prefill_ref(q, query_start, k_cache, v_cache, block_tables, seq_lens, scale,
                dtype: str) -> np.ndarray:
    """Paged attention of a prompt (or a chunk of one) over the cache, fp64 ``[T, Hq, D]``.

    "Paged KV", "运行阶段": at prefill a sequence takes blocks in order and its
    K/V are filled in, so the prompt's tokens are in the cache (the write is
    ``write_ref``) before they attend.  Sequence ``b`` owns query rows
    ``query_start[b] .. query_start[b + 1] - 1``: its ``n_b`` newest tokens, at
    positions ``seq_lens[b] - n_b .. seq_lens[b] - 1`` (earlier tokens, if any,
    are context already cached).  The token at position ``p`` attends to the
    cached tokens ``0 .. p``, itself included and nothing after it: the decode
    step is the case ``n_b = 1``.  Attention itself is ``softmax_attention``
    with the consecutive head grouping of ``decode_ref``.
    """
    T, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in range(len(seq_lens)):
        r0, r1 = int(query_start[b]), int(query_start[b + 1])
        L, n = int(seq_lens[b]), r1 - r0
        if n > L:
            raise ValueError(f"sequence {b} has {n} new tokens but only {L} cached")
        K = widen(gather_sequence(k_cache, block_tables[b], L), dtype)
        V = widen(gather_sequence(v_cache, block_tables[b], L), dtype)
        for i in range(n):
            p = L - n + i
            for h in range(Hq):
                kvh = h // group
                out[r0 + i, h] = softmax_attention(qf[r0 + i, h], K[:p + 1, kvh], V[:p + 1, kvh],
                                                   scale)
    return out


# ---------------------------------------------------------------------------- FP8 KV
# "Paged KV", section "局限性": some KV quantization schemes store FP8 with a
# scale per block.  Read here as OCP FP8 E4M3 codes (1 sign, 4 exponent bits
# with bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest finite
# 448) and one fp32 scale per (physical block, kv head), for K and for V: a
# cached element is scale * value(code).

def e4m3_value(code) -> np.ndarray:
    """The real value of each E4M3 code (uint8), fp64; NaN for S.1111.111."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


_E4M3_POS = e4m3_value(np.arange(0x7F))          # codes 0x00 .. 0x7E, increasing


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each (exactly representable fp64) value, uint8.

    Round to nearest, ties to the code with an even mantissa; magnitudes above
    448 saturate to 448; NaN gives S.1111.111.  The nearest grid point is found
    by search over the 127 non-negative finite values, not by bit arithmetic.
    """
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    idx = np.searchsorted(_E4M3_POS, np.minimum(mag, 448.0))     # first grid value >= mag
    hi = np.minimum(idx, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - np.minimum(mag, 448.0)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    code = np.where(mag >= 448.0, 0x7E, np.where(pick_hi, hi, lo)).astype(np.int64)
    code = np.where(np.isnan(x), 0x7F, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def write_fp8_ref(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale) -> None:
    """Slot-mapping write into FP8 pools (uint8 codes), in place.

    Each element x (bf16 bit patterns in ``k``/``v``) of kv head ``h`` of a
    token whose slot lies in block ``blk`` becomes
    ``e4m3_encode(fp32(x / scale[blk, h]))``: the quotient is the binary32
    division of the two binary32 values, the same decision the device takes.
    Negative slots are skipped, as by ``write_ref``.  Tokens are taken in
    order, a run of them at a time: inside a run every token's codes are formed
    at once and a slot named twice keeps its later token, so the result is
    that of writing the tokens one after another.
    """
    bs = k_cache.shape[1]
    ks = np.asarray(k_scale, dtype=np.float32)
    vs = np.asarray(v_scale, dtype=np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    run = 4096
    for r0 in range(0, slots.size, run):
        part = slots[r0:r0 + run]
        rows = np.nonzero(part >= 0)[0]
        # the last occurrence of each slot in the run: the first in reverse
        _, first_rev = np.unique(part[rows][::-1], return_index=True)
        rows = np.sort(rows[::-1][first_rev])
        blk, off = part[rows] // bs, part[rows] % bs
        for src, cache, sc in ((k, k_cache, ks), (v, v_cache, vs)):
            x = widen(np.asarray(src)[r0 + rows], "bf16").astype(np.float32)   # [n, Hkv, D]
            cache[blk, off] = e4m3_encode((x / sc[blk][:, :, None]).astype(np.float64))


def dequantize_fp8(cache, scale) -> np.ndarray:
    """FP8 pool (uint8 codes) -> fp64 values: scale[blk, h] * value(code)."""
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return e4m3_value(cache) * s[:, None, :, None]


def contiguous_ref(q, k_seqs, v_seqs, scale, dtype: str) -> np.ndarray:
    """The same attention over contiguous per-sequence K/V, fp64 ``[B, Hq, D]``.

    ``k_seqs[b]`` / ``v_seqs[b]`` hold sequence ``b``'s tokens in logical order
    as ``[L_b, Hkv, D]`` arrays: the max-length contiguous layout that paging
    replaces ("Paged KV", "问题背景").  No block table is involved.
    """
    B, Hq, D = q.shape
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        K = widen(k_seqs[b], dtype)
        V = widen(v_seqs[b], dtype)
        Hkv = K.shape[1]
        group = Hq // Hkv
        for h in range(Hq):
            out[b, h] = softmax_attention(qf[b, h], K[:, h // group], V[:, h // group], scale)
    return out


def brute_ref(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype: str) -> np.ndarray:
    """Paged decode attention in pure-Python loops (``math.fsum``, ``math.exp``).

    For tiny inputs only.  It walks the block table token by token and shares
    no vectorised step with ``decode_ref``.
    """
    B, Hq, D = q.shape
    bs, Hkv = k_cache.shape[1], k_cache.shape[2]
    group = Hq // Hkv
    qf = widen(q, dtype).tolist()
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        for h in range(Hq):
            kvh = h // group
            scores, vrows = [], []
            for t in range(L):
                blk = int(block_tables[b][t // bs])
                off = t % bs
                krow = widen(k_cache[blk, off, kvh], dtype).tolist()
                vrow = widen(v_cache[blk, off, kvh], dtype).tolist()
                scores.append(float(scale) * math.fsum(a * c for a, c in zip(qf[b][h], krow)))
                vrows.append(vrow)
            if L == 0:
                continue
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            den = math.fsum(w)
            for d in range(D):
                out[b, h, d] = math.fsum(w[t] * vrows[t][d] for t in range(L)) / den
    return out


def splitk_ref(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype: str,
               partition_tokens: int) -> np.ndarray:
    """Decode attention computed per token partition and merged, fp64.

    Each partition ``p`` of ``partition_tokens`` logical tokens keeps its own
    maximum ``m_p``, its sum ``l_p = sum exp(s - m_p)`` and its unnormalised
    output ``a_p = sum exp(s - m_p) v``.  The merge rescales every partition to
    the global maximum ``M``: ``out = sum_p e^(m_p - M) a_p / sum_p e^(m_p - M) l_p``.
    This is the block-wise computation that "Paged KV", "与 FlashAttention 的关系"
    says can be combined with block-wise storage; it is a self-check of the
    rescaling identity, not a second definition.
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        K = widen(gather_sequence(k_cache, block_tables[b], L), dtype)
        V = widen(gather_sequence(v_cache, block_tables[b], L), dtype)
        for h in range(Hq):
            kvh = h // group
            parts = []
            for p0 in range(0, L, partition_tokens):
                s = float(scale) * (K[p0:p0 + partition_tokens, kvh] @ qf[b, h])
                m_p = s.max()
                e = np.exp(s - m_p)
                parts.append((m_p, e.sum(), e @ V[p0:p0 + partition_tokens, kvh]))
            M = max(m for m, _, _ in parts)
            num = sum(math.exp(m - M) * a for m, _, a in parts)
            den = sum(math.exp(m - M) * l for m, l, _ in parts)
            out[b, h] = num / den
    return out
