"""Seeded synthetic workloads for the paged decode path.

This module only draws inputs: sequence lengths, the physical block pool and
its free order, block tables and slot numbers (through ``BlockManager``), and
the Q/K/V values.  It holds none of the attention, write or copy arithmetic,
and it is the one piece of code that both the GPU path's callers and the
oracle's callers use, so that both see identical inputs.

Five decode workloads are defined, each named by what it is:

1. ``tiny_mha``: fp32, 4 sequences of lengths {5, 17, 32, 40}, 2 q heads = 2 kv
   heads, head_dim 64, block_size 16, a pool of 16 blocks handed out in a
   seeded random order, scale 1/sqrt(64).
2. ``llama7b_mha``: bf16, 64 sequences, lengths uniform on [128, 2048],
   32 q = 32 kv heads, head_dim 128, block_size 16.
3. ``llama3_8b_gqa``: bf16, 256 sequences, lengths lognormal (median 1024,
   sigma 1 in log space) clipped to [16, 8192], 32 q / 8 kv heads, head_dim 128,
   block_size 16.
4. ``long_context``: bf16, 8 sequences of 32768 tokens, 64 q / 8 kv heads,
   head_dim 128, block_size 32 or 64; 1% of K rows are multiplied by 8 to
   stretch the softmax range.
5. ``prefix_sharing``: bf16, 4 prompts x 8 samples, 32 q / 8 kv heads,
   head_dim 128, block_size 8 or 16; each prompt's prefix blocks are shared by
   its 8 samples, which then grow 256-token tails (``PrefixSharingWorkload``).

Recipe (numpy ``default_rng(seed)``, draws in this order): lengths; the free
order of the pool (a permutation); q; K; V; the outlier mask.  Values are
binary32 normal draws rounded to bfloat16 with round-to-nearest-even for the
bf16 workloads.  Pool size is ceil(1.1 * blocks needed) unless fixed.

FP8 pools take the same tokens; their per-(block, kv head) scales follow the
usual max-abs calibration (``fp8_block_scales``): the largest magnitude among
the tokens a block will hold, divided by 448 (the largest E4M3 value), so
that no element saturates.  The scales are inputs of the write, chosen here
as a caller would choose them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .block_manager import BlockManager

__all__ = [
    "CONFIGS",
    "bf16_round",
    "DecodeWorkload",
    "make_decode_workload",
    "PrefixSharingWorkload",
    "PrefillWorkload",
    "fp8_block_scales",
]


def bf16_round(x) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Input generation only.  The inputs never hold NaN or infinity.  Works in
    chunks with in-place integer steps so that the full-size pools (10^9
    values) round in seconds.
    """
    src = np.ascontiguousarray(x, dtype=np.float32)
    flat = src.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape, dtype=np.uint16)
    tmp = np.empty(min(flat.size, _CHUNK), dtype=np.uint32)
    for s in range(0, flat.size, _CHUNK):
        bits = flat[s:s + _CHUNK]
        t = tmp[:bits.size]
        np.right_shift(bits, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        np.add(t, 0x7FFF, out=t)
        np.add(t, bits, out=t)
        np.right_shift(t, 16, out=t)
        out[s:s + _CHUNK] = t
    return out.reshape(src.shape)


_CHUNK = 1 << 22


@dataclass(frozen=True)
class ConfigSpec:
    name: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seed: int
    lengths: str            # "fixed", "uniform", "lognormal"
    fixed_lens: Sequence[int] = ()
    num_blocks: Optional[int] = None
    k_outlier_frac: float = 0.0
    k_outlier_mult: float = 8.0


CONFIGS: Dict[int, ConfigSpec] = {
    1: ConfigSpec("tiny_mha", "f32", 4, 2, 2, 64, 16, 1, "fixed", (5, 17, 32, 40), num_blocks=16),
    2: ConfigSpec("llama7b_mha", "bf16", 64, 32, 32, 128, 16, 2, "uniform"),
    3: ConfigSpec("llama3_8b_gqa", "bf16", 256, 32, 8, 128, 16, 3, "lognormal"),
    4: ConfigSpec("long_context", "bf16", 8, 64, 8, 128, 32, 4, "fixed", (32768,) * 8,
                  k_outlier_frac=0.01),
    5: ConfigSpec("prefix_sharing", "bf16", 32, 32, 8, 128, 16, 5, "prefix"),
}


def _normal(rng, shape, dtype: str) -> np.ndarray:
    """binary32 standard normal draws, rounded to bfloat16 for ``"bf16"``.

    Drawn in consecutive chunks from ``rng``; the values equal those of one
    ``rng.standard_normal(shape, dtype=np.float32)`` call.
    """
    if dtype == "f32":
        return rng.standard_normal(shape, dtype=np.float32)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = bf16_round(rng.standard_normal(m, dtype=np.float32))
    return out.reshape(shape)


def _draw_lengths(spec: ConfigSpec, rng, num_seqs: int) -> np.ndarray:
    if spec.lengths == "fixed":
        lens = np.array(list(spec.fixed_lens)[:num_seqs], dtype=np.int64)
        if len(lens) < num_seqs:
            lens = np.resize(lens, num_seqs)
        return lens
    if spec.lengths == "uniform":
        return rng.integers(128, 2048, size=num_seqs, endpoint=True).astype(np.int64)
    if spec.lengths == "lognormal":
        z = rng.standard_normal(num_seqs)
        return np.clip(np.rint(1024.0 * np.exp(z)), 16, 8192).astype(np.int64)
    raise ValueError(spec.lengths)


def fp8_block_scales(k, v, slots, num_blocks: int, block_size: int, unused=np.nan):
    """Per-(block, kv head) fp32 scales of an FP8 pool for the bf16 tokens
    ``k``/``v`` ``[N, Hkv, D]`` written to ``slots`` ``[N]`` (-1: not written):
    max |x| over the block's tokens of that head / 448, 1.0 where that max is 0,
    ``unused`` for blocks that receive no token.  Returns (k_scale, v_scale),
    each ``[num_blocks, Hkv]`` float32.  Input preparation only.
    """
    slots = np.asarray(slots, dtype=np.int64)
    Hkv = k.shape[1]
    res = []
    for x in (k, v):
        amax = np.full((num_blocks, Hkv), -1.0, np.float32)
        for s in range(0, len(slots), 1 << 14):
            part = np.ascontiguousarray(x[s:s + (1 << 14)])
            mag = np.abs((part.astype(np.uint32) << np.uint32(16)).view(np.float32)).max(axis=2)
            sl = slots[s:s + (1 << 14)]
            ok = sl >= 0
            np.maximum.at(amax, sl[ok] // block_size, mag[ok])
        sc = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0))
        res.append(np.where(amax < 0, np.float32(unused), sc).astype(np.float32))
    return res[0], res[1]


@dataclass
class DecodeWorkload:
    """One decode step: prefill state, the step's writes, then attention.

    ``k_tokens``/``v_tokens`` hold every sequence's tokens in logical order,
    concatenated (``cu_seqlens`` delimits them); the last token of each
    sequence is the one this step writes.  ``prefill_rows``/``prefill_slots``
    put all earlier tokens into the pool, ``step_rows``/``step_slots`` the new
    ones.
    """
    name: str
    dtype: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: np.float32
    seq_lens: np.ndarray
    cu_seqlens: np.ndarray
    q: np.ndarray
    k_tokens: np.ndarray
    v_tokens: np.ndarray
    block_tables: np.ndarray
    prefill_rows: np.ndarray
    prefill_slots: np.ndarray
    step_rows: np.ndarray
    step_slots: np.ndarray
    copy_pairs: np.ndarray
    fresh_blocks_in_step: int = 0
    manager: Optional[BlockManager] = field(default=None, repr=False)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def seq_tokens(self, b: int):
        """Logical ``[L_b, Hkv, D]`` K and V of sequence ``b`` (views)."""
        s, e = int(self.cu_seqlens[b]), int(self.cu_seqlens[b + 1])
        return self.k_tokens[s:e], self.v_tokens[s:e]

    def empty_caches(self, fill: str = "nan"):
        """Host K and V pools; unused slots hold NaN (``"nan"``) or zero."""
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        if self.dtype == "f32":
            val = np.float32(np.nan) if fill == "nan" else np.float32(0)
            return np.full(shape, val, np.float32), np.full(shape, val, np.float32)
        val = 0x7FC0 if fill == "nan" else 0
        return np.full(shape, val, np.uint16), np.full(shape, val, np.uint16)

    def slot_of_row(self) -> np.ndarray:
        """Slot of every token row (prefill and step), int64 ``[T]``."""
        out = np.full(self.k_tokens.shape[0], -1, np.int64)
        out[self.prefill_rows] = self.prefill_slots
        out[self.step_rows] = self.step_slots
        return out

    def fp8_scales(self, unused=np.nan):
        """``fp8_block_scales`` of this workload's tokens (bf16 workloads)."""
        return fp8_block_scales(self.k_tokens, self.v_tokens, self.slot_of_row(), self.num_blocks,
                                self.block_size, unused)

    def kv_bytes(self) -> int:
        """K+V bytes the decode step must read: sum_b L_b * Hkv * D * 2 * elem."""
        return int(self.seq_lens.sum()) * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes


def make_decode_workload(config: int, *, block_size: Optional[int] = None,
                         num_seqs: Optional[int] = None,
                         seq_lens: Optional[Sequence[int]] = None,
                         seed: Optional[int] = None,
                         table_pad: int = 0,
                         heads: Optional[Sequence[int]] = None,
                         head_dim: Optional[int] = None,
                         dtype: Optional[str] = None) -> DecodeWorkload:
    """Build decode workload ``config`` (1-4), optionally resized.

    ``seq_lens`` replaces the length draw (the draw is still made so that the
    later draws do not move); ``num_seqs`` changes the batch; ``heads``
    (q heads, kv heads), ``head_dim`` and ``dtype`` reshape it for parity cases.
    """
    spec = CONFIGS[config]
    if heads is not None or head_dim is not None or dtype is not None:
        import dataclasses
        hq, hkv = heads if heads is not None else (spec.num_q_heads, spec.num_kv_heads)
        spec = dataclasses.replace(spec, num_q_heads=int(hq), num_kv_heads=int(hkv),
                                   head_dim=spec.head_dim if head_dim is None else int(head_dim),
                                   dtype=spec.dtype if dtype is None else dtype)
    if spec.lengths == "prefix":
        raise ValueError("use PrefixSharingWorkload for the prefix-sharing workload")
    bs = spec.block_size if block_size is None else int(block_size)
    seed = spec.seed if seed is None else int(seed)
    B = spec.num_seqs if num_seqs is None else int(num_seqs)
    if seq_lens is not None:
        B = len(seq_lens)
    rng = np.random.default_rng(seed)
    lens = _draw_lengths(spec, rng, B)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
    if (lens < 1).any():
        raise ValueError("every sequence holds at least its new token")
    need = int(sum(math.ceil(int(L) / bs) for L in lens))
    NB = spec.num_blocks if (spec.num_blocks is not None and block_size is None
                             and seq_lens is None and num_seqs is None) else math.ceil(1.1 * need)
    NB = max(NB, need)
    order = rng.permutation(NB)
    mgr = BlockManager(NB, bs, order)
    Hq, Hkv, D = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    cu = np.zeros(B + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])

    prefill_rows, prefill_slots = [], []
    for b in range(B):
        mgr.add_sequence(b)
        slots, cows = mgr.append_tokens(b, int(lens[b]) - 1)
        assert not cows
        prefill_rows.append(np.arange(cu[b], cu[b + 1] - 1))
        prefill_slots.append(np.asarray(slots, dtype=np.int64))
    step_slots, fresh = [], 0
    for b in range(B):
        fresh += int((int(lens[b]) - 1) % bs == 0)
        s, cow = mgr.append_token(b)
        assert cow is None
        step_slots.append(s)

    q = _normal(rng, (B, Hq, D), spec.dtype)
    k = _normal(rng, (T, Hkv, D), spec.dtype)
    v = _normal(rng, (T, Hkv, D), spec.dtype)
    if spec.k_outlier_frac > 0:
        mask = rng.random((T, Hkv)) < spec.k_outlier_frac
        if spec.dtype == "bf16":
            kf = (k[mask].astype(np.uint32) << np.uint32(16)).view(np.float32)
            k[mask] = bf16_round(kf * np.float32(spec.k_outlier_mult))
        else:
            k[mask] = k[mask] * np.float32(spec.k_outlier_mult)

    width = max(math.ceil(int(L) / bs) for L in lens)
    return DecodeWorkload(
        name=spec.name, dtype=spec.dtype, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, num_blocks=NB,
        scale=np.float32(1.0 / math.sqrt(D)),
        seq_lens=lens.astype(np.int32), cu_seqlens=cu, q=q, k_tokens=k, v_tokens=v,
        block_tables=mgr.tables_array(list(range(B)), width=width, pad=table_pad),
        prefill_rows=np.concatenate(prefill_rows) if prefill_rows else np.zeros(0, np.int64),
        prefill_slots=np.concatenate(prefill_slots) if prefill_slots else np.zeros(0, np.int64),
        step_rows=(cu[1:] - 1).astype(np.int64), step_slots=np.asarray(step_slots, np.int64),
        copy_pairs=np.zeros((0, 2), np.int64), fresh_blocks_in_step=fresh, manager=mgr)


@dataclass
class SharingStep:
    """Inputs of one decode step of the prefix-sharing workload."""
    step: int
    q: np.ndarray               # [B, Hq, D]
    k_new: np.ndarray           # [B, Hkv, D]: the token each sample writes
    v_new: np.ndarray
    slot_mapping: np.ndarray    # [B] int64
    copy_pairs: np.ndarray      # [n, 2] int64, to run before the writes
    block_tables: np.ndarray    # [B, MB] int32
    seq_lens: np.ndarray        # [B] int32


class PrefixSharingWorkload:
    """Parallel sampling over shared prompt prefixes.

    ``prompts`` prompts of ``prefix_len`` tokens are prefilled once each; every
    prompt is forked into ``samples`` sequences that reference the prompt's
    blocks (reference count = samples).  Step ``s`` (1-based) has every sample
    write its token at position ``prefix_len + s - 1`` and then attend over
    ``prefix_len + s`` tokens.  When the last prefix block is only partly full,
    the first step copies it for every sharer but the last, which writes in
    place ("PagedAttention 动态内存分页", "写时复制与内存共享").
    """

    def __init__(self, prefix_len: int = 2044, tail_len: int = 256, block_size: int = 16,
                 prompts: int = 4, samples: int = 8, seed: int = 5,
                 num_q_heads: int = 32, num_kv_heads: int = 8, head_dim: int = 128):
        self.prefix_len, self.tail_len, self.block_size = prefix_len, tail_len, block_size
        self.prompts, self.samples, self.seed = prompts, samples, seed
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.dtype = "bf16"
        self.scale = np.float32(1.0 / math.sqrt(head_dim))
        self.num_seqs = prompts * samples
        # Size the pool by a dry run of the whole schedule, then add 10%.
        dry = BlockManager(10 ** 7, block_size)
        self._schedule(dry, run_steps=tail_len)
        self.blocks_needed = dry.peak_used
        self.num_blocks = math.ceil(1.1 * self.blocks_needed)
        rng = np.random.default_rng(seed)
        self._order = rng.permutation(self.num_blocks)
        Hkv, D = num_kv_heads, head_dim
        self.prefix_k = _normal(rng, (prompts, prefix_len, Hkv, D), "bf16")
        self.prefix_v = _normal(rng, (prompts, prefix_len, Hkv, D), "bf16")
        self.tail_k = _normal(rng, (self.num_seqs, tail_len, Hkv, D), "bf16")
        self.tail_v = _normal(rng, (self.num_seqs, tail_len, Hkv, D), "bf16")
        self.width = math.ceil((prefix_len + tail_len) / block_size)
        self.reset()

    def _schedule(self, mgr: BlockManager, run_steps: int):
        for p in range(self.prompts):
            mgr.add_sequence((p, 0))
            mgr.append_tokens((p, 0), self.prefix_len)
            for j in range(1, self.samples):
                mgr.fork((p, 0), (p, j))
        for _ in range(run_steps):
            for p in range(self.prompts):
                for j in range(self.samples):
                    mgr.append_token((p, j))

    def reset(self) -> None:
        """Start over from an empty pool (same seeded free order)."""
        self.manager = BlockManager(self.num_blocks, self.block_size, self._order)
        self.steps_done = 0
        self._prefilled = False

    @property
    def seq_ids(self) -> List:
        return [(p, j) for p in range(self.prompts) for j in range(self.samples)]

    def prefill(self):
        """Prefill every prompt once; returns ``(k [4P,Hkv,D], v, slots [4P])``."""
        assert not self._prefilled
        slots = []
        for p in range(self.prompts):
            self.manager.add_sequence((p, 0))
            s, cows = self.manager.append_tokens((p, 0), self.prefix_len)
            assert not cows
            slots.extend(s)
            for j in range(1, self.samples):
                self.manager.fork((p, 0), (p, j))
        self._prefilled = True
        Hkv, D = self.num_kv_heads, self.head_dim
        return (self.prefix_k.reshape(-1, Hkv, D), self.prefix_v.reshape(-1, Hkv, D),
                np.asarray(slots, dtype=np.int64))

    def next_step(self) -> SharingStep:
        assert self._prefilled and self.steps_done < self.tail_len
        s = self.steps_done + 1
        slots, pairs = [], []
        for sid in self.seq_ids:
            slot, cow = self.manager.append_token(sid)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        self.steps_done = s
        rng = np.random.default_rng((self.seed, s))
        q = bf16_round(rng.standard_normal((self.num_seqs, self.num_q_heads, self.head_dim),
                                           dtype=np.float32))
        return SharingStep(
            step=s, q=q, k_new=self.tail_k[:, s - 1].copy(), v_new=self.tail_v[:, s - 1].copy(),
            slot_mapping=np.asarray(slots, dtype=np.int64),
            copy_pairs=np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
            block_tables=self.manager.tables_array(self.seq_ids, width=self.width),
            seq_lens=np.full(self.num_seqs, self.prefix_len + s, dtype=np.int32))

    def logical_tokens(self, b: int, length: int):
        """Sample ``b``'s first ``length`` tokens in logical order (K, V)."""
        p = b // self.samples
        n_tail = length - self.prefix_len
        k = np.concatenate([self.prefix_k[p], self.tail_k[b, :n_tail]])
        v = np.concatenate([self.prefix_v[p], self.tail_v[b, :n_tail]])
        return k, v

    def empty_caches(self, fill: str = "nan"):
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        val = 0x7FC0 if fill == "nan" else 0
        return np.full(shape, val, np.uint16), np.full(shape, val, np.uint16)


class PrefillWorkload:
    """Prompts (or prompt chunks after cached context) in a paged pool.

    Sequence ``b`` holds ``context[b] + new[b]`` tokens, placed by a block
    manager over a seeded free order ("Paged KV", "运行阶段": prefill takes
    blocks in order).  All tokens' K/V are written with one slot mapping
    (``slots``, rows of ``k_tokens``/``v_tokens`` in sequence order); the
    ``new[b]`` newest tokens of each sequence are the query rows ``q`` split by
    ``query_start``.  Values are standard normals rounded to bf16.
    """

    def __init__(self, context, new, block_size: int = 16, num_q_heads: int = 32,
                 num_kv_heads: int = 8, head_dim: int = 128, seed: int = 7):
        context, new = [int(c) for c in context], [int(n) for n in new]
        if len(context) != len(new):
            raise ValueError("context and new must have one entry per sequence")
        self.block_size, self.head_dim = block_size, head_dim
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.dtype = "bf16"
        self.scale = np.float32(1.0 / math.sqrt(head_dim))
        self.num_seqs = len(new)
        self.seq_lens = np.array([c + n for c, n in zip(context, new)], dtype=np.int32)
        self.query_start = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        self.num_tokens = int(self.query_start[-1])
        rng = np.random.default_rng(seed)
        need = sum(-(-int(L) // block_size) for L in self.seq_lens)
        self.num_blocks = max(1, math.ceil(1.1 * need))
        self.manager = BlockManager(self.num_blocks, block_size, rng.permutation(self.num_blocks))
        slots = []
        for b, L in enumerate(self.seq_lens):
            self.manager.add_sequence(b)
            s, _ = self.manager.append_tokens(b, int(L))
            slots.extend(s)
        self.slots = np.asarray(slots, dtype=np.int64)
        total = int(self.seq_lens.sum())
        Hkv, D = num_kv_heads, head_dim
        self.k_tokens = _normal(rng, (total, Hkv, D), "bf16")
        self.v_tokens = _normal(rng, (total, Hkv, D), "bf16")
        self.q = _normal(rng, (self.num_tokens, num_q_heads, D), "bf16")
        width = max(1, max(-(-int(L) // block_size) for L in self.seq_lens))
        self.block_tables = self.manager.tables_array(list(range(self.num_seqs)), width=width)

    def empty_caches(self, fill: str = "nan"):
        shape = (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)
        val = 0x7FC0 if fill == "nan" else 0
        return np.full(shape, val, np.uint16), np.full(shape, val, np.uint16)

    def flops(self) -> int:
        """Multiply-adds x 2 of Q.K^T and P.V: 4 D Hq (p + 1) per new token at position p."""
        total = 0
        for b in range(self.num_seqs):
            n = int(self.query_start[b + 1] - self.query_start[b])
            L = int(self.seq_lens[b])
            total += sum(L - n + i + 1 for i in range(n))
        return 4 * self.head_dim * self.num_q_heads * total


# ---------------------------------------------------------------------------- device upload
def torch_tensor(a: np.ndarray, dtype: str, device):
    """Host array -> device tensor; bf16 bit patterns become torch.bfloat16 bit for bit."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def empty_device_caches(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
                        dtype: str, device, fill: str = "nan"):
    """Device K and V pools filled with NaN (bf16 0x7FC0 / fp32 0x7FC00000) or zeros."""
    import torch
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    val = float("nan") if fill == "nan" else 0.0
    shape = (num_blocks, block_size, num_kv_heads, head_dim)
    return torch.full(shape, val, dtype=tdt, device=device), torch.full(shape, val, dtype=tdt, device=device)


def host_bits(t) -> np.ndarray:
    """Device tensor -> host array in the oracle's storage convention (uint16 for bf16)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
