"""Host-side block manager: the physical block pool, block tables, reference
counts, copy-on-write decisions and slot mapping.

It holds no attention arithmetic and touches no device memory; it decides
*where* each token goes and which blocks must be copied, and the device calls
(``pkv_kv_write``, ``pkv_block_copy``, ``pkv_attention_decode``) consume its
output.

Sources, by page title and section:

* "Paged KV" (miraclefarms wiki), "初始化阶段": the KV memory is cut into N
  equal physical blocks whose ids start out in a free pool.
* "Paged KV", "运行阶段": every sequence keeps a block table (logical block j
  -> physical block); prefill takes blocks in order; at decode each new token
  goes into the next slot of the active block, and a new block is taken when
  the active one is full.
* "PagedAttention 动态内存分页", "块粒度与块表": the table grows at its tail
  on demand; internal waste is bounded by one block.
* "PagedAttention 动态内存分页", "写时复制与内存共享": sequences forked from one
  prompt share its physical blocks, and a shared block is copied only when a
  sharer must write into it.
* "PagedAttention 动态内存分页", "动态块分配与回收": blocks are taken lazily,
  when a token needs them, and returned to the pool as soon as a sequence ends.
* "Paged KV", "支持 Prefix Cache": several sequences may hold read-only
  references to one physical block; ``shared_prefix_groups`` describes such
  sharing for ``pkv_attention_decode_shared``.
"""
from __future__ import annotations

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["PoolExhausted", "BlockManager"]


class PoolExhausted(RuntimeError):
    """Raised when a block is needed and the free pool is empty."""


class BlockManager:
    """Block pool with per-sequence tables and copy-on-write.

    Parameters
    ----------
    num_blocks:
        Number of physical blocks in the pool.
    block_size:
        Tokens per block.
    free_order:
        Order in which free block ids are handed out (default ``0..N-1``).  A
        seeded permutation here scatters every sequence over the pool.
    """

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Iterable[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks must be >= 0 and block_size > 0")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = list(range(self.num_blocks)) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self._free: deque = deque(order)
        self.refcount: List[int] = [0] * self.num_blocks
        self.tables: Dict[object, List[int]] = {}
        self.lengths: Dict[object, int] = {}
        self.peak_used = 0

    # -- pool -----------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    @property
    def num_used(self) -> int:
        return self.num_blocks - len(self._free)

    def _take(self) -> int:
        if not self._free:
            raise PoolExhausted(f"no free block left in a pool of {self.num_blocks}")
        blk = self._free.popleft()
        assert self.refcount[blk] == 0
        self.refcount[blk] = 1
        self.peak_used = max(self.peak_used, self.num_used)
        return blk

    def _release(self, blk: int) -> None:
        self.refcount[blk] -= 1
        assert self.refcount[blk] >= 0
        if self.refcount[blk] == 0:
            self._free.append(blk)

    # -- sequences ------------------------------------------------------------
    def add_sequence(self, seq_id) -> None:
        if seq_id in self.tables:
            raise KeyError(f"sequence {seq_id!r} exists")
        self.tables[seq_id] = []
        self.lengths[seq_id] = 0

    def fork(self, parent, child) -> None:
        """``child`` starts as a read-only sharer of all of ``parent``'s blocks."""
        if child in self.tables:
            raise KeyError(f"sequence {child!r} exists")
        table = list(self.tables[parent])
        for blk in table:
            self.refcount[blk] += 1
        self.tables[child] = table
        self.lengths[child] = self.lengths[parent]

    def free_sequence(self, seq_id) -> None:
        for blk in self.tables.pop(seq_id):
            self._release(blk)
        del self.lengths[seq_id]

    def append_token(self, seq_id) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the sequence's next token.

        Returns ``(slot, cow)`` where ``slot = block * block_size + offset`` and
        ``cow`` is ``(src, dst)`` when the active block was shared and had to be
        copied before this write, else ``None``.
        """
        table = self.tables[seq_id]
        pos = self.lengths[seq_id]
        bs = self.block_size
        cow = None
        if pos % bs == 0:
            # The active block is full (or there is none yet): take a new one.
            blk = self._take()
            table.append(blk)
        else:
            blk = table[-1]
            if self.refcount[blk] > 1:
                # Shared partial block: copy it, then write into the copy.
                new = self._take()
                cow = (blk, new)
                self.refcount[blk] -= 1
                table[-1] = new
                blk = new
        self.lengths[seq_id] = pos + 1
        return blk * bs + pos % bs, cow

    def append_tokens(self, seq_id, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        slots, cows = [], []
        for _ in range(n):
            s, c = self.append_token(seq_id)
            slots.append(s)
            if c is not None:
                cows.append(c)
        return slots, cows

    # -- views ----------------------------------------------------------------
    def block_table(self, seq_id) -> List[int]:
        return list(self.tables[seq_id])

    def tables_array(self, seq_ids: Sequence, width: Optional[int] = None,
                     pad: int = 0) -> np.ndarray:
        """``[len(seq_ids), width]`` int32 block tables; unused entries = ``pad``."""
        width = max((len(self.tables[s]) for s in seq_ids), default=0) if width is None else width
        out = np.full((len(seq_ids), width), pad, dtype=np.int32)
        for i, s in enumerate(seq_ids):
            t = self.tables[s]
            if len(t) > width:
                raise ValueError("table wider than width")
            out[i, :len(t)] = t
        return out

    def shared_prefix_groups(self, seq_ids: Sequence
                             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """Groups of ``seq_ids`` that share their leading physical blocks.

        Sequences whose first block is the same physical block form a group
        (two members or more, in order of first appearance).  A group's shared
        length is the number of leading table entries that all its members
        have in common, in tokens, capped by its shortest member: every member
        maps each token below it to the same slot.  Returns ``(offsets [G+1],
        members, lens [G])`` as int32 arrays, members being indices into
        ``seq_ids``, the layout ``pkv_attention_decode_shared`` takes.
        """
        by_first: Dict[int, List[int]] = {}
        for i, s in enumerate(seq_ids):
            table = self.tables[s]
            if table:
                by_first.setdefault(table[0], []).append(i)
        offsets, members, lens = [0], [], []
        for idx in by_first.values():
            if len(idx) < 2:
                continue
            tables = [self.tables[seq_ids[i]] for i in idx]
            width = min(len(t) for t in tables)
            k = 0
            while k < width and all(t[k] == tables[0][k] for t in tables):
                k += 1
            shortest = min(self.lengths[seq_ids[i]] for i in idx)
            members.extend(idx)
            offsets.append(len(members))
            lens.append(min(k * self.block_size, shortest))
        return (np.asarray(offsets, np.int32), np.asarray(members, np.int32),
                np.asarray(lens, np.int32))

    def internal_fragmentation(self, seq_id) -> int:
        """Reserved but unused slots of one sequence (at most block_size - 1)."""
        return len(self.tables[seq_id]) * self.block_size - self.lengths[seq_id]
