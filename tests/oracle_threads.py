"""The fp64 oracle over many sequences at once, on a thread pool.

Test infrastructure: this only splits a call of the oracle into calls over
single sequences (or single query rows, or disjoint runs of tokens) and runs
them on threads; every value still comes from ``oracle``.  NumPy's fp64
kernels release the interpreter lock, so the pieces run in parallel, and BLAS
is held to one thread per worker so that the workers do not oversubscribe the
cores.  The pool takes the cores this process may run on, at most 16 (the CPU
share of one GPU on the boxes the GPU tests run on).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

try:
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None

MAX_WORKERS = 16


def workers() -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def _map(fn, items):
    items = list(items)
    if threadpool_limits is not None:
        with threadpool_limits(limits=1), ThreadPoolExecutor(workers()) as ex:
            return list(ex.map(fn, items))
    with ThreadPoolExecutor(workers()) as ex:
        return list(ex.map(fn, items))


def decode_rows(q, k_cache, v_cache, block_tables, seq_lens, scale, dtype, rows=None):
    """``oracle.decode_ref`` of the sequences ``rows`` (default: all), one call
    per sequence; returns ``[len(rows), Hq, D]`` fp64."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    if rows.size == 0:
        return np.zeros((0,) + q.shape[1:], np.float64)

    def one(b):
        return oracle.decode_ref(q[b:b + 1], k_cache, v_cache, block_tables[b:b + 1],
                                 seq_lens[b:b + 1], scale, dtype)[0]

    return np.stack(_map(one, rows.tolist()))


def decode_fp8_rows(q_bits, k_codes, v_codes, k_scale, v_scale, block_tables, seq_lens, scale,
                    rows=None):
    """``oracle.decode_ref`` over ``oracle.dequantize_fp8`` of FP8 pools, one
    sequence at a time: each sequence's blocks are dequantized on their own
    (with their scales) and renumbered in table order, so no whole pool is
    widened to fp64.  ``q_bits`` are bf16 bit patterns."""
    rows = np.arange(q_bits.shape[0]) if rows is None else np.asarray(rows)
    bs = k_codes.shape[1]

    def one(b):
        L = int(seq_lens[b])
        nblk = -(-L // bs)
        blocks = np.asarray(block_tables[b, :nblk], np.int64)
        kd = oracle.dequantize_fp8(k_codes[blocks], k_scale[blocks])
        vd = oracle.dequantize_fp8(v_codes[blocks], v_scale[blocks])
        table = np.arange(max(nblk, 1), dtype=np.int32)[None]
        return oracle.decode_ref(oracle.widen(q_bits[b:b + 1], "bf16"), kd, vd, table,
                                 np.array([L], np.int32), scale, "f64")[0]

    return np.stack(_map(one, rows.tolist()))


def write_fp8(k, v, slots, k_cache, v_cache, k_scale, v_scale, parts=64):
    """``oracle.write_fp8_ref`` of ``parts`` consecutive runs of tokens, on
    threads.  The slots must be distinct (then the runs touch disjoint slots
    and their order does not matter)."""
    slots = np.asarray(slots, np.int64)
    live = slots[slots >= 0]
    if np.unique(live).size != live.size:
        raise ValueError("write_fp8 on threads needs distinct slots")
    pieces = [p for p in np.array_split(np.arange(slots.size), parts) if p.size]

    def one(p):
        oracle.write_fp8_ref(k[p], v[p], slots[p], k_cache, v_cache, k_scale, v_scale)

    _map(one, pieces)


def prefill_rows(q, query_start, k_cache, v_cache, block_tables, seq_lens, scale, dtype, rows):
    """``oracle.prefill_ref`` of the query rows ``rows``, each its own call: the
    row of token ``i`` of sequence ``b`` is the one-token prefill at position
    ``seq_lens[b] - n_b + i``."""
    rows = np.asarray(rows)
    seq_of = np.searchsorted(query_start, rows, side="right") - 1

    def one(rb):
        r, b = rb
        n = int(query_start[b + 1] - query_start[b])
        i = int(r - query_start[b])
        L = int(seq_lens[b]) - n + i + 1          # the token's own position + 1
        return oracle.prefill_ref(q[r:r + 1], np.array([0, 1]), k_cache, v_cache,
                                  block_tables[b:b + 1], np.array([L]), scale, dtype)[0]

    return np.stack(_map(one, zip(rows.tolist(), seq_of.tolist())))
