"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--block-size BS]
    python bench.py --report-all      # one line per workload, then the metric line
    python bench.py --read-probe      # plain streaming read: the practical HBM rate
    python bench.py --copy-probe      # 1 GiB device copy (counter calibration)

A step is one pass of the hot path over one batch: the slot-mapping write of
every sequence's new token (pkv_kv_write), then decode attention over all
cached tokens (pkv_attention_decode: the balanced-schedule kernel and the
reduce of the sequences it cuts).  For the prefix-sharing workload the step
also holds the copy-on-write block copies of its first divergent step.  The
default workload is the batch-256 Llama-3-8B-shaped GQA decode (32 q / 8 kv
heads, head_dim 128, block_size 16, lognormal lengths, median 1024, clipped to
[16, 8192]; seed 3), synthetic bf16 data resident in HBM.

Cache honesty: the step rotates over several identical copies of the KV pool
(--pools, default 3), so that no step finds the previous step's blocks in the
L2 / MALL caches (the prefix-sharing pool, 67 MB of unique K/V, is
cache-resident by nature and is reported as such).

The default run prints one JSON line: value = KV GB/s of the whole step (KV
bytes the step's attention must read / step time), plus the attention-only
rate, tokens/s, a roofline entry for the decode call and the fp64 CPU oracle
timed on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attn KV GB/s (% of HBM peak) + tokens/s, GQA batch 256"
COUNTERS = os.path.join(ROOT, "profiles", "decode_balanced_llama3_8b_gqa_b256_hbm_counters.md")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--block-size", type=int, default=None)
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--pools", type=int, default=3)
    p.add_argument("--prefix", type=int, default=2044, help="prefix-sharing workload: prompt tokens")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate budget of the CPU oracle sample")
    p.add_argument("--report-cpu-seconds", type=float, default=4.0,
                   help="approximate budget of the CPU oracle sample of each --report-all line")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--report-all", action="store_true",
                   help="one line per workload (config 2, 4 at bs 32/64 with the balanced schedule "
                        "and with 512-token partitions, 5 at bs 8/16, FP8, prefill), then the "
                        "metric line")
    p.add_argument("--only", default=None,
                   help="only these --report-all lines, comma-separated: fp8, prefill, mha, "
                        "long32, long32_p512, long64, long64_p512, swap, sharing4, sharing64 "
                        "(for profiling one kernel's workload)")
    p.add_argument("--read-probe", action="store_true",
                   help="only time a plain streaming read of 4 GiB (context for the roofline)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    p.add_argument("--fp8", action="store_true",
                   help="only the batch-256 GQA decode step over FP8 E4M3 pools")
    p.add_argument("--prefill", action="store_true",
                   help="only time paged prefill (prompt write + causal attention) workloads")
    p.add_argument("--counter-pass", action="store_true",
                   help="only run 4 decode calls of the workload (a 1 GiB write between calls "
                        "evicts the pool from the caches), then 3 streaming reads of 2 GiB: "
                        "a short program for hardware-counter passes")
    return p.parse_args()


def copy_probe(torch):
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def read_probe(torch):
    """Plain streaming read of 4 GiB with the streaming hint, several grid sizes."""
    import ctypes
    from paged_kv_cache_330_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build with `python -m paged_kv_cache_330_amd.build`")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    buf = torch.ones(4 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for blocks in (8192, 16384, 32768, 65536):
        ts = []
        for _ in range(12):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if lib.pkv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                         ctypes.c_void_p(sink.data_ptr()), blocks, stream) != 0:
                raise RuntimeError("stream probe launch failed")
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[blocks] = round(buf.numel() / (statistics.median(ts[2:]) * 1e-3) / 1e9, 1)
    print(json.dumps({"read_probe_bytes": buf.numel(), "gbps_by_workgroups": res,
                      "best_gbps": max(res.values()),
                      "best_frac_of_peak": round(max(res.values()) / HBM_PEAK_GBPS, 4)}), flush=True)
    del buf
    torch.cuda.empty_cache()
    paged_read_probe(torch, lib, sink, stream)


def paged_read_probe(torch, lib, sink, stream):
    """The metric workload's K/V blocks, read in block-table order with the
    decode kernels' wave layout and no compute: what the decode could reach
    if its compute and bookkeeping cost nothing."""
    import ctypes
    import numpy as np
    from paged_kv_cache_330_amd.workloads import empty_device_caches, make_decode_workload
    lib.pkv_probe_paged_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    w = make_decode_workload(3)
    bs, hkv = w.block_size, w.num_kv_heads
    order = np.concatenate([w.block_tables[b, :-(-int(L) // bs)]
                            for b, L in enumerate(w.seq_lens)]).astype(np.int32)
    assert order.min() >= 0 and order.max() < w.num_blocks
    ids = torch.from_numpy(order).cuda()
    pools = []
    for _ in range(2):
        kc, vc = empty_device_caches(w.num_blocks, bs, hkv, w.head_dim, "bf16", "cuda", fill="zero")
        kc.normal_()
        vc.normal_()
        pools.append((kc, vc))
    nbytes = len(order) * bs * hkv * w.head_dim * 2 * 2
    res = {}
    for wgs in (256, 512, 1024):
        ts = []
        for i in range(12):
            kc, vc = pools[i % 2]
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if lib.pkv_probe_paged_read(ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
                                        ctypes.c_void_p(ids.data_ptr()), len(order), bs, hkv,
                                        ctypes.c_void_p(sink.data_ptr()), wgs, stream) != 0:
                raise RuntimeError("paged read probe launch failed")
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        res[wgs] = round(nbytes / (statistics.median(ts[2:]) * 1e-3) / 1e9, 1)
    print(json.dumps({"paged_read_probe": w.name, "blocks": len(order), "bytes": nbytes,
                      "gbps_by_workgroups": res, "best_gbps": max(res.values()),
                      "best_frac_of_peak": round(max(res.values()) / HBM_PEAK_GBPS, 4)}), flush=True)


def counter_pass(torch, args):
    """Four decode calls and three plain streaming reads, nothing else timed."""
    import ctypes
    from paged_kv_cache_330_amd import ops
    from paged_kv_cache_330_amd.build import PROBE_LIB
    from paged_kv_cache_330_amd.workloads import make_decode_workload
    ops.load_library()
    w = make_decode_workload(args.config, block_size=args.block_size)
    st = decode_step_state(torch, ops, w, 1, args.partition_tokens)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for i in range(4):
        flush.fill_(i)
        st.run(0)
    torch.cuda.synchronize()
    ops.pkv_check_device_errors()
    del st, flush
    lib = ctypes.CDLL(PROBE_LIB)
    lib.pkv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        if lib.pkv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                     ctypes.c_void_p(sink.data_ptr()), 65536, stream) != 0:
            raise RuntimeError("stream probe launch failed")
    torch.cuda.synchronize()
    print(json.dumps({"counter_pass": "done", "workload": w.name}), flush=True)


def measured_traffic():
    """HBM bytes per decode call from the committed counter summary, or None.

    The summary records the sha256 of the library sources it was taken with;
    when the sources have changed since, the figure no longer describes the
    kernels and None is returned.
    """
    import re
    from paged_kv_cache_330_amd.build import source_digest
    try:
        text = open(COUNTERS).read()
    except OSError:
        return None
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    val = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not sha or not val or sha.group(1) != source_digest():
        return None
    return int(val.group(1))


# The GPU machines give one GPU a share of 16 host cores (more may be visible):
# the oracle's thread pool takes the cores this process may run on, at most 16.
ORACLE_MAX_THREADS = 16


def _oracle_threads():
    cores = len(os.sched_getaffinity(0))
    return max(1, min(ORACLE_MAX_THREADS, cores)), cores


def _time_oracle(units, weights, one, budget_s, per_pass=None):
    """Times the fp64 oracle on a bounded sample.

    ``one(u)`` runs the oracle on work unit ``u`` (a sequence, a query row);
    ``weights`` are the units' relative costs (tokens).  A one-unit
    calibration sizes the sample: the first ``n`` units that fill about
    ``budget_s`` seconds on the thread pool; when all units take less, whole
    passes repeat until the budget is spent.  ``per_pass(units)`` runs first
    in every pass (the step's writes and copies).  Returns
    (n, passes, seconds, threads, visible cores)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    threads, cores = _oracle_threads()
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        one(units[0])
        per_w = (time.perf_counter() - t0) / max(1, int(weights[0]))
        cum = np.cumsum(np.asarray(weights, dtype=np.int64))
        target = budget_s * threads / max(per_w, 1e-9)
        n = int(min(len(units), max(threads, np.searchsorted(cum, target) + 1)))
        sample = units[:n]
        passes = 0
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=threads) as ex:
            while True:
                if per_pass is not None:
                    per_pass(sample)
                list(ex.map(one, sample))
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= budget_s or n < len(units):
                    break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    return n, passes, dt, threads, cores


def _baseline_entry(value, unit, n, passes, dt, threads, cores, sample, **extra):
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "host_cpus_visible": cores,
            "thread_cap": ORACLE_MAX_THREADS, **extra}


def cpu_baseline(w, budget_s):
    """The fp64 oracle on a bounded sample of decode workload ``w``.

    A pass is ``write_ref`` of the step's new tokens of sequences 0..n-1
    followed by ``decode_ref`` of those sequences (one call per sequence on
    the thread pool); KV GB/s counts the K/V bytes the sample's attention
    reads, as the GPU figure does."""
    import oracle

    kc, vc = w.empty_caches("zero")
    t0 = time.perf_counter()
    oracle.write_ref(w.k_tokens[w.prefill_rows], w.v_tokens[w.prefill_rows], w.prefill_slots, kc, vc)
    prefill_s = time.perf_counter() - t0

    def one(r):
        return oracle.decode_ref(w.q[r:r + 1], kc, vc, w.block_tables[r:r + 1],
                                 w.seq_lens[r:r + 1], w.scale, w.dtype)

    def per_pass(rows):
        oracle.write_ref(w.k_tokens[w.step_rows[rows]], w.v_tokens[w.step_rows[rows]],
                         w.step_slots[rows], kc, vc)

    n, passes, dt, threads, cores = _time_oracle(list(range(w.num_seqs)), w.seq_lens, one,
                                                 budget_s, per_pass)
    tokens = int(w.seq_lens[:n].sum())
    kv = passes * tokens * w.num_kv_heads * w.head_dim * 2 * w.elem_bytes
    return _baseline_entry(
        round(kv / dt / 1e9, 4), "GB/s", n, passes, dt, threads, cores,
        (f"{passes} pass(es) of write_ref of {n} new tokens + decode_ref of sequences "
         f"0..{n - 1} ({tokens} of {int(w.seq_lens.sum())} cached tokens) of the same "
         f"workload, fp64 NumPy, {threads} threads, {dt:.1f} s (prefill write_ref of "
         f"the pool, untimed: {prefill_s:.1f} s)"),
        tokens_per_s=round(passes * n / dt, 3))


def cpu_baseline_fp8(w, ks, vs, budget_s):
    """The fp64 oracle on a bounded sample of decode workload ``w`` over FP8
    pools: a pass is ``write_fp8_ref`` of the new tokens of sequences 0..n-1,
    then per sequence ``dequantize_fp8`` of its blocks and ``decode_ref``.
    KV GB/s counts 1 byte per cached element, as the GPU figure does."""
    import numpy as np
    import oracle

    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    kc, vc = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    t0 = time.perf_counter()
    oracle.write_fp8_ref(w.k_tokens[w.prefill_rows], w.v_tokens[w.prefill_rows], w.prefill_slots,
                         kc, vc, ks, vs)
    prefill_s = time.perf_counter() - t0
    q = oracle.widen(w.q, "bf16")

    def one(r):
        L = int(w.seq_lens[r])
        nblk = -(-L // w.block_size)
        blocks = w.block_tables[r, :nblk].astype(np.int64)
        kd = oracle.dequantize_fp8(kc[blocks], ks[blocks])
        vd = oracle.dequantize_fp8(vc[blocks], vs[blocks])
        return oracle.decode_ref(q[r:r + 1], kd, vd, np.arange(nblk, dtype=np.int32)[None],
                                 w.seq_lens[r:r + 1], w.scale, "f64")

    def per_pass(rows):
        oracle.write_fp8_ref(w.k_tokens[w.step_rows[rows]], w.v_tokens[w.step_rows[rows]],
                             w.step_slots[rows], kc, vc, ks, vs)

    n, passes, dt, threads, cores = _time_oracle(list(range(w.num_seqs)), w.seq_lens, one,
                                                 budget_s, per_pass)
    tokens = int(w.seq_lens[:n].sum())
    kv = passes * tokens * w.num_kv_heads * w.head_dim * 2
    return _baseline_entry(
        round(kv / dt / 1e9, 4), "GB/s", n, passes, dt, threads, cores,
        (f"{passes} pass(es) of write_fp8_ref of {n} new tokens + dequantize_fp8 and "
         f"decode_ref of sequences 0..{n - 1} ({tokens} of {int(w.seq_lens.sum())} cached "
         f"tokens), fp64 NumPy, {threads} threads, {dt:.1f} s (prefill write_fp8_ref of the "
         f"pool, untimed: {prefill_s:.1f} s)"),
        tokens_per_s=round(passes * n / dt, 3))


def cpu_baseline_sharing(prefix, bs, prompts, final, budget_s):
    """The fp64 oracle on the prefix-sharing workload at its first divergent
    step or its last: the pool is built by the oracle's own writes and copies
    of every earlier step (untimed); a pass is the step's ``copy_ref`` and
    ``write_ref`` and ``decode_ref`` of sequences 0..n-1.  The oracle has one
    definition of attention: the same pass serves the plain and the
    shared-prefix decode.  KV GB/s counts the logical bytes every sequence
    reads."""
    import oracle
    from paged_kv_cache_330_amd.workloads import PrefixSharingWorkload

    ws = PrefixSharingWorkload(prefix_len=prefix, block_size=bs, prompts=prompts)
    kc, vc = ws.empty_caches("zero")
    t0 = time.perf_counter()
    pk, pv, ps = ws.prefill()
    oracle.write_ref(pk, pv, ps, kc, vc)
    st = ws.next_step()
    while final and ws.steps_done < ws.tail_len:
        oracle.copy_ref(kc, vc, st.copy_pairs)
        oracle.write_ref(st.k_new, st.v_new, st.slot_mapping, kc, vc)
        st = ws.next_step()
    build_s = time.perf_counter() - t0

    def one(r):
        return oracle.decode_ref(st.q[r:r + 1], kc, vc, st.block_tables[r:r + 1],
                                 st.seq_lens[r:r + 1], ws.scale, "bf16")

    def per_pass(rows):
        oracle.copy_ref(kc, vc, st.copy_pairs)
        oracle.write_ref(st.k_new[rows], st.v_new[rows], st.slot_mapping[rows], kc, vc)

    n, passes, dt, threads, cores = _time_oracle(list(range(ws.num_seqs)), st.seq_lens, one,
                                                 budget_s, per_pass)
    tokens = int(st.seq_lens[:n].sum())
    kv = passes * tokens * ws.num_kv_heads * ws.head_dim * 2 * 2
    return _baseline_entry(
        round(kv / dt / 1e9, 4), "GB/s", n, passes, dt, threads, cores,
        (f"{passes} pass(es) of copy_ref of {len(st.copy_pairs)} pairs + write_ref of {n} new "
         f"tokens + decode_ref of sequences 0..{n - 1} ({tokens} logical tokens) at step "
         f"{ws.steps_done}, fp64 NumPy, {threads} threads, {dt:.1f} s (pool built by the "
         f"oracle, untimed: {build_s:.1f} s)"),
        tokens_per_s=round(passes * n / dt, 3))


def cpu_baseline_swap(blocks, budget_s, chunk=64):
    """The oracle's ``transfer_ref`` on the block-swap workload: a device-shaped
    pool of 2 * ``blocks`` blocks and a host pool of ``blocks`` (bs 16, 8 kv
    heads, head_dim 128, bf16 bit patterns, which a transfer moves unchanged).
    A unit is ``chunk`` pairs swapped out and then back in; GB/s counts the K+V
    bytes moved, both directions together, as the GPU figure ``swap_gbps``."""
    import numpy as np
    import oracle

    rng = np.random.default_rng(11)
    shape = (blocks * 2, 16, 8, 128)
    kc = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
    hk = np.empty((blocks,) + shape[1:], dtype=np.uint16)
    hv = np.empty_like(hk)
    src = rng.permutation(blocks * 2)[:blocks]
    pairs = np.stack([src, np.arange(blocks)], 1)
    units = [pairs[i:i + chunk] for i in range(0, blocks, chunk)]

    def one(u):
        oracle.transfer_ref(hk, hv, kc, vc, u)
        oracle.transfer_ref(kc, vc, hk, hv, u[:, ::-1])

    n, passes, dt, threads, cores = _time_oracle(units, [len(u) for u in units], one, budget_s)
    moved = passes * 2 * sum(len(u) for u in units[:n]) * 2 * 16 * 8 * 128 * 2
    return _baseline_entry(
        round(moved / dt / 1e9, 4), "GB/s", n, passes, dt, threads, cores,
        (f"{passes} pass(es) of transfer_ref out and back in of {n} chunks of {chunk} "
         f"blocks ({min(blocks, n * chunk)} of {blocks}), {threads} threads, {dt:.1f} s"))


def cpu_baseline_prefill(w, budget_s, rows_wanted=4096):
    """The fp64 oracle on a bounded sample of prefill workload ``w``: a pass is
    ``write_ref`` of every prompt token, then ``prefill_ref`` of an evenly
    strided sample of query rows (each row its own one-token call at its
    position).  TFLOP/s counts the algorithmic flops of the sampled rows."""
    import numpy as np
    import oracle

    kc, vc = w.empty_caches("zero")
    stride = max(1, w.num_tokens // rows_wanted)
    rows = np.arange(0, w.num_tokens, stride)
    rng = np.random.default_rng(0)
    rows = rows[rng.permutation(rows.size)]          # the sample's prefix spans all positions
    seq_of = np.searchsorted(w.query_start, rows, side="right") - 1
    pos = np.array([int(w.seq_lens[b]) - int(w.query_start[b + 1] - w.query_start[b])
                    + int(r - w.query_start[b]) for r, b in zip(rows, seq_of)])

    def one(i):
        r, b = int(rows[i]), int(seq_of[i])
        return oracle.prefill_ref(w.q[r:r + 1], np.array([0, 1]), kc, vc, w.block_tables[b:b + 1],
                                  np.array([pos[i] + 1]), w.scale, "bf16")

    def per_pass(_):
        oracle.write_ref(w.k_tokens, w.v_tokens, w.slots, kc, vc)

    n, passes, dt, threads, cores = _time_oracle(list(range(rows.size)), pos + 1, one, budget_s,
                                                 per_pass)
    flops = passes * 4 * w.head_dim * w.num_q_heads * int((pos[:n] + 1).sum())
    return _baseline_entry(
        round(flops / dt / 1e12, 6), "TFLOP/s", n, passes, dt, threads, cores,
        (f"{passes} pass(es) of write_ref of all {len(w.slots)} prompt tokens + prefill_ref of "
         f"{n} query rows (every {stride}th row, shuffled, each at its own position), fp64 "
         f"NumPy, {threads} threads, {dt:.1f} s"),
        prompt_tokens_per_s=round(passes * n / dt, 3))


# --------------------------------------------------------------------------- device state
class Step:
    """Device tensors of one decode step and the phases that run it."""

    def __init__(self, torch, ops, pools, q, bt, sl, k_new, v_new, slots, pairs, scale,
                 partition_tokens, groups=None, fp8_scales=None):
        self.torch, self.ops = torch, ops
        self.fp8 = fp8_scales  # (k_scale, v_scale) device tensors: FP8 pools
        self.pools, self.q, self.bt, self.sl = pools, q, bt, sl
        self.k_new, self.v_new, self.slots, self.pairs = k_new, v_new, slots, pairs
        self.scale, self.part = scale, partition_tokens
        self.groups = groups  # (offsets, members, lens) device tensors: shared-prefix decode
        B, Hq, D = q.shape
        kc, vc = pools[0]
        self.out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
        if groups is None:
            need = ops.pkv_attention_workspace_bytes(kc, vc, B, Hq, bt.shape[1], partition_tokens)
        else:
            need = ops.pkv_attention_shared_workspace_bytes(kc, vc, B, Hq, groups[2].shape[0])
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)

    def decode_only(self, i):
        """The decode call of step i alone (no copies, no write)."""
        kc, vc = self.pools[i % len(self.pools)]
        if self.fp8 is not None and self.groups is not None:
            ks, vs = self.fp8
            self.ops.pkv_attention_decode_shared_fp8(self.out, self.q, kc, vc, ks, vs, self.bt,
                                                     self.sl, self.scale, *self.groups,
                                                     workspace=self.ws)
        elif self.fp8 is not None:
            ks, vs = self.fp8
            self.ops.pkv_attention_decode_fp8(self.out, self.q, kc, vc, ks, vs, self.bt, self.sl,
                                              self.scale, self.part, self.ws)
        elif self.groups is None:
            self.ops.pkv_attention_decode(self.out, self.q, kc, vc, self.bt, self.sl, self.scale,
                                          self.part, self.ws)
        else:
            self.ops.pkv_attention_decode_shared(self.out, self.q, kc, vc, self.bt, self.sl,
                                                 self.scale, *self.groups, workspace=self.ws)

    def run(self, i, ev=None):
        """Copies (if any), write, decode on pool copy i; ev = 4 events or None."""
        kc, vc = self.pools[i % len(self.pools)]
        if ev:
            ev[0].record()
        if self.fp8 is not None:
            ks, vs = self.fp8
            if self.pairs is not None:
                self.ops.pkv_block_copy_fp8(kc, vc, ks, vs, self.pairs)
            if ev:
                ev[1].record()
            self.ops.pkv_kv_write_fp8(self.k_new, self.v_new, self.slots, kc, vc, ks, vs)
            if ev:
                ev[2].record()
            if self.groups is None:
                self.ops.pkv_attention_decode_fp8(self.out, self.q, kc, vc, ks, vs, self.bt,
                                                  self.sl, self.scale, self.part, self.ws)
            else:
                self.ops.pkv_attention_decode_shared_fp8(self.out, self.q, kc, vc, ks, vs,
                                                         self.bt, self.sl, self.scale,
                                                         *self.groups, workspace=self.ws)
            if ev:
                ev[3].record()
            return
        if self.pairs is not None:
            self.ops.pkv_block_copy(kc, vc, self.pairs)
        if ev:
            ev[1].record()
        self.ops.pkv_kv_write(self.k_new, self.v_new, self.slots, kc, vc)
        if ev:
            ev[2].record()
        if self.groups is None:
            self.ops.pkv_attention_decode(self.out, self.q, kc, vc, self.bt, self.sl, self.scale,
                                          self.part, self.ws)
        else:
            self.ops.pkv_attention_decode_shared(self.out, self.q, kc, vc, self.bt, self.sl,
                                                 self.scale, *self.groups, workspace=self.ws)
        if ev:
            ev[3].record()


def decode_step_state(torch, ops, w, npools, partition_tokens):
    """Pools holding the prefill of decode workload `w`, and its step."""
    from paged_kv_cache_330_amd.workloads import empty_device_caches, torch_tensor
    dev = "cuda"
    kt, vt = torch_tensor(w.k_tokens, w.dtype, dev), torch_tensor(w.v_tokens, w.dtype, dev)
    pre = torch.from_numpy(w.prefill_rows).to(dev)
    pre_slots = torch.from_numpy(w.prefill_slots).to(dev)
    k_pre, v_pre = kt[pre].contiguous(), vt[pre].contiguous()
    step = torch.from_numpy(w.step_rows).to(dev)
    k_new, v_new = kt[step].contiguous(), vt[step].contiguous()
    del kt, vt
    pools = []
    for _ in range(npools):
        kc, vc = empty_device_caches(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                     w.dtype, dev, fill="zero")
        ops.pkv_kv_write(k_pre, v_pre, pre_slots, kc, vc)
        pools.append((kc, vc))
    del k_pre, v_pre
    return Step(torch, ops, pools, torch_tensor(w.q, w.dtype, dev),
                torch.from_numpy(w.block_tables).to(dev), torch.from_numpy(w.seq_lens).to(dev),
                k_new, v_new, torch.from_numpy(w.step_slots).to(dev), None, float(w.scale),
                partition_tokens)


def fp8_step_state(torch, ops, w, npools, partition_tokens):
    """FP8 pools (E4M3 codes, max-abs block scales) holding the prefill of
    decode workload `w`, and its step."""
    from paged_kv_cache_330_amd.workloads import torch_tensor
    dev = "cuda"
    ks_h, vs_h = w.fp8_scales(unused=1.0)
    ks, vs = torch.from_numpy(ks_h).to(dev), torch.from_numpy(vs_h).to(dev)
    kt, vt = torch_tensor(w.k_tokens, "bf16", dev), torch_tensor(w.v_tokens, "bf16", dev)
    pre = torch.from_numpy(w.prefill_rows).to(dev)
    pre_slots = torch.from_numpy(w.prefill_slots).to(dev)
    k_pre, v_pre = kt[pre].contiguous(), vt[pre].contiguous()
    step = torch.from_numpy(w.step_rows).to(dev)
    k_new, v_new = kt[step].contiguous(), vt[step].contiguous()
    del kt, vt
    shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
    pools = []
    for _ in range(npools):
        kc = torch.zeros(shape, dtype=torch.uint8, device=dev)
        vc = torch.zeros(shape, dtype=torch.uint8, device=dev)
        ops.pkv_kv_write_fp8(k_pre, v_pre, pre_slots, kc, vc, ks, vs)
        pools.append((kc, vc))
    del k_pre, v_pre
    return Step(torch, ops, pools, torch_tensor(w.q, "bf16", dev),
                torch.from_numpy(w.block_tables).to(dev), torch.from_numpy(w.seq_lens).to(dev),
                k_new, v_new, torch.from_numpy(w.step_slots).to(dev), None, float(w.scale),
                partition_tokens, fp8_scales=(ks, vs))


def sharing_step_state(torch, ops, ws, final, partition_tokens, shared=False, fp8=False):
    """Pool of the prefix-sharing workload at its first divergent step (with its
    copy-on-write copies) or at its last step; returns (Step, seq_lens).  With
    `shared` the step decodes with pkv_attention_decode_shared, the groups
    taken from the block manager.  With `fp8` the pools hold E4M3 codes: each
    prompt block's scales are its own max-abs / 448, every other block's the
    prompts' overall max-abs / 448 (the tails are drawn from the same
    distribution)."""
    import numpy as np
    from paged_kv_cache_330_amd.workloads import (empty_device_caches, fp8_block_scales,
                                                  torch_tensor)
    dev = "cuda"
    pk, pv, ps = ws.prefill()
    if fp8:
        shape = (ws.num_blocks, ws.block_size, ws.num_kv_heads, ws.head_dim)
        kc = torch.zeros(shape, dtype=torch.uint8, device=dev)
        vc = torch.zeros(shape, dtype=torch.uint8, device=dev)
        sc = []
        for s in fp8_block_scales(pk, pv, ps, ws.num_blocks, ws.block_size):
            s[np.isnan(s)] = np.nanmax(s)
            sc.append(torch.from_numpy(s).to(dev))
        fp8_scales = tuple(sc)

        def write(k, v, slots):
            ops.pkv_kv_write_fp8(k, v, slots, kc, vc, *fp8_scales)

        def copy(pairs):
            ops.pkv_block_copy_fp8(kc, vc, *fp8_scales, pairs)
    else:
        kc, vc = empty_device_caches(ws.num_blocks, ws.block_size, ws.num_kv_heads, ws.head_dim,
                                     "bf16", dev, fill="zero")
        fp8_scales = None

        def write(k, v, slots):
            ops.pkv_kv_write(k, v, slots, kc, vc)

        def copy(pairs):
            ops.pkv_block_copy(kc, vc, pairs)
    write(torch_tensor(pk, "bf16", dev), torch_tensor(pv, "bf16", dev),
          torch.from_numpy(ps).to(dev))
    st = ws.next_step()
    while final and ws.steps_done < ws.tail_len:  # apply every step but the last
        if len(st.copy_pairs):
            copy(torch.from_numpy(st.copy_pairs).to(dev))
        write(torch_tensor(st.k_new, "bf16", dev), torch_tensor(st.v_new, "bf16", dev),
              torch.from_numpy(st.slot_mapping).to(dev))
        st = ws.next_step()
    pairs = torch.from_numpy(st.copy_pairs).to(dev) if len(st.copy_pairs) else None
    groups = None
    if shared:
        groups = tuple(torch.from_numpy(a).to(dev)
                       for a in ws.manager.shared_prefix_groups(ws.seq_ids))
    step = Step(torch, ops, [(kc, vc)], torch_tensor(st.q, "bf16", dev),
                torch.from_numpy(st.block_tables).to(dev), torch.from_numpy(st.seq_lens).to(dev),
                torch_tensor(st.k_new, "bf16", dev), torch_tensor(st.v_new, "bf16", dev),
                torch.from_numpy(st.slot_mapping).to(dev), pairs, float(ws.scale),
                partition_tokens, groups, fp8_scales=fp8_scales)
    return step, st.seq_lens


def time_steps(torch, step, steps, warmup):
    """Warm up, then time exactly `steps` steps between two synchronisations;
    then run the same `steps` steps again with stream events around each phase
    for the per-phase times.  The wall time comes from the first pass, which
    has no events between its launches (each event is a command of its own on
    the stream).

    Re-running a step is idempotent: its copies, writes and decode see the same
    pool contents every time."""
    for i in range(warmup):
        step.run(i)
    torch.cuda.synchronize()
    step.ops.pkv_check_device_errors()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step.ops.pkv_check_device_errors()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step.run(warmup + steps + i, events[i])
    torch.cuda.synchronize()
    step.ops.pkv_check_device_errors()
    ms = lambda a, b: [e[a].elapsed_time(e[b]) for e in events]  # noqa: E731
    return wall, ms(0, 1), ms(1, 2), ms(2, 3)


def time_decode_calls(torch, step, calls, first):
    """Mean duration (ms) of `calls` back-to-back decode calls on the rotating
    pools, from two events on the stream the calls run on (torch's current
    stream, which the binding passes to the library) around all of them."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(calls):
        step.decode_only(first + i)
    e1.record()
    torch.cuda.synchronize()
    step.ops.pkv_check_device_errors()
    return e0.elapsed_time(e1) / calls


def attn_bytes(seq_lens, B, Hq, Hkv, D, bs, es):
    """Algorithmic bytes of one decode call: K/V rows, q, fp32 out, table entries, lengths."""
    kv = int(sum(int(L) for L in seq_lens)) * Hkv * D * 2 * es
    entries = int(sum(math.ceil(int(L) / bs) for L in seq_lens))
    return kv, kv + B * Hq * D * es + B * Hq * D * 4 + 4 * entries + 4 * B


def attn_bytes_fp8(seq_lens, B, Hq, Hkv, D, bs):
    """Algorithmic bytes of one FP8 decode call: 1-byte K/V codes, a K and a V
    fp32 scale per (table entry, kv head), bf16 q, fp32 out, table entries,
    lengths."""
    kv = int(sum(int(L) for L in seq_lens)) * Hkv * D * 2
    entries = int(sum(math.ceil(int(L) / bs) for L in seq_lens))
    return kv, kv + 8 * entries * Hkv + B * Hq * D * 2 + B * Hq * D * 4 + 4 * entries + 4 * B


def _pct(xs, p):
    import numpy as np
    return float(np.percentile(xs, p))


def summary(name, extra, seq_lens, B, Hq, Hkv, D, bs, steps, wall, t_copy, t_write, t_attn,
            n_pairs=0, es=2):
    """Figures of one timed workload (`es` bytes per stored element)."""
    kv, alg = attn_bytes(seq_lens, B, Hq, Hkv, D, bs, es)
    attn_ms = statistics.median(t_attn)
    ms_per_step = wall * 1e3 / steps
    row = Hkv * D * es
    res = {
        "workload": name, **extra, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
        "head_dim": D, "block_size": bs, "seq_len_sum": int(sum(int(L) for L in seq_lens)),
        "ms_per_step": round(ms_per_step, 4),
        "t_attn_us": {"median": round(attn_ms * 1e3, 2),
                      "p10": round(_pct(t_attn, 10) * 1e3, 2),
                      "p90": round(_pct(t_attn, 90) * 1e3, 2)},
        "attn_kv_gbps": round(kv / (attn_ms * 1e-3) / 1e9, 2),
        "attn_hbm_frac": round(kv / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "attn_alg_gbps": round(alg / (statistics.mean(t_attn) * 1e-3) / 1e9, 2),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "attn_tokens_per_s": round(B / (attn_ms * 1e-3), 1),
        "t_write_us": round(statistics.median(t_write) * 1e3, 2),
        "write_gbps": round((2 * 2 * B * row + 8 * B) / (statistics.median(t_write) * 1e-3) / 1e9, 2),
    }
    if n_pairs:
        cb = 2 * 2 * n_pairs * bs * row + 16 * n_pairs
        res["t_copy_us"] = round(statistics.median(t_copy) * 1e3, 2)
        res["copy_pairs"] = n_pairs
        res["copy_gbps"] = round(cb / (statistics.median(t_copy) * 1e-3) / 1e9, 2)
    return res, kv, alg


def swap_report(torch, ops, args, blocks=2048, reps=5):
    """Swap 2048 blocks of the batch-256 GQA pool shape (bs 16, 8 kv heads,
    head_dim 128, bf16: 64 KiB of K+V per block) out to pinned host memory and
    back in, with pkv_block_transfer; GB/s of K+V moved each way."""
    dev = "cuda"
    shape = (blocks * 2, 16, 8, 128)
    kc = torch.randn(shape, device=dev).to(torch.bfloat16)
    vc = torch.randn(shape, device=dev).to(torch.bfloat16)
    hk = torch.empty((blocks, 16, 8, 128), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    src = torch.randperm(blocks * 2, device=dev)[:blocks]
    out_pairs = torch.stack([src, torch.arange(blocks, device=dev)], 1).contiguous()
    in_pairs = torch.stack([torch.arange(blocks, device=dev), src], 1).contiguous()
    nbytes = 2 * blocks * 16 * 8 * 128 * 2
    res = {"workload": "block_swap", "blocks": blocks, "bytes_each_way": nbytes}
    for name, call in (("out", lambda: ops.pkv_block_transfer(hk, hv, kc, vc, out_pairs)),
                       ("in", lambda: ops.pkv_block_transfer(kc, vc, hk, hv, in_pairs))):
        call()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ops.pkv_check_device_errors()
        ms = statistics.median(ts)
        res[f"swap_{name}_us"] = round(ms * 1e3, 1)
        res[f"swap_{name}_gbps"] = round(nbytes / (ms * 1e-3) / 1e9, 2)
    res["swap_gbps"] = round(2 * nbytes / ((res["swap_out_us"] + res["swap_in_us"]) * 1e-6) / 1e9, 2)
    with_baseline(res, args, cpu_baseline_swap, blocks, gpu_key="swap_gbps")
    print(json.dumps({"report": res}), flush=True)
    del kc, vc, hk, hv
    torch.cuda.empty_cache()


def with_baseline(res, args, fn, *a, gpu_key="attn_kv_gbps"):
    """Adds the oracle timed on the host (unless --no-cpu-baseline) to a report line."""
    if not args.no_cpu_baseline:
        base = fn(*a, args.report_cpu_seconds)
        res["cpu_baseline"] = base
        res["gpu_over_cpu"] = round(res[gpu_key] / base["value"], 1)
    return res


def report_all(torch, ops, args, only=None):
    """One JSON line per workload other than the metric's (shorter runs), each
    with the oracle timed beside it on the host; `only`: the names of the
    lines to run (all when None)."""
    want = lambda name: only is None or name in only  # noqa: E731
    if want("fp8"):
        fp8_report(torch, ops, args)
    if want("prefill"):
        prefill_report(torch, ops, args)
    from paged_kv_cache_330_amd.workloads import PrefixSharingWorkload, make_decode_workload
    steps, warmup = 20, 3
    # the Llama-7B MHA batch; the long-context batch at both block sizes, with
    # the balanced schedule and with its stated 512-token partitions (64 per
    # sequence, merged by the split-K reduce)
    for name, config, bs, part in (("mha", 2, None, 0), ("long32", 4, 32, 0),
                                   ("long32_p512", 4, 32, 512), ("long64", 4, 64, 0),
                                   ("long64_p512", 4, 64, 512)):
        if not want(name):
            continue
        w = make_decode_workload(config, block_size=bs)
        st = decode_step_state(torch, ops, w, args.pools, part)
        wall, t_copy, t_write, t_attn = time_steps(torch, st, steps, warmup)
        res, _, alg = summary(w.name, {"seed": w.seed}, w.seq_lens, w.num_seqs, w.num_q_heads,
                              w.num_kv_heads, w.head_dim, w.block_size, steps, wall, t_copy,
                              t_write, t_attn)
        res["schedule"] = "balanced" if part == 0 else f"partitions of {part} tokens"
        t_call = time_decode_calls(torch, st, steps, 3 * steps)
        res["mean_call_us"] = round(t_call * 1e3, 2)
        res["call_alg_hbm_frac"] = round(alg / (t_call * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        del st
        torch.cuda.empty_cache()
        print(json.dumps({"report": with_baseline(res, args, cpu_baseline, w)}), flush=True)
    if want("swap"):
        swap_report(torch, ops, args)
    # the prefix-sharing workload as stated (4 prompts x 8 samples) at both
    # block sizes, first divergent and last step; then 64 prompts x 8 samples
    # (512 sequences, 1.07 GB of unique K/V, 4.8 GB read by the plain decode),
    # also over FP8 pools
    cases = [(4, bs, final) for bs in (8, 16) for final in (False, True)] + [(64, 16, True)]
    sharing_baselines = {}
    for prompts, bs, final in cases:
        if not want(f"sharing{prompts}"):
            continue
        kinds = [(False, False), (True, False)]
        if prompts == 64:
            kinds += [(False, True), (True, True)]
        for shared, fp8 in kinds:
            ws = PrefixSharingWorkload(prefix_len=args.prefix, block_size=bs, prompts=prompts)
            st, lens = sharing_step_state(torch, ops, ws, final, args.partition_tokens,
                                          shared, fp8)
            wall, t_copy, t_write, t_attn = time_steps(torch, st, steps, warmup)
            n_pairs = 0 if st.pairs is None else int(st.pairs.shape[0])
            name = "prefix_sharing_shared_decode" if shared else "prefix_sharing"
            es = 1 if fp8 else 2
            extra = {"prompts": prompts, "samples": ws.samples, "prefix": args.prefix,
                     "step": ws.steps_done, "seed": ws.seed}
            if fp8:
                name += "_fp8_e4m3"
                extra["kv_dtype"] = "fp8_e4m3"
            res, kv, _ = summary(
                name, extra, lens, ws.num_seqs, ws.num_q_heads, ws.num_kv_heads, ws.head_dim, bs,
                steps, wall, t_copy, t_write, t_attn, n_pairs, es=es)
            if fp8:  # bf16 K/V in, 1-byte codes out, slots and scales read
                B, rowe = ws.num_seqs, ws.num_kv_heads * ws.head_dim
                wb = B * rowe * 2 * (2 + 1) + 8 * B + 2 * 4 * B * ws.num_kv_heads
                res["write_gbps"] = round(wb / (statistics.median(t_write) * 1e-3) / 1e9, 2)
            # K/V bytes held once: the prompts' prefixes and every sample's own tail
            unique = (ws.prompts * ws.prefix_len
                      + ws.num_seqs * (int(lens[0]) - ws.prefix_len)) \
                * ws.num_kv_heads * ws.head_dim * 2 * es
            res["unique_kv_bytes"] = unique
            res["unique_kv_gbps"] = round(
                unique / (res["t_attn_us"]["median"] * 1e-6) / 1e9, 2)
            res["unique_hbm_frac"] = round(res["unique_kv_gbps"] / HBM_PEAK_GBPS, 4)
            res["note"] = ("attn_kv_gbps counts the bytes every sequence reads (logical); "
                           "unique_kv_gbps the bytes the pool holds once")
            del st
            torch.cuda.empty_cache()
            if not args.no_cpu_baseline:
                key = (prompts, bs, final)
                if key not in sharing_baselines:
                    sharing_baselines[key] = cpu_baseline_sharing(
                        args.prefix, bs, prompts, final, args.report_cpu_seconds)
                base = sharing_baselines[key]
                if fp8:   # the oracle over bf16 pools; the GPU figure counts 1-byte codes
                    res["cpu_baseline_note"] = "oracle over the bf16 pools of the same step"
                res["cpu_baseline"] = base
                res["gpu_over_cpu"] = round(res["attn_tokens_per_s"] / base["tokens_per_s"], 1)
            print(json.dumps({"report": res}), flush=True)


def fp8_report(torch, ops, args, steps=20, warmup=3):
    """The batch-256 GQA decode step over FP8 E4M3 pools with a scale per
    (block, kv head): the write encodes the step's bf16 K/V, the decode reads
    1-byte codes.  KV GB/s counts the bytes the pools hold (1 per element)."""
    from paged_kv_cache_330_amd.workloads import make_decode_workload
    w = make_decode_workload(3)
    st = fp8_step_state(torch, ops, w, args.pools, args.partition_tokens)
    wall, t_copy, t_write, t_attn = time_steps(torch, st, steps, warmup)
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    res, _, _ = summary(w.name + "_fp8_e4m3", {"seed": w.seed, "kv_dtype": "fp8_e4m3",
                                               "scales": "per (block, kv head), max-abs / 448"},
                        w.seq_lens, B, Hq, Hkv, D, bs, steps, wall, t_copy, t_write, t_attn, es=1)
    kv, alg = attn_bytes_fp8(w.seq_lens, B, Hq, Hkv, D, bs)
    res["attn_alg_gbps"] = round(alg / (statistics.mean(t_attn) * 1e-3) / 1e9, 2)
    res["attn_alg_hbm_frac"] = round(res["attn_alg_gbps"] / HBM_PEAK_GBPS, 4)
    res["algorithmic_bytes_per_launch"] = alg
    # the write reads bf16 K/V and the slots, writes 1-byte codes, reads scales
    wb = B * Hkv * D * 2 * (2 + 1) + 8 * B + 2 * 4 * B * Hkv
    res["write_gbps"] = round(wb / (statistics.median(t_write) * 1e-3) / 1e9, 2)
    del st
    torch.cuda.empty_cache()
    ks, vs = w.fp8_scales(unused=1.0)
    print(json.dumps({"report": with_baseline(res, args, cpu_baseline_fp8, w, ks, vs)}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0

PREFILL_WORKLOADS = [
    # name, context tokens per sequence, new tokens per sequence, sequences
    ("prefix_sharing_prompts", 0, 2044, 4),
    ("llama3_8b_prompts_16x2048", 0, 2048, 16),
    ("chunks_512_after_4096", 4096, 512, 8),
]


def prefill_report(torch, ops, args, reps=10):
    """Paged prefill of Llama-3-8B-shaped prompts (32 q / 8 kv heads, head_dim
    128, bf16, block size 16): the write of every prompt token through the
    slot mapping, then causal attention of the new tokens; then the same over
    FP8 E4M3 pools.  The attention is bound by the matrix cores: algorithmic
    flops = 4 D Hq (p + 1) per new token at position p, against the dense
    bf16 MFMA peak."""
    from paged_kv_cache_330_amd.workloads import (PrefillWorkload, empty_device_caches,
                                                  torch_tensor)
    dev = "cuda"
    for name, ctx, new, nseq in PREFILL_WORKLOADS:
        w = PrefillWorkload([ctx] * nseq, [new] * nseq, block_size=16, seed=13)
        kc, vc = empty_device_caches(w.num_blocks, 16, w.num_kv_heads, w.head_dim, "bf16", dev,
                                     fill="zero")
        kt, vt = torch_tensor(w.k_tokens, "bf16", dev), torch_tensor(w.v_tokens, "bf16", dev)
        slots = torch.from_numpy(w.slots).to(dev)
        q = torch_tensor(w.q, "bf16", dev)
        qs = torch.from_numpy(w.query_start).to(dev)
        bt = torch.from_numpy(w.block_tables).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        out = torch.empty((w.num_tokens, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
        write = lambda: ops.pkv_kv_write(kt, vt, slots, kc, vc)  # noqa: E731
        attend = lambda: ops.pkv_attention_prefill(out, q, qs, kc, vc, bt, sl, float(w.scale))  # noqa: E731
        res = {"workload": name, "num_seqs": nseq, "context_tokens": ctx, "new_tokens": new,
               "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
               "head_dim": w.head_dim, "block_size": 16}
        for label, call in (("write", write), ("attn", attend)):
            call()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ops.pkv_check_device_errors()
            res[f"t_{label}_us"] = round(statistics.median(ts) * 1e3, 2)
        row = w.num_kv_heads * w.head_dim * 2
        wbytes = 2 * 2 * len(w.slots) * row + 8 * len(w.slots)
        res["write_gbps"] = round(wbytes / (res["t_write_us"] * 1e-6) / 1e9, 1)
        flops = w.flops()
        tflops = flops / (res["t_attn_us"] * 1e-6) / 1e12
        res["attn_flops"] = flops
        res["attn_tflops"] = round(tflops, 1)
        res["attn_mfma_frac"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)
        res["prompt_tokens_per_s"] = round(w.num_tokens / ((res["t_write_us"] + res["t_attn_us"]) * 1e-6), 1)
        # the same prompts over FP8 E4M3 pools (max-abs block scales)
        from paged_kv_cache_330_amd.workloads import fp8_block_scales
        ks_h, vs_h = fp8_block_scales(w.k_tokens, w.v_tokens, w.slots, w.num_blocks, 16, unused=1.0)
        ks, vs = torch.from_numpy(ks_h).to(dev), torch.from_numpy(vs_h).to(dev)
        k8 = torch.zeros(kc.shape, dtype=torch.uint8, device=dev)
        v8 = torch.zeros_like(k8)
        write8 = lambda: ops.pkv_kv_write_fp8(kt, vt, slots, k8, v8, ks, vs)  # noqa: E731
        attend8 = lambda: ops.pkv_attention_prefill_fp8(out, q, qs, k8, v8, ks, vs, bt, sl,  # noqa: E731
                                                        float(w.scale))
        for label, call in (("write_fp8", write8), ("attn_fp8", attend8)):
            call()
            torch.cuda.synchronize()
            ts = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            ops.pkv_check_device_errors()
            res[f"t_{label}_us"] = round(statistics.median(ts) * 1e3, 2)
        res["attn_fp8_tflops"] = round(flops / (res["t_attn_fp8_us"] * 1e-6) / 1e12, 1)
        del kc, vc, kt, vt, k8, v8
        torch.cuda.empty_cache()
        res = with_baseline(res, args, cpu_baseline_prefill, w, gpu_key="attn_tflops")
        print(json.dumps({"report": res}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the paged decode path "
              "here is a single-GPU build", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(torch)
        return
    if args.read_probe:
        read_probe(torch)
        return
    if args.counter_pass:
        counter_pass(torch, args)
        return

    from paged_kv_cache_330_amd import ops
    from paged_kv_cache_330_amd.workloads import make_decode_workload

    ops.load_library()
    if args.prefill:
        prefill_report(torch, ops, args)
        return
    if args.fp8:
        fp8_report(torch, ops, args)
        return
    if args.only:
        report_all(torch, ops, args, set(args.only.split(",")))
        return
    if args.report_all:
        report_all(torch, ops, args)
    t_gen = time.perf_counter()
    w = make_decode_workload(args.config, block_size=args.block_size)
    t_gen = time.perf_counter() - t_gen
    st = decode_step_state(torch, ops, w, args.pools, args.partition_tokens)
    wall, t_copy, t_write, t_attn = time_steps(torch, st, args.steps, args.warmup)
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    rep, kv_bytes, alg = summary(w.name, {}, w.seq_lens, B, Hq, Hkv, D, bs, args.steps, wall,
                                 t_copy, t_write, t_attn, es=w.elem_bytes)
    ms_per_step = wall * 1e3 / args.steps
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    t_call = time_decode_calls(torch, st, args.steps, 3 * args.steps)
    achieved = alg / (t_call * 1e-3) / 1e9
    flops = 4 * Hq * D * int(w.seq_lens.sum())
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": w.name, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": bs, "seq_len_sum": rep["seq_len_sum"],
            "seq_len_max": int(w.seq_lens.max()), "seq_len_min": int(w.seq_lens.min()),
            "schedule": ("balanced" if args.partition_tokens == 0 else
                         f"partitions of {args.partition_tokens} tokens"),
            "num_blocks": w.num_blocks, "kv_pool_copies": len(st.pools), "seed": w.seed,
            "out_dtype": "f32",
        },
        "hbm_frac_step": round(value / HBM_PEAK_GBPS, 4),
        "attn_kv_gbps": rep["attn_kv_gbps"],
        "attn_hbm_frac": rep["attn_hbm_frac"],
        "tokens_per_s": rep["tokens_per_s"],
        "attn_tokens_per_s": rep["attn_tokens_per_s"],
        "t_attn_us": rep["t_attn_us"],
        "t_write_us": rep["t_write_us"],
        "write_gbps": rep["write_gbps"],
        "attn_tflops": round(flops / (statistics.median(t_attn) * 1e-3) / 1e12, 3),
        "kv_bytes_per_step": kv_bytes,
        "roofline": {
            "kernel": ("pkv_attention_decode: " + ("decode_balanced_kernel + balanced_reduce_kernel"
                       if args.partition_tokens == 0 else "decode_mfma_kernel + splitk_reduce_kernel")),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": (measured_traffic() if (args.config, args.block_size,
                                                 args.partition_tokens) == (3, None, 0) else None),
            "algorithmic_bytes_per_launch": alg,
            "mean_call_us": round(t_call * 1e3, 2),
            "timing": f"events around {args.steps} back-to-back decode calls",
        },
        "workload_gen_s": round(t_gen, 2),
    }
    del st
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        res["gpu_over_cpu"] = round(res["attn_kv_gbps"] / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
