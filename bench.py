"""Benchmark of the paged decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--block-size BS]

A step is one pass of the hot path over one batch: the slot-mapping write of
every sequence's new token (pkv_kv_write), then decode attention over all
cached tokens (pkv_attention_decode: the balanced-schedule kernel and the
reduce of the sequences it cuts).  The
default workload is the batch-256 Llama-3-8B-shaped GQA decode (32 q / 8 kv
heads, head_dim 128, block_size 16, lognormal lengths, median 1024, clipped to
[16, 8192]; seed 3), synthetic bf16 data resident in HBM.

Cache honesty: the step rotates over several identical copies of the KV pool
(--pools, default 3), so that no step finds the previous step's blocks in the
L2 / MALL caches.

Prints one JSON line: value = KV GB/s of the whole step (KV bytes the step's
attention must read / step time), plus the attention-only rate, tokens/s, a
roofline entry for the decode call and the fp64 CPU oracle timed on a bounded
sample of the same workload.
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


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=3)
    p.add_argument("--block-size", type=int, default=None)
    p.add_argument("--partition-tokens", type=int, default=0)
    p.add_argument("--pools", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate budget of the CPU oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return p.parse_args()


def copy_probe(torch):
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}), flush=True)


def cpu_baseline(w, budget_s):
    """The fp64 oracle on a bounded sample of the same workload.

    A pass is ``write_ref`` of the step's new tokens followed by ``decode_ref``
    of a prefix of the batch (sequences 0..n-1), parallel over sequences.  The
    prefix is sized from a one-sequence calibration to about ``budget_s``
    seconds; when the whole batch takes less, whole passes repeat until the
    budget is spent.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle

    kc, vc = w.empty_caches("zero")
    t0 = time.perf_counter()
    oracle.write_ref(w.k_tokens[w.prefill_rows], w.v_tokens[w.prefill_rows], w.prefill_slots, kc, vc)
    prefill_s = time.perf_counter() - t0
    workers = max(1, min(16, len(os.sched_getaffinity(0))))

    def run(r):
        return oracle.decode_ref(w.q[[r]], kc, vc, w.block_tables[[r]], w.seq_lens[[r]],
                                 w.scale, w.dtype)

    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        t0 = time.perf_counter()
        run(0)
        per_token = (time.perf_counter() - t0) / max(1, int(w.seq_lens[0]))
        target_tokens = budget_s * workers / max(per_token, 1e-9)
        cum = np.cumsum(w.seq_lens.astype(np.int64))
        n = int(min(w.num_seqs, max(workers, np.searchsorted(cum, target_tokens) + 1)))
        rows = list(range(n))
        passes = 0
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            while True:
                oracle.write_ref(w.k_tokens[w.step_rows[rows]], w.v_tokens[w.step_rows[rows]],
                                 w.step_slots[rows], kc, vc)
                list(ex.map(run, rows))
                passes += 1
                dt = time.perf_counter() - t0
                if dt >= budget_s or n < w.num_seqs:
                    break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    tokens = int(w.seq_lens[rows].sum())
    kv = passes * tokens * w.num_kv_heads * w.head_dim * 2 * w.elem_bytes
    return {
        "value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": workers, "kind": "oracle",
        "sample": (f"{passes} pass(es) of write_ref of {n} new tokens + decode_ref of sequences "
                   f"0..{n - 1} ({tokens} of {int(w.seq_lens.sum())} cached tokens) of the same "
                   f"workload, fp64 NumPy, {workers} threads, {dt:.1f} s (prefill write_ref of "
                   f"the pool, untimed: {prefill_s:.1f} s)"),
        "seconds": round(dt, 3),
        "tokens_per_s": round(passes * n / dt, 3),
    }


COUNTERS = os.path.join(ROOT, "profiles", "decode_balanced_llama3_8b_gqa_b256_hbm_counters.md")


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the paged decode path "
              "here is a single-GPU build", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(torch)
        return

    from paged_kv_cache_330_amd import ops
    from paged_kv_cache_330_amd.workloads import (empty_device_caches, make_decode_workload,
                                                  torch_tensor)

    ops.load_library()
    dev = "cuda"
    t_gen = time.perf_counter()
    w = make_decode_workload(args.config, block_size=args.block_size)
    t_gen = time.perf_counter() - t_gen
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size
    es = w.elem_bytes

    kt, vt = torch_tensor(w.k_tokens, w.dtype, dev), torch_tensor(w.v_tokens, w.dtype, dev)
    pre = torch.from_numpy(w.prefill_rows).to(dev)
    pre_slots = torch.from_numpy(w.prefill_slots).to(dev)
    k_pre, v_pre = kt[pre].contiguous(), vt[pre].contiguous()
    step = torch.from_numpy(w.step_rows).to(dev)
    k_new, v_new = kt[step].contiguous(), vt[step].contiguous()
    step_slots = torch.from_numpy(w.step_slots).to(dev)
    del kt, vt
    pools = []
    for _ in range(args.pools):
        kc, vc = empty_device_caches(w.num_blocks, bs, Hkv, D, w.dtype, dev, fill="zero")
        ops.pkv_kv_write(k_pre, v_pre, pre_slots, kc, vc)
        pools.append((kc, vc))
    del k_pre, v_pre
    q = torch_tensor(w.q, w.dtype, dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws_bytes = ops.pkv_attention_workspace_bytes(pools[0][0], pools[0][1], B, Hq, bt.shape[1],
                                                 args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    ops.pkv_check_device_errors()

    def one_step(i, ev=None):
        kc, vc = pools[i % len(pools)]
        if ev:
            ev[0].record()
        ops.pkv_kv_write(k_new, v_new, step_slots, kc, vc)
        if ev:
            ev[1].record()
        ops.pkv_attention_decode(out, q, kc, vc, bt, sl, float(w.scale), args.partition_tokens, ws)
        if ev:
            ev[2].record()

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    ops.pkv_check_device_errors()

    # Timed region: exactly K steps, synchronised on both sides.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ops.pkv_check_device_errors()

    t_write = [e[0].elapsed_time(e[1]) for e in events]    # ms
    t_attn = [e[1].elapsed_time(e[2]) for e in events]
    ms_per_step = wall * 1e3 / args.steps
    attn_ms = statistics.median(t_attn)
    write_ms = statistics.median(t_write)

    total_tokens = int(w.seq_lens.sum())
    kv_bytes = w.kv_bytes()
    table_entries = int(sum(math.ceil(int(L) / bs) for L in w.seq_lens))
    attn_alg_bytes = kv_bytes + B * Hq * D * es + B * Hq * D * 4 + 4 * table_entries + 4 * B
    write_alg_bytes = 2 * (2 * B * Hkv * D * es) + 8 * B
    flops = 4 * Hq * D * total_tokens
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    attn_gbps = kv_bytes / (attn_ms * 1e-3) / 1e9
    achieved = attn_alg_bytes / (statistics.mean(t_attn) * 1e-3) / 1e9

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
            "head_dim": D, "block_size": bs, "seq_len_sum": total_tokens,
            "seq_len_max": int(w.seq_lens.max()), "seq_len_min": int(w.seq_lens.min()),
            "schedule": ("balanced" if args.partition_tokens == 0 else
                         f"partitions of {args.partition_tokens} tokens"),
            "num_blocks": w.num_blocks,
            "kv_pool_copies": len(pools), "seed": w.seed, "out_dtype": "f32",
        },
        "hbm_frac_step": round(value / HBM_PEAK_GBPS, 4),
        "attn_kv_gbps": round(attn_gbps, 2),
        "attn_hbm_frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(B / (ms_per_step * 1e-3), 1),
        "attn_tokens_per_s": round(B / (attn_ms * 1e-3), 1),
        "t_attn_us": {"median": round(attn_ms * 1e3, 2),
                      "p10": round(float(np.percentile(t_attn, 10)) * 1e3, 2),
                      "p90": round(float(np.percentile(t_attn, 90)) * 1e3, 2)},
        "t_write_us": round(write_ms * 1e3, 2),
        "write_gbps": round(write_alg_bytes / (write_ms * 1e-3) / 1e9, 2),
        "attn_tflops": round(flops / (attn_ms * 1e-3) / 1e12, 3),
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
            "algorithmic_bytes_per_launch": attn_alg_bytes,
        },
        "workload_gen_s": round(t_gen, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        res["gpu_over_cpu"] = round(res["attn_kv_gbps"] / res["cpu_baseline"]["value"], 1)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
