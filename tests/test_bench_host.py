"""Host-side pieces of bench.py, on the CPU: the oracle baselines that every
report line carries run on small workloads and report what they timed."""
import numpy as np

import bench
from paged_kv_cache_330_amd.workloads import PrefillWorkload, make_decode_workload


def check_entry(e, unit):
    assert e["kind"] == "oracle" and e["unit"] == unit
    assert e["value"] > 0 and e["seconds"] > 0
    assert 1 <= e["cores"] <= bench.ORACLE_MAX_THREADS and e["cores"] <= e["host_cpus_visible"]
    assert str(e["cores"]) + " threads" in e["sample"]


def test_decode_baselines():
    w = make_decode_workload(3, seq_lens=[40, 300, 17, 1000, 5], block_size=16)
    check_entry(bench.cpu_baseline(w, 0.2), "GB/s")
    ks, vs = w.fp8_scales(unused=1.0)
    check_entry(bench.cpu_baseline_fp8(w, ks, vs, 0.2), "GB/s")


def test_sharing_and_prefill_baselines():
    e = bench.cpu_baseline_sharing(60, 8, 2, False, 0.2)
    check_entry(e, "GB/s")
    assert "copy_ref of 14 pairs" in e["sample"]            # 2 prompts x 7 copies at step 1
    pw = PrefillWorkload([0, 10], [300, 40], block_size=16, seed=13)
    check_entry(bench.cpu_baseline_prefill(pw, 0.2), "TFLOP/s")


def test_swap_baseline():
    e = bench.cpu_baseline_swap(128, 0.2, chunk=16)
    check_entry(e, "GB/s")
    assert "chunks of 16 blocks" in e["sample"]


def test_algorithmic_bytes():
    # K/V rows + bf16 q + fp32 out + table entries + lengths
    kv, alg = bench.attn_bytes([16, 17], 2, 4, 2, 128, 16, 2)
    assert kv == 33 * 2 * 128 * 2 * 2
    assert alg == kv + 2 * 4 * 128 * 2 + 2 * 4 * 128 * 4 + 4 * 3 + 4 * 2
    kv8, alg8 = bench.attn_bytes_fp8([16, 17], 2, 4, 2, 128, 16)
    assert kv8 == kv // 2 and alg8 == kv8 + 8 * 3 * 2 + 2 * 4 * 128 * 2 + 2 * 4 * 128 * 4 + 4 * 3 + 8
    assert np.isclose(bench.HBM_PEAK_GBPS, 8000.0)
