"""Host checks of the seeded input generator (no method arithmetic involved)."""
import os

import numpy as np
import torch

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_splitmix64_reference_outputs():
    # SplitMix64 seeded with 0: first outputs of the published reference generator.
    key = 0
    out = W.splitmix_u64(key, np.arange(3, dtype=np.uint64))
    assert [hex(int(v)) for v in out] == ["0xe220a8397b1dcdaf", "0x6e789e6aa1b965f4", "0x6c45d188009454f"]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-30, 30, 100000)).astype(np.float32)
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_normal_table_moments():
    t = W.normal_table().astype(np.float64)
    assert abs(t.mean()) < 1e-6 and abs(t.std() - 1.0) < 2e-3
    assert np.all(np.diff(t) > 0)


def test_generator_determinism_and_shapes():
    wl = W.WORKLOADS[2]
    a = wl.kv_f32(W.TENSOR_K, 0, 3, 100, 5)
    b = wl.kv_f32(W.TENSOR_K, 0, 3, 102, 3)
    assert np.array_equal(a[2:], b)
    sig = wl.key_sigma()
    assert sig.shape == (8, 128) and np.array_equal(sig, wl.key_sigma())
    assert np.all(np.sort(sig, axis=1)[:, -3:].min(axis=1) > 2.0)  # three outlier channels per head
    q = wl.q_f32(0)
    assert q.shape == (1, 32, 128)
    lens = W.WORKLOADS[4].context_lengths()
    assert lens.min() >= 1024 and lens.max() <= 16384
    table, pool = W.WORKLOADS[4].block_table()
    used = table[table >= 0]
    assert np.array_equal(np.sort(used), np.arange(pool))


def test_bench_cpu_baseline_runs_on_a_small_sample():
    """bench.py's cpu_baseline leg (the oracle timed on a sample of one decode step) runs and
    reports its sample, on a shortened version of the 32k workload."""
    import dataclasses
    import importlib.util

    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    wl = dataclasses.replace(W.WORKLOADS[3], context=400)
    r = bench.cpu_baseline(wl, target_seconds=0.01, max_units=2, workers=1)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["value"] > 0 and r["value_1core"] > 0
    assert r["sample"].startswith("1 of ") or r["sample"].startswith("2 of ")
    r = bench.cpu_baseline(wl, target_seconds=0.01, max_units=4, workers=2)  # two forked workers
    assert r["cores"] == 2 and r["value"] > 0 and r["value"] <= r["value_1core"] * 1.5
