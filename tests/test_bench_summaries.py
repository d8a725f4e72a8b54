"""Host checks of bench.py's profiler summaries: split-kernel dispatches of every instantiation are
assigned to the phases of the dispatch plan in launch order, and the counter summary scales each
counter by the calibration copy's known size."""
import csv
import importlib.util
import json
import os
import sqlite3

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("_bench_for_summaries", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


PLAN = [
    {"phase": "warm-up fused steps", "launches": 2, "untimed_first": 2},
    {"phase": "fused split kernel, cold", "launches": 3, "untimed_first": 1},
    {"phase": "attention-only split kernel, cold", "launches": 2, "untimed_first": 0},
    {"phase": "paged K4V2: cold", "launches": 2, "untimed_first": 1},
    {"phase": "rotated 131k: cold", "launches": 3, "untimed_first": 1},
]
HEAD = "void kvq_attn::kvq_attn_split_kernel<4, 2, 4, 1, 1>(kvq_attn::KvqAttnArgs)"
ROT = "void kvq_attn::kvq_attn_split_kernel<4, 2, 8, 2, 1>(kvq_attn::KvqAttnArgs)"


def _dispatches():
    """(kernel name, fetch KiB, write KiB, duration ns) in launch order, other kernels between."""
    d = [(HEAD, 1, 1, 100)] * 2
    d += [("other_kernel", 5, 5, 7)]
    d += [(HEAD, 999, 999, 500)] + [(HEAD, 100, 2, 90)] * 2  # first launch untimed
    d += [(HEAD, 80, 1, 80)] * 2
    d += [("(anonymous namespace)::stream_copy_kernel(...)", 512, 256, 40)]
    d += [(HEAD, 777, 777, 1)] + [(HEAD, 30, 1, 20)]
    d += [(ROT, 999, 999, 1)] + [(ROT, 600, 3, 1200)] * 2
    return d


def _bench_json(tmp_path):
    res = {"config": {"workload": "w"}, "split_kernel_dispatch_plan": PLAN, "value": 1, "gpu_us_per_step": 1,
           "split_kernel_us_cold": 1, "split_kernel_us_warm": 1, "combine_us": 1,
           "attention_split_kernel": {"us_cold": 1, "us_warm": 1},
           "roofline": {"frac": 0.5, "frac_warm": 0.6, "stream_ceiling_GBs": 5900}}
    p = tmp_path / "bench.json"
    p.write_text("noise\n" + json.dumps(res) + "\n")
    return str(p)


def _write_counters(d, counter, col):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Correlation_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        rows = [dict(Dispatch_Id=i + 1, Correlation_Id=i + 1, Kernel_Name=k, Counter_Name=counter,
                     Counter_Value=vals[col]) for i, (k, *vals) in enumerate(_dispatches())]
        for r in reversed(rows):  # file order is not launch order
            w.writerow(r)


def test_summarize_pmc_slices_by_plan_and_scales(tmp_path):
    B = _bench()
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", 0)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", 1)
    out = tmp_path / "traffic.json"
    copy_bytes = 1 << 20  # 1024 KiB: fetch counter reads 512 KiB -> factor 2, write 256 KiB -> factor 4
    B.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), _bench_json(tmp_path), copy_bytes, str(out))
    tr = json.loads(out.read_text())
    assert tr["fetch_scale"] == pytest.approx(2.0) and tr["write_scale"] == pytest.approx(4.0)
    ph = tr["phases"]
    assert ph["fused split kernel, cold"]["read_bytes_per_launch"] == 100 * 1024 * 2
    assert ph["fused split kernel, cold"]["write_bytes_per_launch"] == 2 * 1024 * 4
    assert tr["bytes_per_launch"] == 100 * 1024 * 2 + 2 * 1024 * 4
    assert ph["attention-only split kernel, cold"]["read_bytes_per_launch"] == 80 * 1024 * 2
    assert ph["paged K4V2: cold"]["read_bytes_per_launch"] == 30 * 1024 * 2
    assert ph["rotated 131k: cold"]["read_bytes_per_launch"] == 600 * 1024 * 2
    assert ph["rotated 131k: cold"]["instantiation"] == "<4, 2, 8, 2, 1>"


def test_summarize_pmc_rejects_a_plan_mismatch(tmp_path):
    B = _bench()
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", 0)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", 1)
    bj = tmp_path / "bench.json"
    res = json.loads(open(_bench_json(tmp_path)).read().splitlines()[-1])
    res["split_kernel_dispatch_plan"][0]["launches"] = 3
    bj.write_text(json.dumps(res))
    with pytest.raises(SystemExit):
        B.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(bj), 1 << 20, str(tmp_path / "t.json"))


def test_summarize_trace_reads_rocpd_database(tmp_path):
    B = _bench()
    d = tmp_path / "trace"
    os.makedirs(d)
    con = sqlite3.connect(str(d / "run_results.db"))
    con.execute("create table kernels (name text, start integer, end integer)")
    t = 1000
    for k, _, _, ns in _dispatches():
        con.execute("insert into kernels values (?, ?, ?)", (k, t, t + ns))
        t += ns + 10
    con.commit()
    con.close()
    md = tmp_path / "out.md"
    B.summarize_trace(str(d), _bench_json(tmp_path), str(md), "cmd")
    text = md.read_text()
    assert "expects 12." in text
    assert "| fused split kernel, cold | `<4, 2, 4, 1, 1>` | 3 | 2 | 0.09 |" in text
    assert "| rotated 131k: cold | `<4, 2, 8, 2, 1>` | 3 | 2 | 1.20 |" in text
    assert "| warm-up fused steps | `<4, 2, 4, 1, 1>` | 2 | 0 |" in text
