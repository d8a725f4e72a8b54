#!/usr/bin/env python3
"""Benchmark of the decode hot path on one MI355X.

One step = one pass of the whole hot path over one batch: append one new token
per sequence (fused quantize + pack of the token leaving the recent window),
then decode attention of every query head over its whole cache (split-K kernel
+ cross-split combine).  Workload: batch 16, 32 query / 8 kv heads, d = 128,
32768-token context, 4-bit keys in groups of 32 and 2-bit values in groups of
128 with fp16 scale/zero, the most recent 128 tokens kept in bf16, bf16 queries.

Prints one JSON line (metric, value = microseconds per step, roofline of the
attention kernels, oracle CPU baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "K4V2 decode-attention µs/step + achieved HBM GB/s (% of peak), 32k ctx"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_b16_L32k.json")


def split_kernel_bytes(wl, L, per_token_head, win_elem_bytes, q_elem_bytes=2):
    """Algorithmic HBM bytes of one split-kernel launch with every sequence at length L.

    Per (sequence, kv head) unit: the quantized tokens' payload and metadata
    (per_token_head bytes each), the recent-window tokens' keys and values, and
    the unit's query heads.  Partial results (an artefact of splitting) are not counted.
    """
    nq = max(0, L - wl.window)
    nw = min(L, wl.window)
    units = wl.batch * wl.num_kv_heads
    per_unit = nq * per_token_head + nw * 2 * wl.head_dim * win_elem_bytes + wl.group_q * wl.head_dim * q_elem_bytes
    return units * per_unit


def append_bytes(wl, L, n):
    """Algorithmic HBM bytes of appending n tokens to every sequence of length L.

    Per (sequence, kv head): every new key/value row is read once; the up to R rows that end
    in the window ring are written there; each token that leaves the window (read back from
    the ring) or that is already older than the window on arrival is written quantized.
    """
    row = 2 * wl.head_dim * (4 if wl.kv_dtype == "f32" else 2)  # key + value row
    per_th = (wl.head_dim * wl.k_bits // 8 + (wl.head_dim // wl.k_group) * 4 + wl.head_dim * wl.v_bits // 8
              + (wl.head_dim // wl.v_group) * 4)
    R = wl.window
    ring = min(n, R)
    evicted = sum(1 for i in range(ring) if L + i - R >= 0)
    direct = max(0, n - R)
    per_unit = n * row + ring * row + evicted * (row + per_th) + direct * per_th
    return wl.batch * wl.num_kv_heads * per_unit


def source_digest():
    """Digest of the sources the split kernel is built from (invalidates stored counter data)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixed_precision_kv_kvq_amd", "csrc")
    for name in ("kvq_attn_impl.h", "kvq_layout.h", "kvq_internal.h", "kvq_quant.h", "kvq_attn_inst.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


SPLIT_KERNEL = "kvq_attn_split_kernel<4, 2, 4, 1, 1>"  # the instantiation of the timed decode step
SPLIT_PREFIX = "kvq_attn_split_kernel<"  # every instantiation (the dispatch plan counts them all)
CALIBRATION_KERNEL = "stream_copy_kernel"  # kvq_gen_stream_copy: a copy of known size
# phases whose per-launch counters are kept in the traffic file (decode step; paged and rotated
# workloads), each keyed by its phase name in the dispatch plan
TRAFFIC_PHASES = ("fused split kernel, cold", "attention-only split kernel, cold", "paged K4V2: cold",
                  "rotated 131k: cold")


def progress(msg):
    """A progress line on stderr (long runs report each phase as it starts)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _split_name(name):
    """The template instantiation of a split-kernel dispatch name, e.g. '<4, 2, 4, 1, 1>'."""
    name = name.replace("  ", " ")
    i = name.find(SPLIT_PREFIX)
    return name[i + len(SPLIT_PREFIX) - 1:name.index(">", i) + 1]


def _plan_slices(split_rows, plan):
    """Yield (phase, all rows of the phase, timed rows) by walking the dispatch plan over the
    split-kernel dispatches in launch order."""
    i = 0
    for ph in plan:
        seg = split_rows[i:i + ph["launches"]]
        i += ph["launches"]
        yield ph, seg, seg[ph["untimed_first"]:]


def _last_json(path):
    with open(path) as fh:
        return json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])


def summarize_pmc(fetch_dir, write_dir, bench_json, copy_bytes, out_path=TRAFFIC_FILE):
    """Per-launch HBM bytes of the split kernel in the phases of TRAFFIC_PHASES from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE, in KiB per dispatch) of `bench.py
    --copy-calibration-mib N` with the same arguments, each counter scaled by the ratio of the
    calibration copy's known bytes to what the same counter reports for it.  Dispatches are
    assigned to phases by the dispatch plan the run printed (bench_json)."""
    import csv
    import glob

    plan = _last_json(bench_json)["split_kernel_dispatch_plan"]

    def read(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r.get("Dispatch_Id") or r["Correlation_Id"]))
        split = [r for r in rows if SPLIT_PREFIX in r["Kernel_Name"].replace("  ", " ")]
        cal = [float(r["Counter_Value"]) for r in rows if CALIBRATION_KERNEL in r["Kernel_Name"]]
        if not split or not cal:
            raise SystemExit(f"{counter}: no split-kernel or calibration rows under {d}")
        if len(split) != sum(p["launches"] for p in plan):
            raise SystemExit(f"{counter}: {len(split)} split-kernel dispatches, the plan expects "
                             f"{sum(p['launches'] for p in plan)}")
        per = {}
        for ph, _, timed in _plan_slices(split, plan):
            if ph["phase"] in TRAFFIC_PHASES and timed:
                per[ph["phase"]] = (sum(float(r["Counter_Value"]) for r in timed) / len(timed), len(timed),
                                    _split_name(timed[0]["Kernel_Name"]))
        return per, sum(cal) / len(cal)

    fetch, fc = read(fetch_dir, "FETCH_SIZE")
    write, wc = read(write_dir, "WRITE_SIZE")
    f_factor = copy_bytes / (fc * 1024.0)
    w_factor = copy_bytes / (wc * 1024.0)
    phases = {}
    for name in TRAFFIC_PHASES:
        if name in fetch and name in write:
            rd = int(fetch[name][0] * 1024.0 * f_factor)
            wr = int(write[name][0] * 1024.0 * w_factor)
            phases[name] = {"instantiation": fetch[name][2], "launches": [fetch[name][1], write[name][1]],
                            "fetch_kib_raw": fetch[name][0], "write_kib_raw": write[name][0],
                            "read_bytes_per_launch": rd, "write_bytes_per_launch": wr, "bytes_per_launch": rd + wr}
    head = phases.get(TRAFFIC_PHASES[0])
    out = {
        "kernel": SPLIT_KERNEL,
        "source_digest": source_digest(),
        "copy_bytes": copy_bytes, "copy_fetch_kib_raw": fc, "copy_write_kib_raw": wc,
        "fetch_scale": f_factor, "write_scale": w_factor,
        "bytes_per_launch": head["bytes_per_launch"] if head else None,
        "phases": phases,
    }
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def stored_traffic(phase):
    """Counter-measured HBM bytes per launch of a phase, or None when absent or taken from other
    kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    if tr.get("source_digest") != source_digest():
        return None
    return (tr.get("phases") or {}).get(phase, {}).get("bytes_per_launch")


def summarize_trace(trace_dir, bench_json, out_md, command):
    """Per-phase average durations of the split kernel (every instantiation) and the other
    kernels' averages from a `rocprofv3 --kernel-trace` run of this script, sliced by the
    dispatch plan the run printed."""
    import csv
    import glob

    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    for f in glob.glob(os.path.join(trace_dir, "**", "*results.db"), recursive=True):  # rocpd database output
        import sqlite3

        con = sqlite3.connect(f)
        rows += [{"Kernel_Name": n, "Start_Timestamp": a, "End_Timestamp": b}
                 for n, a, b in con.execute("select name, start, end from kernels")]
        con.close()
    if not rows:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    res = _last_json(bench_json)
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def dur(r):
        return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # ns -> µs

    split = [r for r in rows if SPLIT_PREFIX in r["Kernel_Name"].replace("  ", " ")]
    plan = res["split_kernel_dispatch_plan"]
    expect = sum(p["launches"] for p in plan)
    lines = [f"# Kernel trace of `{res['config']['workload']}` and the bench's other workloads", "",
             "Command (repository root on the GPU box):", "", "```", command, "```", "",
             f"Split kernel (`kvq_attn::kvq_attn_split_kernel<KB, VB, G, P, NVG>`, every instantiation): "
             f"{len(split)} dispatches; the dispatch plan printed by the run expects {expect}"
             + ("." if len(split) == expect else " (MISMATCH: phases below are unreliable)."), "",
             "| phase | instantiation | launches | timed | trace avg µs | trace min µs | trace max µs |",
             "|---|---|---:|---:|---:|---:|---:|"]
    for ph, seg, timed in _plan_slices(split, plan):
        inst = _split_name(seg[0]["Kernel_Name"]) if seg else ""
        if timed:
            d = [dur(r) for r in timed]
            lines.append(f"| {ph['phase']} | `{inst}` | {ph['launches']} | {len(timed)} | {sum(d) / len(d):.2f} | "
                         f"{min(d):.2f} | {max(d):.2f} |")
        else:
            lines.append(f"| {ph['phase']} | `{inst}` | {ph['launches']} | 0 | | | |")
    rf = res["roofline"]
    lines += ["", "Bench figures of the same run (HIP events):", "",
              f"- value (µs per fused decode step, wall clock): {res['value']}; events: {res['gpu_us_per_step']}",
              f"- fused split kernel cold / warm (µs): {res['split_kernel_us_cold']} / {res['split_kernel_us_warm']}"
              f" (roofline frac cold {rf['frac']}, warm {rf['frac_warm']}; streaming ceiling "
              f"{rf['stream_ceiling_GBs']} GB/s)",
              f"- attention-only split kernel cold / warm (µs): {res['attention_split_kernel']['us_cold']} / "
              f"{res['attention_split_kernel']['us_warm']}",
              f"- merge (µs): {res['combine_us']}", "", "Other kernels (all dispatches):", "",
              "| kernel | dispatches | avg µs |", "|---|---:|---:|"]
    by = {}
    for r in rows:
        if SPLIT_PREFIX in r["Kernel_Name"].replace("  ", " "):
            continue
        by.setdefault(r["Kernel_Name"][:90], []).append(dur(r))
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1]))[:14]:
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _oracle_units_worker(job):
    """Worker of cpu_baseline: the oracle's decode-step work for some (sequence, kv head) units,
    one thread, returning the timed seconds per unit."""
    import numpy as np

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle as O
    import workloads as W

    wl, units, budget = job
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        L = wl.context + 1
        prm = dict(k_bits=wl.k_bits, k_group=wl.k_group, v_bits=wl.v_bits, v_group=wl.v_group, window=wl.window,
                   rotation=wl.rotation)
        q = wl.q_f32(0).astype(np.float64)
        g = wl.group_q
        scale = 1.0 / np.sqrt(wl.head_dim)
        times = []
        for b, kvh in units:
            Kx = wl.kv_f32(W.TENSOR_K, b, kvh, 0, L).astype(np.float64)
            Vx = wl.kv_f32(W.TENSOR_V, b, kvh, 0, L).astype(np.float64)
            stored = O.build_unit_cache(Kx, Vx, L - 1, prm)  # cache before the step (untimed)
            t0 = time.perf_counter()
            nq = max(0, L - wl.window)
            ev = nq - 1  # the token that leaves the window in this step
            kc, ks, kz = O.quantize(Kx[ev:ev + 1], wl.k_bits, wl.k_group)
            vc, vs, vz = O.quantize(Vx[ev:ev + 1], wl.v_bits, wl.v_group)
            k_codes = np.concatenate([stored["k_codes"], kc])
            k_scale = np.concatenate([stored["k_scale"], ks])
            k_zero = np.concatenate([stored["k_zero"], kz])
            v_codes = np.concatenate([stored["v_codes"], vc])
            v_scale = np.concatenate([stored["v_scale"], vs])
            v_zero = np.concatenate([stored["v_zero"], vz])
            cache = dict(nq=nq, k_hat=O.dequantize(k_codes, k_scale, k_zero, wl.k_group),
                         v_hat=O.dequantize(v_codes, v_scale, v_zero, wl.v_group),
                         k_win=Kx[nq:L], v_win=Vx[nq:L])
            for h in range(kvh * g, (kvh + 1) * g):
                O.unit_attention(q[b, h], cache, scale, wl.rotation)
            times.append(time.perf_counter() - t0)
            if sum(times) >= budget:
                break
        return times
    finally:
        if ctx:
            ctx.__exit__(None, None, None)


def cpu_worker_count():
    """Host threads the CPU baseline uses: the cores this process may run on, at most 16 (the
    host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, target_seconds=12.0, max_units=None, workers=None):
    """The CPU oracle timed on one decode step of the workload, on all host cores.

    Per (sequence, kv head) unit the oracle does what a decode step needs given its stored
    cache: quantize the token leaving the window, dequantize the stored codes, and run attention
    for the unit's query heads (building the stored cache is untimed).  Units are dealt round-robin
    to `workers` single-threaded processes that run concurrently; each stops after about
    target_seconds / workers of timed work.  The step time on all cores is the largest per-worker
    sum of unit times scaled to the worker's share of the whole step; the single-core figure is
    the sum over all units (each measured on one core), scaled to the whole step.
    Must run before this process initialises the GPU (the workers are forked)."""
    import multiprocessing as mp

    units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)][: max_units or None]
    n_all = wl.batch * wl.num_kv_heads
    W_ = workers or cpu_worker_count()
    W_ = max(1, min(W_, len(units)))
    shares = [units[w::W_] for w in range(W_)]
    jobs = [(wl, sh, max(target_seconds / W_, 0.5)) for sh in shares]
    t0 = time.perf_counter()
    if W_ == 1:
        res = [_oracle_units_worker(jobs[0])]
    else:
        ctx = mp.get_context("fork")  # forked children run numpy only (no pickled target)
        q = ctx.Queue()

        def run(i, job):
            q.put((i, _oracle_units_worker(job)))

        procs = [ctx.Process(target=run, args=(i, job)) for i, job in enumerate(jobs)]
        for pr in procs:
            pr.start()
        got = dict(q.get() for _ in procs)
        for pr in procs:
            pr.join()
        res = [got[i] for i in range(len(jobs))]
    wall = time.perf_counter() - t0
    done = sum(len(r) for r in res)
    cpu_s = sum(sum(r) for r in res)
    per_unit = cpu_s / done
    # all cores: each worker's measured rate applied to its share of the full step
    per_worker_step = [sum(r) / len(r) * (n_all / W_) for r in res if r]
    step_all = max(per_worker_step)
    return {
        "value": round(step_all * 1e6, 1),
        "unit": "µs/step",
        "cores": W_,
        "kind": "oracle",
        "value_1core": round(per_unit * n_all * 1e6, 1),
        "sample": f"{done} of {n_all} (sequence, kv head) units of one decode step at L={wl.context + 1} on "
                  f"{W_} single-threaded processes ({cpu_s:.1f} s of timed CPU work, {wall:.1f} s wall), "
                  f"scaled to the full step",
    }


def paged_sweep(torch, dev, reps, stream, ceiling_GBs, plan):
    """The paged batch-8 workload (lengths 1k-16k, 16-token pages through a random block table) for
    each bit pair: its cache filled by one append of every sequence's rows; the decode attention's
    split kernel (kvq_decode_partials, read-only) timed cold (cycling over copies of the page pool
    far above the Infinity Cache) and warm, against the same launch with every split sized from the
    longest sequence (KVQ_PAGES_PER_SPLIT=32, the plan before splits were sized per sequence); the
    merge; and the error-budget diagnostics against the original rows for decode step 0's query."""
    import numpy as np

    import mixed_precision_kv_kvq_amd as K
    import workloads as W
    from workloads.device import DeviceGenerator

    rows, eb_rows = [], []
    small_ceiling = None
    for kb, vb in W.SWEEP_BITS + W.PLANE_BITS:
        wl = W.WORKLOADS[4].with_bits(kb, vb)
        Lb = wl.context_lengths()
        Lmax = int(Lb.max())
        table_np, pool = wl.block_table()
        table = torch.from_numpy(table_np).to(dev)
        prm = K.make_params(wl.head_dim, wl.num_q_heads, wl.num_kv_heads, kb, wl.k_group, vb, wl.v_group, wl.window,
                            0, K.KVQ_BF16, wl.block_size)
        cb = K.CacheBuffers(prm, wl.batch, pool, table)
        gen = DeviceGenerator(wl)
        k_ref = gen.kv(W.TENSOR_K, 0, Lmax)
        v_ref = gen.kv(W.TENSOR_V, 0, Lmax)
        before = torch.zeros(wl.batch, dtype=torch.int32, device=dev)
        n_new = torch.from_numpy(Lb.astype(np.int32)).to(dev)
        K.kvq_quantize_append(prm, cb.struct, before, n_new, k_ref, v_ref, Lmax)
        q = gen.q(0)
        per_th = wl.head_dim * kb // 8 + (wl.head_dim // wl.k_group) * 4 + wl.head_dim * vb // 8 \
            + (wl.head_dim // wl.v_group) * 4
        qpages = -(-Lb // 16)
        nbytes = int(wl.num_kv_heads * (Lb.sum() * per_th + qpages.sum() * 4)
                     + wl.batch * wl.num_q_heads * wl.head_dim * 2)
        if small_ceiling is None:
            # the read-only streaming ceiling at this launch's size (the first bit pair, K4V2)
            small_ceiling = stream_ceiling(torch, nbytes, stream, reps)
        n_cp = copies_for(nbytes)
        copies = [cb] + [clone_cache(K, torch, cb, prm, wl.batch, pool, table) for _ in range(n_cp - 1)]
        wsb = K.kvq_decode_workspace_bytes(prm, wl.batch, Lmax)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
        calls = [K.bound_call("kvq_decode_partials", prm, c.struct, n_new, Lmax, q, K.KVQ_BF16, 0.0, ws, wsb,
                              stream=stream) for c in copies]
        warm = time_calls(torch, calls[:1], reps, stream)
        cold = time_rotating(torch, calls, reps, stream)
        plan(f"paged K{kb}V{vb}: warm", 1 + reps, 1)
        plan(f"paged K{kb}V{vb}: cold", n_cp + reps, n_cp)
        comb = time_calls(torch, [K.bound_call("kvq_decode_combine", prm, wl.batch, Lmax, K.KVQ_BF16, ws, out,
                                               K.KVQ_F32, stream=stream)], reps, stream)
        splits = K.kvq_decode_splits(prm, wl.batch, Lmax, K.KVQ_BF16)
        old_env = os.environ.get("KVQ_PAGES_PER_SPLIT")
        os.environ["KVQ_PAGES_PER_SPLIT"] = "32"
        try:
            wsb2 = K.kvq_decode_workspace_bytes(prm, wl.batch, Lmax)
            ws2 = torch.empty(wsb2, dtype=torch.uint8, device=dev)
            calls2 = [K.bound_call("kvq_decode_partials", prm, c.struct, n_new, Lmax, q, K.KVQ_BF16, 0.0, ws2, wsb2,
                                   stream=stream) for c in copies]
            cold_uniform = time_rotating(torch, calls2, reps, stream)
            plan(f"paged K{kb}V{vb}: cold, uniform plan", n_cp + reps, n_cp)
        finally:
            if old_env is None:
                os.environ.pop("KVQ_PAGES_PER_SPLIT", None)
            else:
                os.environ["KVQ_PAGES_PER_SPLIT"] = old_env
        rf = kernel_roofline(cold, warm, nbytes, ceiling_GBs)
        rf["frac_of_size_matched_stream_ceiling_cold"] = round(nbytes / cold / 1e3 / small_ceiling["best"]["cold_GBs"], 4)
        rows.append(dict(k_bits=kb, v_bits=vb, row_stride_splits=splits, combine_us=round(comb, 2),
                         traffic=stored_traffic(f"paged K{kb}V{vb}: cold"),
                         uniform_plan_us_cold=round(cold_uniform, 2),
                         uniform_plan_frac_cold=round(nbytes / cold_uniform / 1e3 / PEAK_HBM_GBS, 4), **rf))
        del copies, calls, calls2, ws2
        # error-budget diagnostics on the same cache
        hs = torch.empty((wl.batch, wl.num_q_heads, K.KVQ_EB_HEAD), dtype=torch.float32, device=dev)
        us = torch.empty((wl.batch, wl.num_kv_heads, K.KVQ_EB_UNIT), dtype=torch.float32, device=dev)
        ewsb = K.kvq_error_budget_workspace_bytes(prm, wl.batch, Lmax)
        ews = torch.empty(ewsb, dtype=torch.uint8, device=dev)
        K.kvq_error_budget(prm, cb.struct, n_new, Lmax, k_ref, v_ref, q, K.KVQ_BF16, 0.0, hs, us, ews, ewsb)
        torch.cuda.synchronize()
        h_ = hs.cpu().numpy().astype(np.float64)
        u_ = us.cpu().numpy().astype(np.float64)
        eb_rows.append({
            "k_bits": kb, "v_bits": vb, "payload_bits_per_key_value_pair": kb + vb,
            "rel_reconstruction_error_keys": round(float(np.sqrt(u_[..., 0].sum() / u_[..., 4].sum())), 4),
            "rel_reconstruction_error_values": round(float(np.sqrt(u_[..., 1].sum() / u_[..., 5].sum())), 4),
            "median_rms_score_error": round(float(np.median(h_[..., 1])), 4),
            "median_weight_total_variation": round(float(np.median(h_[..., 2])), 4),
            "median_rel_output_error_values_only": round(float(np.median(h_[..., 3] / h_[..., 6])), 4),
            "median_rel_output_error_keys_only": round(float(np.median(h_[..., 4] / h_[..., 6])), 4),
            "median_rel_output_error_both": round(float(np.median(h_[..., 5] / h_[..., 6])), 4),
        })
        del cb, k_ref, v_ref, table, ws
        torch.cuda.synchronize()
    wl = W.WORKLOADS[4]
    sweep = {"workload": wl.name, "lengths": [int(x) for x in wl.context_lengths()],
             "what": "kvq_decode_partials (split kernel, read-only) per bit pair; algorithmic bytes = codes and "
                     "metadata of every stored token-head + block-table entries + queries; cold: cycling over copies "
                     "of the page pool; uniform plan: every split sized from the longest sequence; "
                     "frac_of_stream_ceiling_cold against the 32k decode step's streaming ceiling, "
                     "frac_of_size_matched_stream_ceiling_cold against stream_ceiling_at_this_size (the "
                     "read-only streaming kernel over the K4V2 launch's byte count)",
             "stream_ceiling_at_this_size": small_ceiling, "rows": rows}
    ebs = {"workload": wl.name, "query": "decode step 0", "rows": eb_rows}
    return sweep, ebs


def rotated_131k(torch, dev, reps, stream, ceiling_GBs, plan):
    """The batch-64 x 131072-token workload with rotated keys (64 query / 8 kv heads): bulk prefill of
    the whole context (appends of 4096 tokens per sequence back to back, all inputs generated into
    HBM first), then the decode attention's split kernel timed back to back on two copies of
    the 7.8 GB cache (cold: every launch reads data far beyond the Infinity Cache) and the merge."""
    import mixed_precision_kv_kvq_amd as K
    import workloads as W
    from workloads.device import DeviceGenerator

    wl = W.WORKLOADS[5]
    B, Hq, Hkv, d, L = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.context
    prm = K.make_params(d, Hq, Hkv, wl.k_bits, wl.k_group, wl.v_bits, wl.v_group, 0, 1, K.KVQ_BF16, 0)
    cb = K.CacheBuffers(prm, B, L)
    gen = DeviceGenerator(wl)
    chunk = 4096
    # every chunk's rows generated into HBM first (34.4 GB of bf16 keys and values), then the
    # appends back to back between two events, arguments marshalled beforehand
    pre = []
    for t0 in range(0, L, chunk):
        pre.append((gen.kv(W.TENSOR_K, t0, chunk), gen.kv(W.TENSOR_V, t0, chunk),
                    torch.full((B,), t0, dtype=torch.int32, device=dev)))
    calls = [K.bound_call("kvq_quantize_append", prm, cb.struct, before, None, k, v, chunk, stream=stream)
             for k, v, before in pre]
    progress(f"rotated 131k: {len(pre)} chunks of inputs generated")
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    e[0].record(stream)
    for f in calls:
        f()
    e[1].record(stream)
    torch.cuda.synchronize()
    app_us = e[0].elapsed_time(e[1]) * 1e3
    del pre, calls
    per_th = d * wl.k_bits // 8 + (d // wl.k_group) * 4 + d * wl.v_bits // 8 + (d // wl.v_group) * 4
    prefill_bytes = B * Hkv * L * (2 * d * 2 + per_th)  # every row read once, its codes written once
    q = gen.q(0)
    lens = torch.full((B,), L, dtype=torch.int32, device=dev)
    nbytes = B * Hkv * L * per_th + B * Hq * d * 2
    copies = [cb, clone_cache(K, torch, cb, prm, B, L)]
    wsb = K.kvq_decode_workspace_bytes(prm, B, L)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.int16, device=dev)
    calls = [K.bound_call("kvq_decode_partials", prm, c.struct, lens, L, q, K.KVQ_BF16, 0.0, ws, wsb, stream=stream)
             for c in copies]
    cold = time_rotating(torch, calls, reps, stream)
    plan("rotated 131k: cold", 2 + reps, 2)
    warm = time_calls(torch, calls[:1], reps, stream)
    plan("rotated 131k: warm", 1 + reps, 1)
    comb = time_calls(torch, [K.bound_call("kvq_decode_combine", prm, B, L, K.KVQ_BF16, ws, out, K.KVQ_BF16,
                                           stream=stream)], reps, stream)
    del copies, calls, cb, ws
    torch.cuda.synchronize()
    rf = kernel_roofline(cold, warm, nbytes, ceiling_GBs)
    rf["traffic"] = stored_traffic("rotated 131k: cold")
    return {"workload": wl.name, "what": "kvq_decode_partials (split kernel, read-only, rotated query) + "
                                         "kvq_decode_combine (bf16 output); algorithmic bytes = codes and metadata "
                                         "of every token-head + queries",
            "split_kernel": rf, "combine_us": round(comb, 2), "attention_us_cold": round(cold + comb, 2),
            "effective_tokens_per_s": round(B * L / ((cold + comb) * 1e-6), 1),
            "prefill_quantize": {"what": f"{L // chunk} appends of {chunk} tokens per sequence (key rotation, fp64 "
                                         f"quantizer) back to back between two events, every chunk's inputs "
                                         f"generated into HBM before", "us": round(app_us, 1),
                                 "algorithmic_bytes": int(prefill_bytes),
                                 "achieved_GBs": round(prefill_bytes / app_us / 1e3, 1),
                                 "frac_of_peak": round(prefill_bytes / app_us / 1e3 / PEAK_HBM_GBS, 4)}}


# --------------------------------------------------------------------------------------------
# Timing helpers (HIP events on the launch stream)
# --------------------------------------------------------------------------------------------
def time_calls(torch, calls, reps, stream, warm=1):
    """Average µs per repetition of the call list, launched back to back between two events."""
    for _ in range(warm):
        for f in calls:
            f()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    e[0].record(stream)
    for _ in range(reps):
        for f in calls:
            f()
    e[1].record(stream)
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) * 1e3 / reps


def time_rotating(torch, calls, reps, stream):
    """Average µs per launch of reps launches cycling through `calls` (one launch each), back to
    back between two events.  With calls over distinct buffers whose total is well above the
    256 MB Infinity Cache, every launch reads data evicted since its previous use ("cold")."""
    for f in calls:  # first touch
        f()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    e[0].record(stream)
    for i in range(reps):
        calls[i % len(calls)]()
    e[1].record(stream)
    torch.cuda.synchronize()
    return e[0].elapsed_time(e[1]) * 1e3 / reps


def copies_for(nbytes, floor=4):
    """Buffers to rotate over so that between two uses of one buffer at least 1.5 GiB of other
    data is read (six times the Infinity Cache)."""
    return max(floor, -(-int(1.5 * 2 ** 30) // max(int(nbytes), 1)) + 1)


def clone_cache(K, torch, src, params, batch, capacity, table=None):
    """An independent copy of a cache's buffers (same contents)."""
    c = K.CacheBuffers(params, batch, capacity, table)
    c.pages.copy_(src.pages)
    if src.k_win is not None:
        c.k_win.copy_(src.k_win)
        c.v_win.copy_(src.v_win)
    return c


def stream_ceiling(torch, nbytes, stream, reps=20):
    """Read-only streaming of nbytes per launch (kvq_gen_stream_read), cold (rotating over
    buffers well above the Infinity Cache) and warm (one buffer), for a few launch widths and
    both load kinds; the best cold rate is the practical ceiling of a read-once kernel."""
    from workloads.device import stream_read_call

    n = copies_for(nbytes)
    nbytes = (int(nbytes) // 16) * 16
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n)]
    for b_ in bufs:
        b_.fill_(1)
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    rows = []
    for blocks in (1024, 2048, 4096, 8192):
        for nt in (0, 1):
            calls = [stream_read_call(b_, nbytes, sink, blocks, bool(nt), stream) for b_ in bufs]
            cold = time_rotating(torch, calls, reps, stream)
            warm = time_calls(torch, calls[:1], reps, stream)
            rows.append({"blocks": blocks, "nontemporal": bool(nt), "cold_us": round(cold, 2),
                         "cold_GBs": round(nbytes / cold / 1e3, 1), "warm_us": round(warm, 2),
                         "warm_GBs": round(nbytes / warm / 1e3, 1)})
    del bufs
    best = max(rows, key=lambda r: r["cold_GBs"])
    return {"bytes_per_launch": nbytes, "buffers": n, "best": best, "sweep": rows}


def kernel_roofline(cold_us, warm_us, nbytes, ceiling_GBs):
    cold = nbytes / cold_us / 1e3
    warm = nbytes / warm_us / 1e3
    return {"us_cold": round(cold_us, 2), "us_warm": round(warm_us, 2), "algorithmic_bytes": int(nbytes),
            "GBs_cold": round(cold, 1), "GBs_warm": round(warm, 1), "frac_cold": round(cold / PEAK_HBM_GBS, 4),
            "frac_warm": round(warm / PEAK_HBM_GBS, 4),
            "frac_of_stream_ceiling_cold": round(cold / ceiling_GBs, 4) if ceiling_GBs else None}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--reps", type=int, default=20, help="launches per kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the timed steps")
    ap.add_argument("--no-unfused", action="store_true",
                    help="skip the unfused baseline and the error-budget diagnostics")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads (paged bit-width sweep, rotated 131k batch 64)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device copy of this many MiB before the steps (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "BENCH_JSON", "COPY_MIB"),
                    help="write the split kernel's per-launch HBM traffic from two --pmc runs and exit")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "BENCH_JSON", "OUT_MD", "COMMAND"),
                    help="per-phase split-kernel durations of a --kernel-trace run of this script, and exit")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.summarize_pmc[2],
                      int(args.summarize_pmc[3]) << 20)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path shards over (sequence, kv head) "
                                   "units across GPUs by design but no multi-GPU run is part of this build",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import workloads as W

    wl = W.WORKLOADS[3]
    # The oracle baseline runs first, in forked single-threaded workers, before this process
    # touches the GPU.
    cpu_res = None if args.no_cpu_baseline else cpu_baseline(wl, args.cpu_seconds)
    if cpu_res is not None:
        progress(f"oracle baseline: {cpu_res['value']} {cpu_res['unit']}")

    import numpy as np
    import torch

    import mixed_precision_kv_kvq_amd as K
    from workloads.device import DeviceGenerator

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    B, Hq, Hkv, d, R = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.window
    L0 = wl.context
    total_steps = args.warmup + 2 * args.steps  # fused steps, then as many through separate launches
    params = K.make_params(d, Hq, Hkv, wl.k_bits, wl.k_group, wl.v_bits, wl.v_group, R, 0, K.KVQ_BF16, 0)
    cap = L0 + total_steps
    cache = K.CacheBuffers(params, B, cap)
    gen = DeviceGenerator(wl)
    stream = torch.cuda.current_stream()
    reps = args.reps

    # ---- set-up: prefill the cache with the context (bulk append + quantize, timed apart) ----
    t_setup = time.time()
    chunk = 2048
    # all prefill inputs generated into HBM first (2.1 GB of bf16 rows), then the appends
    # back to back between two events
    pre = []
    for t0 in range(0, L0, chunk):
        n = min(chunk, L0 - t0)
        pre.append((t0, n, gen.kv(W.TENSOR_K, t0, n), gen.kv(W.TENSOR_V, t0, n),
                    torch.full((B,), t0, dtype=torch.int32, device=dev)))
    prefill_bytes = sum(append_bytes(wl, t0, n) for t0, n, _, _, _ in pre)
    # arguments marshalled before timing, so the launches reach the GPU back to back; the library's
    # first kernel launch in a process loads its code object (about a millisecond), so one untimed
    # append to a scratch cache comes first
    warm_cache = K.CacheBuffers(params, B, 64)
    K.kvq_quantize_append(params, warm_cache.struct, pre[0][4], None, pre[0][2], pre[0][3], 16)
    torch.cuda.synchronize()
    del warm_cache
    pre_calls = [K.bound_call("kvq_quantize_append", params, cache.struct, before, None, k, v, n, stream=stream)
                 for t0, n, k, v, before in pre]
    ev_p = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev_p[0].record(stream)
    for f in pre_calls:
        f()
    ev_p[1].record(stream)
    torch.cuda.synchronize()
    prefill_us = ev_p[0].elapsed_time(ev_p[1]) * 1e3
    progress(f"prefill of {L0} tokens: {prefill_us:.0f} us")
    del pre, pre_calls
    # per-step inputs, resident in HBM before timing
    k_steps = [gen.kv(W.TENSOR_K, L0 + s, 1) for s in range(total_steps)]
    v_steps = [gen.kv(W.TENSOR_V, L0 + s, 1) for s in range(total_steps)]
    q_steps = [gen.q(s) for s in range(total_steps)]
    lens = [torch.full((B,), L0 + s, dtype=torch.int32, device=dev) for s in range(total_steps + 1)]
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws_bytes = K.kvq_decode_workspace_bytes(params, B, cap)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)  # no initial contents needed
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    if args.copy_calibration_mib:
        # the generator library's plain copy kernel, reading and writing exactly N bytes each
        from workloads.device import stream_copy

        src = torch.zeros(args.copy_calibration_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            stream_copy(dst, src, src.numel(), stream)
        torch.cuda.synchronize()
        del src, dst

    # One decode step = kvq_decode_step: the split-K launch with the 1-token append fused in (the
    # split holding the new token's ring slot quantizes the token leaving the window), then the
    # cross-split merge.  kvq_decode_step_partials + kvq_decode_combine are exactly its two
    # launches; calling them apart lets HIP events bracket the split kernel alone.  The same steps
    # through separate launches (append kernel, kvq_decode_partials, kvq_decode_combine) are timed
    # next for comparison.  Arguments are marshalled before timing (bound_call), so the Python loop
    # stays ahead of the GPU.
    def step_fused(s, c=cache):
        return (
            K.bound_call("kvq_decode_step_partials", params, c.struct, lens[s], k_steps[s], v_steps[s], L0 + s + 1,
                         q_steps[s], K.KVQ_BF16, 0.0, ws, ws_bytes, stream=stream),
            K.bound_call("kvq_decode_combine", params, B, L0 + s + 1, K.KVQ_BF16, ws, out, K.KVQ_F32,
                         stream=stream),
        )

    def step_separate(s, c=cache):
        return (
            K.bound_call("kvq_quantize_append", params, c.struct, lens[s], None, k_steps[s], v_steps[s], 1,
                         stream=stream),
            K.bound_call("kvq_decode_partials", params, c.struct, lens[s + 1], L0 + s + 1, q_steps[s],
                         K.KVQ_BF16, 0.0, ws, ws_bytes, stream=stream),
            K.bound_call("kvq_decode_combine", params, B, L0 + s + 1, K.KVQ_BF16, ws, out, K.KVQ_F32,
                         stream=stream),
        )

    def run_steps(steps):
        """Wall-clock and event µs per step of back-to-back steps (no event between launches: on
        this runtime an event record delays the next dispatch by a few microseconds)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for st_ in steps:
            for f in st_:
                f()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / len(steps) * 1e6, ev[0].elapsed_time(ev[1]) * 1e3 / len(steps)

    dispatch_plan = []  # split-kernel launches of each phase, in launch order (for kernel traces)

    def plan(phase, launches, untimed_first=0):
        dispatch_plan.append({"phase": phase, "launches": int(launches), "untimed_first": int(untimed_first)})
        progress(f"done: {phase}")

    for s in range(args.warmup):
        for f in step_fused(s):
            f()
    plan("warm-up fused steps", args.warmup, args.warmup)
    torch.cuda.synchronize()
    gclone = None if args.no_graph else clone_cache(K, torch, cache, params, B, cap)  # state before the timed steps

    # ---- timed region: K whole fused steps ----------------------------------------------
    us_per_step, gpu_us_per_step = run_steps([step_fused(args.warmup + i) for i in range(args.steps)])
    plan("timed fused steps", args.steps)
    s0 = args.warmup + args.steps
    sep_us_per_step, sep_gpu_us = run_steps([step_separate(s0 + i) for i in range(args.steps)])
    plan("timed separate-launch steps", args.steps)
    L_last = L0 + total_steps  # every sequence's length after the last step

    # ---- the timed fused steps captured once in a HIP graph and replayed on a copy of the cache
    # taken before them (the second replay repeats the same appends: the same work).
    graph_us_per_step = None
    if gclone is not None:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                s_ = args.warmup + i
                K.kvq_decode_step_partials(params, gclone.struct, lens[s_], k_steps[s_], v_steps[s_], L0 + s_ + 1,
                                           q_steps[s_], K.KVQ_BF16, 0.0, ws, ws_bytes)
                K.kvq_decode_combine(params, B, L0 + s_ + 1, K.KVQ_BF16, ws, out, K.KVQ_F32)
        g.replay()  # warm
        torch.cuda.synchronize()
        ev_g = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev_g[0].record(stream)
        g.replay()
        ev_g[1].record(stream)
        torch.cuda.synchronize()
        graph_us_per_step = ev_g[0].elapsed_time(ev_g[1]) * 1e3 / args.steps
        plan("graph replays of the fused steps", 2 * args.steps, args.steps)
        del g, gclone
        torch.cuda.synchronize()

    # ---- the dominant kernel alone, at the last step's state -----------------------------
    # The fused split kernel of a step at length L_last (append of the token at L_last - 1 + attention
    # over L_last tokens), run on copies of the cache (it rewrites a ring slot and one token of a
    # record each time: the same work on every repetition).  warm: repeated on one copy; cold:
    # cycling over copies whose total is far above the Infinity Cache, so every launch streams its
    # cache from HBM.  The attention-only split kernel (kvq_decode_partials, read-only) is timed the
    # same way.
    per_th = (d * wl.k_bits // 8 + (d // wl.k_group) * 4 + d * wl.v_bits // 8 + (d // wl.v_group) * 4)
    attn_bytes = split_kernel_bytes(wl, L_last, per_th, 2)
    # + per unit: the evicted row read from the ring and the new row written to it (the evicted
    # token's 116 B record write replaces its read in attn_bytes)
    launch_bytes = attn_bytes + B * Hkv * 2 * (2 * d * 2)
    n_cp = copies_for(launch_bytes)
    copies = [clone_cache(K, torch, cache, params, B, cap) for _ in range(n_cp)]
    torch.cuda.synchronize()
    sl = total_steps - 1
    fused_calls = [K.bound_call("kvq_decode_step_partials", params, c.struct, lens[sl], k_steps[sl], v_steps[sl],
                                L_last, q_steps[sl], K.KVQ_BF16, 0.0, ws, ws_bytes, stream=stream) for c in copies]
    attn_calls = [K.bound_call("kvq_decode_partials", params, c.struct, lens[-1], L_last, q_steps[-1], K.KVQ_BF16,
                               0.0, ws, ws_bytes, stream=stream) for c in copies]
    split_warm_us = time_calls(torch, fused_calls[:1], reps, stream)
    plan("fused split kernel, warm", 1 + reps, 1)
    split_cold_us = time_rotating(torch, fused_calls, reps, stream)
    plan("fused split kernel, cold", n_cp + reps, n_cp)
    attn_warm_us = time_calls(torch, attn_calls[:1], reps, stream)
    plan("attention-only split kernel, warm", 1 + reps, 1)
    attn_cold_us = time_rotating(torch, attn_calls, reps, stream)
    plan("attention-only split kernel, cold", n_cp + reps, n_cp)
    combine_call = K.bound_call("kvq_decode_combine", params, B, L_last, K.KVQ_BF16, ws, out, K.KVQ_F32,
                                stream=stream)
    combine_us = time_calls(torch, [combine_call], reps, stream)
    # the separate 1-token append (on a copy of the cache)
    app_call = K.bound_call("kvq_quantize_append", params, copies[0].struct, lens[sl], None, k_steps[sl],
                            v_steps[sl], 1, stream=stream)
    append_us = time_calls(torch, [app_call], reps, stream)
    del copies, fused_calls, attn_calls
    # restore the last step's output (merge of the last separate step's partials)
    for f in step_separate(total_steps - 1)[1:]:
        f()
    plan("restore the last step's output", 1)
    torch.cuda.synchronize()
    ceiling = stream_ceiling(torch, launch_bytes, stream, reps)
    ceil_GBs = ceiling["best"]["cold_GBs"]
    split_rf = kernel_roofline(split_cold_us, split_warm_us, launch_bytes, ceil_GBs)
    attn_rf = kernel_roofline(attn_cold_us, attn_warm_us, attn_bytes, ceil_GBs)

    # ---- unfused baseline at the last step's state: the fused attention (split kernel + merge)
    # against dequantize-to-dense-bf16 + dense attention over the same cache and query.
    unfused = None
    if not args.no_unfused:
        lens_last = lens[-1]
        q_last = q_steps[-1]
        kd = torch.empty((B, Hkv, L_last, d), dtype=torch.int16, device=dev)
        vd = torch.empty_like(kd)
        dws = K.kvq_dense_workspace_bytes(params, B, L_last)
        dw = torch.empty(dws, dtype=torch.uint8, device=dev)
        out_u = torch.empty_like(out)
        deq = K.bound_call("kvq_dequantize_dense", params, cache.struct, lens_last, L_last, kd, vd, stream=stream)
        dense = K.bound_call("kvq_dense_decode_attention", params, B, kd, vd, lens_last, L_last, q_last, K.KVQ_BF16,
                             out_u, K.KVQ_F32, 0.0, dw, dws, stream=stream)
        fused = step_separate(total_steps - 1)[1:]  # kvq_decode_partials + kvq_decode_combine
        fused_us = time_calls(torch, fused, 5, stream)
        plan("unfused comparison: fused attention", 6, 1)
        deq_us = time_calls(torch, [deq], 5, stream)
        dense_us = time_calls(torch, [dense], 5, stream)
        both_us = time_calls(torch, [deq, dense], 5, stream)
        fused[1]()
        torch.cuda.synchronize()
        diff = float((out_u - out).abs().max())
        units = B * Hkv
        nq_last = max(L_last - R, 0)
        deq_bytes = units * (nq_last * per_th + (L_last - nq_last) * 2 * d * 2 + L_last * 2 * d * 2)
        dense_bytes = units * L_last * 2 * d * 2
        unfused = {
            "what": "dequantize the whole cache to dense bf16 K/V (kvq_dequantize_dense), then dense decode "
                    "attention over it (kvq_dense_decode_attention, splits of 256 positions + the same merge); "
                    "fused = kvq_decode_partials + kvq_decode_combine; last step's state, 5 back-to-back "
                    "repetitions between two events each",
            "length": L_last,
            "fused_attention_us": round(fused_us, 2),
            "unfused_us": round(both_us, 2),
            "dequantize_us": round(deq_us, 2), "dequantize_bytes": int(deq_bytes),
            "dequantize_GBs": round(deq_bytes / (deq_us * 1e-6) / 1e9, 1),
            "dense_attention_us": round(dense_us, 2), "dense_attention_bytes": int(dense_bytes),
            "dense_attention_GBs": round(dense_bytes / (dense_us * 1e-6) / 1e9, 1),
            "fusion_speedup": round(both_us / fused_us, 2),
            "max_abs_output_difference": diff,
        }
        del kd, vd, dw
        torch.cuda.synchronize()

    # ---- error-budget diagnostics at the last step's state, against the original rows ----
    errb = None
    if not args.no_unfused:
        lens_last = lens[-1]
        q_last = q_steps[-1]
        k_ref = gen.kv(W.TENSOR_K, 0, L_last)
        v_ref = gen.kv(W.TENSOR_V, 0, L_last)
        hs = torch.empty((B, Hq, K.KVQ_EB_HEAD), dtype=torch.float32, device=dev)
        us = torch.empty((B, Hkv, K.KVQ_EB_UNIT), dtype=torch.float32, device=dev)
        ewsb = K.kvq_error_budget_workspace_bytes(params, B, L_last)
        ews = torch.empty(ewsb, dtype=torch.uint8, device=dev)
        eb = K.bound_call("kvq_error_budget", params, cache.struct, lens_last, L_last, k_ref, v_ref, q_last,
                          K.KVQ_BF16, 0.0, hs, us, ews, ewsb, stream=stream)
        eb_us = time_calls(torch, [eb], 3, stream)
        h_ = hs.cpu().numpy().astype(np.float64)
        u_ = us.cpu().numpy().astype(np.float64)
        nq_last = max(L_last - R, 0)
        eb_bytes = B * Hkv * (L_last * 2 * d * 2 + nq_last * per_th)  # originals and the store, read once
        errb = {
            "what": "kvq_error_budget at the last step's state against the original bf16 rows, 3 launches "
                    "between two events",
            "us": round(eb_us, 1), "unit_bytes_read_once": int(eb_bytes),
            "GBs_vs_read_once": round(eb_bytes / (eb_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(eb_bytes / (eb_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "median_over_heads": {
                "max_score_error": float(np.median(h_[..., 0])), "rms_score_error": float(np.median(h_[..., 1])),
                "weight_total_variation": float(np.median(h_[..., 2])),
                "output_error_values_only": float(np.median(h_[..., 3])),
                "output_error_keys_only": float(np.median(h_[..., 4])),
                "output_error_both": float(np.median(h_[..., 5])), "output_norm": float(np.median(h_[..., 6]))},
            "relative_reconstruction_error": {
                "keys": float(np.sqrt(u_[..., 0].sum() / u_[..., 4].sum())),
                "values": float(np.sqrt(u_[..., 1].sum() / u_[..., 5].sum()))},
        }
        del k_ref, v_ref
        torch.cuda.synchronize()

    traffic = stored_traffic("fused split kernel, cold")

    step_cold_us = split_cold_us + combine_us  # the two launches of a cold decode step
    res = {
        "metric": METRIC,
        "value": round(us_per_step, 2),
        "unit": "µs/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1000.0, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded SplitMix64 normal-quantile generator; key channel std log-normal(0,0.5), "
                "3 outlier channels x10 per kv head)",
        "config": {"workload": f"b16-gqa32x8-L{L0}-win{R}-{args.warmup}+{args.steps}steps", "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": d, "context": L0, "window": R, "k_bits": wl.k_bits,
                   "k_group": wl.k_group, "v_bits": wl.v_bits, "v_group": wl.v_group,
                   "step": "kvq_decode_step: append 1 token/sequence fused into the split-K attention launch, "
                           "then the merge launch"},
        "gpu_us_per_step": round(gpu_us_per_step, 2),
        "graph_us_per_step": None if graph_us_per_step is None else round(graph_us_per_step, 2),
        "separate_launch_step": {"what": "the same steps as append kernel + kvq_decode_partials + "
                                         "kvq_decode_combine (three launches), the next K steps",
                                 "us_per_step": round(sep_us_per_step, 2), "gpu_us_per_step": round(sep_gpu_us, 2)},
        "split_kernel_us_cold": round(split_cold_us, 2),
        "split_kernel_us_warm": round(split_warm_us, 2),
        "attention_split_kernel": dict(attn_rf, what="kvq_decode_partials at the same length (attention only, "
                                                     "read-only)",
                                       traffic=stored_traffic("attention-only split kernel, cold")),
        "combine_us": round(combine_us, 2),
        "decode_append_us_separate_kernel": round(append_us, 2),
        "tokens_per_s": round(B / (us_per_step * 1e-6), 1),
        "effective_tokens_per_s": round(B * L_last / (step_cold_us * 1e-6), 1),
        "effective_tokens_per_s_step": round(B * L_last / (us_per_step * 1e-6), 1),
        "roofline": {"kernel": SPLIT_KERNEL + " (decode step: split-K attention with the 1-token append fused in)",
                     "bound": "hbm", "achieved": split_rf["GBs_cold"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": split_rf["frac_cold"], "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(launch_bytes),
                     "timing": f"cold: {reps} back-to-back launches of a step's split kernel at L={L_last} cycling "
                               f"over {n_cp} copies of the cache ({n_cp * launch_bytes / 1e9:.2f} GB, far above "
                               f"the 256 MB Infinity Cache), between two events",
                     "achieved_warm": split_rf["GBs_warm"], "frac_warm": split_rf["frac_warm"],
                     "stream_ceiling_GBs": ceil_GBs, "stream_ceiling_frac": round(ceil_GBs / PEAK_HBM_GBS, 4),
                     "frac_of_stream_ceiling": split_rf["frac_of_stream_ceiling_cold"]},
        "stream_ceiling": ceiling,
        "setup_s": round(setup_s, 2),
        "prefill_quantize": {
            "what": f"bulk append + quantize of the {L0}-token context, {(L0 + chunk - 1) // chunk} appends of "
                    f"{chunk} tokens per sequence (kvq_quantize_append, arguments marshalled beforehand) back to "
                    f"back between two events, inputs already in HBM",
            "us": round(prefill_us, 1), "algorithmic_bytes": int(prefill_bytes),
            "achieved_GBs": round(prefill_bytes / (prefill_us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(prefill_bytes / (prefill_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "tokens_per_s": round(B * L0 / (prefill_us * 1e-6), 1)},
    }
    if unfused is not None:
        res["unfused_baseline"] = unfused
    if errb is not None:
        res["error_budget"] = errb
    if not args.no_extra:
        sweep, ebs = paged_sweep(torch, dev, reps, stream, ceil_GBs, plan)
        res["paged_sweep"] = sweep
        res["error_budget_bit_pairs"] = ebs
        res["rotated_131k"] = rotated_131k(torch, dev, reps, stream, ceil_GBs, plan)
    if cpu_res is not None:
        res["cpu_baseline"] = cpu_res
    res["split_kernel_dispatch_plan"] = dispatch_plan
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
