"""Build the HIP libraries in-tree with hipcc for gfx950.

* mixed_precision_kv_kvq_amd/libkvq.so — the quantized-KV attention library (C ABI in include/kvq.h)
* workloads/libkvqgen.so                — the device-side input generator (include/kvq_gen.h)

Usage:  python mixed_precision_kv_kvq_amd/build.py [--force] [--jobs N]
(run it as a file: importing the package loads the library it builds)
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import re
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")

EXTRA = os.environ.get("KVQ_EXTRA_FLAGS", "").split()

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    # no packed-fp32 VALU instructions anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    *EXTRA,
]

LIB = os.environ.get("KVQ_LIB_OUT") or os.path.join(PKG, "libkvq.so")
GEN_LIB = os.path.join(ROOT, "workloads", "libkvqgen.so")
BUILD_DIR = os.environ.get("KVQ_BUILD_DIR") or os.path.join(PKG, "_build")


# Bit widths of the split-kernel instantiations: kvq_attn_inst.hip is compiled once per pair
# (about a minute of compiler time each).  7-bit codes (three bit planes) are left out.
WIDTHS = (1, 2, 3, 4, 5, 6, 8)
ATTN_BITS = [(kb, vb) for kb in WIDTHS for vb in WIDTHS]


def _units():
    """Compile units: (source, object, extra flags)."""
    csrc = os.path.join(PKG, "csrc")
    units = []
    for src in sorted(glob.glob(os.path.join(csrc, "*.hip"))):
        if os.path.basename(src) == "kvq_attn_inst.hip":
            for kb, vb in ATTN_BITS:
                units.append((src, os.path.join(BUILD_DIR, f"kvq_attn_k{kb}v{vb}.o"),
                              [f"-DKVQ_KB={kb}", f"-DKVQ_VB={vb}", "-Rpass-analysis=kernel-resource-usage"]))
        else:
            units.append((src, os.path.join(BUILD_DIR, os.path.basename(src) + ".o"), []))
    api = os.path.join(csrc, "kvq_api.cpp")
    units.append((api, os.path.join(BUILD_DIR, "kvq_api.cpp.o"), []))
    headers = sorted(glob.glob(os.path.join(csrc, "*.h"))) + [os.path.join(ROOT, "include", "kvq.h")]
    return units, headers


def _run(cmd):
    t0 = time.time()
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; drop that harmless note.
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out, time.time() - t0


def _spills(out: str) -> list:
    """Split-kernel instantiations that use scratch, from -Rpass-analysis=kernel-resource-usage remarks."""
    bad, name = [], None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and "kvq_attn_split_kernel" in name and int(m.group(1)) > 0:
            bad.append((name, int(m.group(1))))
    return bad


def build(force: bool = True, jobs: int | None = None, verbose: bool = False) -> None:
    """Compile every HIP source for gfx950 and link the shared libraries."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    units, headers = _units()
    newest_header = max(os.path.getmtime(h) for h in headers)
    todo = []
    for src, obj, flags in units:
        if force or not os.path.exists(obj) or os.path.getmtime(obj) < max(os.path.getmtime(src), newest_header):
            todo.append((src, obj, flags))
    jobs = jobs or min(16, os.cpu_count() or 4)
    errors = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        # The attention instantiations report their register use; a spill there is a build error.
        futs = {ex.submit(_run, [HIPCC, *COMMON, *flags, "-c", src, "-o", obj]): (src, obj) for src, obj, flags in todo}
        for f in cf.as_completed(futs):
            rc, out, dt = f.result()
            src, obj = futs[f]
            spills = _spills(out)
            if verbose or rc:
                shown = "\n".join(l for l in out.splitlines() if "remark:" not in l)
                print(f"[build] {os.path.basename(obj)} rc={rc} {dt:.1f}s\n{shown}", file=sys.stderr)
            if spills:
                print(f"[build] {os.path.basename(obj)}: scratch in {spills}", file=sys.stderr)
                os.remove(obj)
            if rc or spills:
                errors.append(os.path.basename(obj))
    if errors:
        raise RuntimeError(f"hipcc failed for: {errors}")
    objs = [obj for _, obj, _ in units]
    if force or todo or not os.path.exists(LIB):
        rc, out, _ = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs])
        if rc:
            raise RuntimeError(f"link failed:\n{out}")
        os.replace(LIB + ".tmp", LIB)
    gen_src = os.path.join(ROOT, "workloads", "gen.hip")
    if force or not os.path.exists(GEN_LIB) or os.path.getmtime(GEN_LIB) < os.path.getmtime(gen_src):
        rc, out, _ = _run([HIPCC, *COMMON, "-shared", "-o", GEN_LIB + ".tmp", gen_src])
        if rc:
            raise RuntimeError(f"generator build failed:\n{out}")
        os.replace(GEN_LIB + ".tmp", GEN_LIB)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--force", action="store_true")
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    t = time.time()
    build(force=a.force, jobs=a.jobs, verbose=a.verbose)
    print(f"built {LIB} and {GEN_LIB} in {time.time() - t:.1f}s")
