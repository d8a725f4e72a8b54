"""Host code of the C-ABI front end (csrc/kvq_api.cpp: validation, sizing, split plans, launch
set-up) built for the host only with AddressSanitizer and UndefinedBehaviorSanitizer, the device
launches replaced by stubs that touch the first and last workspace element their kernels address
(tests/sanitize/launch_stubs.cpp), and driven through every entry point by
tests/sanitize/abi_driver.cpp: valid calls, one broken argument at a time, extreme sizes.  The
workspace sizes the sanitized build computes are compared with the real library's, which pins
the stubs' copies of the error-budget plan constants to the kernels'.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")

FLAGS = ["-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include")]
# host-only HIP compiles: every sanitizer flag applies to the host pass only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    d = tmp_path_factory.mktemp("kvq_sanitized")
    api = os.path.join(ROOT, "mixed_precision_kv_kvq_amd", "csrc", "kvq_api.cpp")
    stubs = os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp")
    drv = os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")
    steps = [
        [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", *FLAGS, *HOST_SAN, "-c", api, "-o", str(d / "api.o")],
        [HIPCC, "--offload-arch=gfx950", "--cuda-host-only", *FLAGS, *HOST_SAN, "-c", stubs, "-o", str(d / "stubs.o")],
        [CLANG, *FLAGS, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-x", "c++", "-c", drv, "-o", str(d / "driver.o")],
        [CLANG, "-fsanitize=address,undefined", str(d / "api.o"), str(d / "stubs.o"), str(d / "driver.o"), "-o",
         str(d / "abi_driver")],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-3000:]}"
    return str(d / "abi_driver")


def test_abi_host_paths_clean_under_asan_and_ubsan(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.strip().splitlines()[-1].startswith("ok ")


def test_sanitized_sizes_match_the_library(driver):
    import mixed_precision_kv_kvq_amd as K

    r = subprocess.run([driver], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    fns = {"decode": K.kvq_decode_workspace_bytes, "dense": K.kvq_dense_workspace_bytes,
           "errbudget": K.kvq_error_budget_workspace_bytes}
    seen = set()
    for line in r.stdout.splitlines():
        f = line.split()
        if f[0] not in fns:
            continue
        hq, hkv, kb, kg, vb, vg, win, rot, dt, blk, vrot, batch, max_len, nbytes = map(int, f[1:])
        prm = K.make_params(128, hq, hkv, kb, kg, vb, vg, win, rot, dt, blk, value_rotation=vrot)
        assert fns[f[0]](prm, batch, max_len) == nbytes, line
        seen.add(f[0])
    assert seen == set(fns)
