"""GPU parity of the error-budget diagnostics (kvq_error_budget), through the C ABI, against
the oracle's error_budget on the same seeded inputs: per (sequence, query head) the score-error,
weight and output-error statistics, per (sequence, kv head) the reconstruction errors.  The
kernel works in fp32 (reconstructions rounded to fp32), the oracle in fp64: relative 2e-3 with a
small absolute floor."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mixed_precision_kv_kvq_amd as K  # noqa: E402
import oracle as O  # noqa: E402
import workloads as W  # noqa: E402
from kvq_harness import GpuRun, oracle_unit, small, to_device_kv  # noqa: E402

RTOL, ATOL = 2e-3, 2e-5

BASE = W.WORKLOADS[2]
CASES = {
    "k4v2-outliers": dict(context=700),
    "k4v4": dict(context=300, v_bits=4),
    "k2v2": dict(context=300, k_bits=2, v_bits=2),
    "k8v8": dict(context=200, k_bits=8, v_bits=8),
    "window-ragged": dict(context=300, window=40),
    "g8-vgroup64": dict(context=170, num_q_heads=16, num_kv_heads=2, v_group=64),
    "f32-query": dict(context=160, q_dtype="f32"),
    "g1": dict(context=150, num_q_heads=8, num_kv_heads=8),
    "rotated-keys-window": dict(context=260, window=24, rotation=True),
    "rotated-values": dict(context=230, value_rotation=True),
    "rotated-both-g8": dict(context=200, num_q_heads=16, num_kv_heads=2, rotation=True, value_rotation=True),
    "g2-window": dict(context=220, num_q_heads=16, num_kv_heads=8, window=24),
    "paged-window": dict(context=0, var_len=(1, 300), block_size=16, window=16, batch=4),
    "ragged-lengths-with-empty": dict(context=0, var_len=(0, 600), batch=4),
    "k3v2": dict(context=300, k_bits=3, v_bits=2),
    "k5v3-window": dict(context=280, window=24, k_bits=5, v_bits=3),
    "k6v5-rotated-both": dict(context=200, k_bits=6, v_bits=5, rotation=True, value_rotation=True),
}


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(CASES))
def test_error_budget_matches_oracle(name):
    wl = small(BASE, config=700 + list(CASES).index(name), **CASES[name])
    say(f"error budget {name}: {CASES[name]}")
    run = GpuRun(wl, chunk=64)
    L = run.current_lengths()
    B, Hkv, Hq, d, g = wl.batch, wl.num_kv_heads, wl.num_q_heads, wl.head_dim, wl.group_q
    max_len = max(int(L.max()), 1)
    k_ref = to_device_kv(wl.kv_batch_f32(W.TENSOR_K, 0, max_len), "bf16")
    v_ref = to_device_kv(wl.kv_batch_f32(W.TENSOR_V, 0, max_len), "bf16")
    seq_lens = torch.from_numpy(L.astype(np.int32)).cuda()
    hs = torch.full((B, Hq, K.KVQ_EB_HEAD), float("nan"), dtype=torch.float32, device="cuda")
    us = torch.full((B, Hkv, K.KVQ_EB_UNIT), float("nan"), dtype=torch.float32, device="cuda")
    qd = K.KVQ_F32 if wl.q_dtype == "f32" else K.KVQ_BF16
    wsb = K.kvq_error_budget_workspace_bytes(run.params, B, max_len)
    ws = torch.full((wsb // 4,), float("nan"), dtype=torch.float32, device="cuda")  # no field may be read unwritten
    K.kvq_error_budget(run.params, run.cache.struct, seq_lens, max_len, k_ref, v_ref, run._q_dev(0), qd, 0.0, hs, us,
                       ws, wsb)
    torch.cuda.synchronize()
    hs = hs.cpu().numpy().astype(np.float64)
    us = us.cpu().numpy().astype(np.float64)
    q = run.q_host(0).astype(np.float64)
    scale = 1.0 / np.sqrt(d)
    for b in range(B):
        for kvh in range(Hkv):
            cache, Kx, Vx = oracle_unit(run, b, kvh)
            for h in range(kvh * g, (kvh + 1) * g):
                head, unit = O.error_budget(q[b, h], Kx, Vx, cache, scale)
                np.testing.assert_allclose(hs[b, h], head, rtol=RTOL, atol=ATOL,
                                           err_msg=f"{name}: head stats (b {b}, head {h})")
            np.testing.assert_allclose(us[b, kvh], unit, rtol=RTOL, atol=ATOL,
                                       err_msg=f"{name}: unit stats (b {b}, kv head {kvh})")
