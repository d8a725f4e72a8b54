"""GPU parity of the decode step with the append fused into the attention launch
(kvq_decode_step): after every step the stored codes and fp16 metadata equal the oracle's bit for
bit (the token that left the window is quantized inside the split kernel by the same fp64
sequence as the append kernels) and the outputs are within the tolerance of the oracle's exact
attention over the cache including the new token.

Cases cover the ring filling up (no token leaves the window until the length reaches R), the
evicted token landing on page and page-pair boundaries (where the quantized splits' last pair
ends), empty sequences in a batch, rotated keys, eight query heads per kv head, other bit widths
and group sizes, paged storage, and the configurations that run the append kernel first (no
window, fp32 rings)."""
import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mixed_precision_kv_kvq_amd as K  # noqa: E402
import workloads as W  # noqa: E402
from kvq_harness import GpuRun, assert_close, compare_codes, oracle_heads, oracle_unit, small  # noqa: E402


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def check_step(run: GpuRun, step: int, o32: np.ndarray):
    wl = run.wl
    g = wl.group_q
    got, ref = [], []
    for b in range(wl.batch):
        L = int(run.current_lengths()[b])
        rb = run.readback(b, 0, L) if L > 0 else None
        for h in range(wl.num_kv_heads):
            cache, Kx, Vx = oracle_unit(run, b, h)
            if rb is not None:
                compare_codes(run, b, h, cache, Kx, Vx, rb)
            ref.append(oracle_heads(run, cache, b, h, step) if L > 0 else np.zeros((g, wl.head_dim)))
            got.append(o32[b, h * g:(h + 1) * g])
    return assert_close(np.concatenate(got), np.concatenate(ref), f"{wl.name} step {step}")


B3 = W.WORKLOADS[3]
CASES = {
    # config-3 shape at reduced size: every step evicts one token into the store
    "cfg3-reduced": small(B3, batch=2, context=1000, steps=5),
    # the ring fills during the run: lengths 125..130 with R = 128
    "ring-fills": small(B3, batch=2, context=125, steps=6),
    # short sequences, window longer than all of them (no eviction at all)
    "window-longer": small(B3, batch=2, context=40, steps=3),
    # evicted positions 16*k - 1 .. 16*k + 2: the last pair ends on a page, then on a pair boundary
    "page-boundary": small(B3, batch=2, context=128 + 30, steps=5),
    "pair-boundary": small(B3, batch=1, context=128 + 62, steps=4),
    # ragged lengths with an empty sequence
    "ragged-with-empty": small(B3, batch=3, context=0, var_len=(0, 400), steps=3),
    "key-rotation": small(B3, batch=2, context=700, steps=3, rotation=True),
    "g8-vgroup64": small(B3, batch=2, num_q_heads=16, num_kv_heads=2, context=600, steps=3, v_group=64),
    "k8v8-kgroup64": small(B3, batch=2, context=500, steps=3, k_bits=8, v_bits=8, k_group=64),
    "k1v1-window16": small(B3, batch=2, context=300, steps=4, k_bits=1, v_bits=1, window=16),
    "window-200": small(B3, batch=2, context=900, steps=3, window=200),  # two window splits
    "paged-window": small(B3, batch=3, context=0, var_len=(200, 700), steps=3, block_size=16, window=32),
    # codes of 3, 5 and 6 bits (bit planes) quantized inside the split kernel
    "k3v2-window32": small(B3, batch=2, context=400, steps=4, k_bits=3, v_bits=2, window=32),
    "k5v3-rotation": small(B3, batch=2, context=500, steps=3, k_bits=5, v_bits=3, rotation=True),
    "k6v2-g8-vgroup64": small(B3, batch=2, num_q_heads=16, num_kv_heads=2, context=300, steps=3, k_bits=6, v_bits=2,
                              v_group=64),
    "k5v6-paged-window": small(B3, batch=3, context=0, var_len=(100, 500), steps=3, block_size=16, window=16,
                               k_bits=5, v_bits=6),
    # append kernel first, then attention (no fusion): no window, and fp32 rings
    "no-window": small(B3, batch=2, context=500, steps=3, window=0),
    "f32-window": small(B3, batch=2, context=500, steps=3, kv_dtype="f32", q_dtype="f32"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_step_matches_oracle(name):
    wl = CASES[name]
    say(f"fused step {name}")
    run = GpuRun(wl)
    for step in range(wl.steps):
        o = run.decode_step(step, phases=(step % 2 == 1))
        check_step(run, step, o)


def test_fused_step_equals_separate_launches():
    """The fused step and append + attention give the same stored cache, and outputs within the
    tolerance of each other (the evicted token is attended by another split, so the fp32
    summation order differs); the fused step's bf16 output is RNE of its fp32 output."""
    wl = small(B3, batch=2, context=800, steps=3)
    say("fused vs separate")
    a, b = GpuRun(wl, device_gen=True), GpuRun(wl, device_gen=True)
    for step in range(wl.steps):
        oa = a.decode_step(step)
        ob = b.decode(step)
        assert_close(oa, ob, f"fused vs separate step {step}")
        L = int(a.current_lengths()[0])
        ra, rb = a.readback(1, 0, L), b.readback(1, 0, L)
        for key in ("k_codes", "v_codes", "k_meta", "v_meta"):
            assert np.array_equal(ra[key], rb[key]), key
    # bf16 output: the same next step, fused, from the two (identical) states
    o32 = a.decode_step(wl.steps)
    ob16 = b.decode_step(wl.steps, out_dtype="bf16")
    rne = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o32))
    assert np.array_equal(ob16, rne), "bf16 output is not RNE of the fp32 output"


def test_fused_step_under_graph_replay():
    """A captured fused step, replayed several times with the cache restored to the state before
    the step (eager copies and synchronizations between replays), equals the eager step."""
    wl = small(B3, batch=2, context=600, steps=1)
    say("fused step graph replay")
    run = GpuRun(wl, device_gen=True)
    snap = [t.clone() for t in (run.cache.pages, run.cache.k_win, run.cache.v_win)]
    pos = run.current_lengths()
    k = run._rows_at(W.TENSOR_K, pos)
    v = run._rows_at(W.TENSOR_V, pos)
    before = torch.from_numpy(pos.astype(np.int32)).cuda()
    max_len = int(pos.max()) + 1
    wsb = K.kvq_decode_workspace_bytes(run.params, wl.batch, max_len)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    q = run._q_dev(0)
    K.kvq_decode_step(run.params, run.cache.struct, before, k, v, max_len, q, K.KVQ_BF16, out, K.KVQ_F32, 0.0, ws,
                      wsb)
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            K.kvq_decode_step(run.params, run.cache.struct, before, k, v, max_len, q, K.KVQ_BF16, out, K.KVQ_F32,
                              0.0, ws, wsb, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        for dst, src in zip((run.cache.pages, run.cache.k_win, run.cache.v_win), snap):
            dst.copy_(src)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
