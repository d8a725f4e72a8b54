"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Quantized codes, scales and zero points are compared bit for bit; attention
outputs (fp32) within max-abs 2e-3 and relative L2 1e-3 of the fp64 oracle
(the tolerance stated for this path, fp32 accumulation); bf16 outputs must
equal round-to-nearest-even of the same kernel's fp32 output.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _gpu_ok():
    return torch.cuda.is_available()


if not _gpu_ok():
    pytest.skip("needs a GPU", allow_module_level=True)

import mixed_precision_kv_kvq_amd as K  # noqa: E402
import workloads as W  # noqa: E402
from kvq_harness import (GpuRun, assert_close, compare_codes, oracle_heads, oracle_unit, small)  # noqa: E402


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def full_check(run: GpuRun, step: int, units=None, out_check_bf16=True):
    """Compare codes and outputs of the given (b, kvh) units (all units by default) at this step."""
    wl = run.wl
    o32 = run.decode(step, "f32")
    if out_check_bf16:
        ob = run.attend(torch.from_numpy(run.current_lengths().astype(np.int32)).cuda(),
                        int(run.current_lengths().max()), run._q_dev(step), "bf16")
        rne = W.bf16_bits_to_f32(W.f32_to_bf16_bits(o32))
        assert np.array_equal(ob, rne), "bf16 output is not RNE of the fp32 output"
    if units is None:
        units = [(b, h) for b in range(wl.batch) for h in range(wl.num_kv_heads)]
    g = wl.group_q
    got, ref = [], []
    rbs = {}
    for b, kvh in units:
        cache, Kx, Vx = oracle_unit(run, b, kvh)
        if b not in rbs:
            L = int(run.current_lengths()[b])
            rbs[b] = run.readback(b, 0, L) if L > 0 else None
        if rbs[b] is not None:
            compare_codes(run, b, kvh, cache, Kx, Vx, rbs[b])
        ref.append(oracle_heads(run, cache, b, kvh, step) if int(run.current_lengths()[b]) > 0
                   else np.zeros((g, wl.head_dim)))
        got.append(o32[b, kvh * g:(kvh + 1) * g])
    return assert_close(np.concatenate(got), np.concatenate(ref), f"{wl.name} step {step}")


# ---------------------------------------------------------------------------
def test_device_generator_matches_host():
    from workloads.device import DeviceGenerator

    for cfg in (1, 2, 5):
        wl = W.WORKLOADS[cfg]
        say(f"generator config {cfg}")
        dg = DeviceGenerator(wl)
        t0 = 1000
        k = dg.kv(W.TENSOR_K, t0, 3).cpu().numpy()
        v = dg.kv(W.TENSOR_V, t0, 3).cpu().numpy()
        q = dg.q(2).cpu().numpy()
        kh, vh, qh = wl.kv_batch_f32(W.TENSOR_K, t0, 3), wl.kv_batch_f32(W.TENSOR_V, t0, 3), wl.q_f32(2)
        if wl.kv_dtype == "bf16":
            kh, vh = W.f32_to_bf16_bits(kh).view(np.int16), W.f32_to_bf16_bits(vh).view(np.int16)
        if wl.q_dtype == "bf16":
            qh = W.f32_to_bf16_bits(qh).view(np.int16)
        assert np.array_equal(k, kh) and np.array_equal(v, vh) and np.array_equal(q, qh)


def test_config1_full():
    wl = W.WORKLOADS[1]
    say(f"config 1 {wl.name}")
    run = GpuRun(wl)
    full_check(run, 0)


def test_config2_full():
    wl = W.WORKLOADS[2]
    say(f"config 2 {wl.name}")
    run = GpuRun(wl)
    full_check(run, 0)


def test_config3_reduced_all_steps():
    """Config-3 structure (window 128, append per step) at a size the oracle covers fully."""
    wl = small(W.WORKLOADS[3], batch=2, context=1000, steps=5, config=103)
    say(f"config 3 reduced {wl}")
    run = GpuRun(wl, chunk=300)
    for s in range(wl.steps):
        full_check(run, s, out_check_bf16=(s == 0))


def test_config4_reduced_sweep():
    for kb, vb in W.SWEEP_BITS:
        wl = small(W.WORKLOADS[4], batch=3, var_len=(20, 700), config=104).with_bits(kb, vb)
        say(f"config 4 reduced K{kb}V{vb}")
        run = GpuRun(wl, chunk=256)
        full_check(run, 0)


def test_config5_reduced():
    wl = small(W.WORKLOADS[5], batch=2, context=1500, config=105)
    say("config 5 reduced")
    run = GpuRun(wl, chunk=512)
    full_check(run, 0)


# ---------------------------------------------------------------------------
# Edge cases (small, full comparison)
# ---------------------------------------------------------------------------
BASE = W.WORKLOADS[2]
EDGE = {
    "single-token": dict(context=1),
    "ragged-17": dict(context=17),
    "ragged-33": dict(context=33),
    "window-longer-than-seq": dict(context=50, window=128),
    "window-equal-seq": dict(context=128, window=128),
    "window-plus-one": dict(context=129, window=128),
    "window-ragged": dict(context=300, window=40),
    "k8v8": dict(context=200, k_bits=8, v_bits=8),
    "k1v1": dict(context=200, k_bits=1, v_bits=1),
    "k2v8": dict(context=90, k_bits=2, v_bits=8),
    "g1": dict(context=150, num_q_heads=8, num_kv_heads=8),
    "g2": dict(context=150, num_q_heads=16, num_kv_heads=8),
    "g8": dict(context=150, num_q_heads=16, num_kv_heads=2),
    "kgroup64-vgroup64": dict(context=150, k_group=64, v_group=64),
    "kgroup128": dict(context=150, k_group=128),
    "f32-kv-window": dict(context=160, window=20, kv_dtype="f32", q_dtype="f32"),
    "f32-q-bf16-kv": dict(context=160, q_dtype="f32"),
    "rotation-window": dict(context=200, window=24, rotation=True),
    "rotation-g8": dict(context=200, num_q_heads=16, num_kv_heads=2, rotation=True),
    "paged-window": dict(context=0, var_len=(1, 300), block_size=16, window=16, batch=4),
    "batch-var-contig": dict(context=0, var_len=(0, 90), batch=5),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_case(name):
    wl = small(BASE, config=200 + list(EDGE).index(name), **EDGE[name])
    say(f"edge {name}: {EDGE[name]}")
    run = GpuRun(wl, chunk=64)
    full_check(run, 0)


# The split plan is made per sequence on the device: a sequence's share of the launch follows its
# length.  Batches with very different lengths, empty sequences, more than 64 sequences (the plan's
# prefix sum runs over chunks of 64), windows, paged storage and decode steps.
RAGGED = {
    "long-and-short": dict(batch=4, context=0, var_len=(16, 6000)),
    "one-long-many-empty": dict(batch=6, context=0, var_len=(0, 1), lengths=[0, 1, 5000, 0, 17, 2]),
    "batch-70": dict(batch=70, num_q_heads=8, num_kv_heads=2, context=0, var_len=(0, 600)),
    "window-ragged-steps": dict(batch=3, context=0, var_len=(50, 3000), window=64, steps=3),
    "paged-ragged": dict(batch=5, context=0, var_len=(1, 4000), block_size=16),
    "g8-rotated-ragged": dict(batch=3, num_q_heads=16, num_kv_heads=2, context=0, var_len=(100, 3000),
                              rotation=True),
}


@pytest.mark.parametrize("name", list(RAGGED))
def test_ragged_split_plan(name):
    kw = dict(RAGGED[name])
    lengths = kw.pop("lengths", None)
    wl = small(BASE, config=400 + list(RAGGED).index(name), **kw)
    say(f"ragged plan {name}: {RAGGED[name]}")
    run = GpuRun(wl, chunk=1024, lengths=lengths)
    for s in range(max(wl.steps, 1)):  # steps == 0: one attention over the context
        full_check(run, s, out_check_bf16=(s == 0))


# Score operands with 8 or 16 (head, query part) rows (8 heads per kv head and/or a query in hi and
# lo parts) are laid out as those rows over whole 32-channel chunks, one accumulator per chunk: key
# groups of 32, 64 and 128 (the group scale of chunk r is group r / (group / 32)), ragged tails,
# bf16 and fp32 windows, decode steps through the fused step (the evicted token scored in the
# window split) and through the append kernel, rotated keys.
ROW_OPERAND = {
    "g8-kgroup64-vgroup64-window": dict(context=301, num_q_heads=16, num_kv_heads=2, k_group=64, v_group=64,
                                        window=40),
    "g8-f32q-kgroup128": dict(context=233, num_q_heads=16, num_kv_heads=2, q_dtype="f32", k_group=128),
    "g4-f32q-kgroup64-window": dict(context=187, q_dtype="f32", k_group=64, window=24),
    "g8-f32kv-window": dict(context=170, num_q_heads=16, num_kv_heads=2, kv_dtype="f32", q_dtype="f32",
                            window=20),
    "g8-fused-steps": dict(batch=2, context=400, num_q_heads=16, num_kv_heads=2, window=32, steps=3),
    "g8-f32q-fused-steps-kgroup64": dict(batch=2, context=350, num_q_heads=16, num_kv_heads=2, q_dtype="f32",
                                         k_group=64, window=32, steps=3),
    "g8-rotated-kgroup128-steps": dict(batch=2, context=500, num_q_heads=16, num_kv_heads=2, rotation=True,
                                       k_group=128, window=0, steps=3),
    "g8-rotated-ragged-kgroup64": dict(batch=3, context=0, var_len=(20, 900), num_q_heads=16, num_kv_heads=2,
                                       rotation=True, k_group=64, window=16),
}


@pytest.mark.parametrize("name", list(ROW_OPERAND))
def test_row_score_operand(name):
    wl = small(BASE, config=900 + list(ROW_OPERAND).index(name), **ROW_OPERAND[name])
    say(f"row operand {name}: {ROW_OPERAND[name]}")
    run = GpuRun(wl, chunk=64)
    for s in range(max(wl.steps, 1)):
        full_check(run, s)


# Codes of 3, 5 and 6 bits, stored as bit planes (4, 2 and 1 bits) and recombined into one MFMA
# operand per pair slot: both append kernels (whole pages and single tokens), every attention
# feature, and decode steps through the append kernel.
NPOW2 = {
    "k3v2": dict(context=300, k_bits=3, v_bits=2),
    "k5v3-window": dict(context=260, k_bits=5, v_bits=3, window=32),
    "k6v2-steps": dict(batch=2, context=600, k_bits=6, v_bits=2, window=0, steps=3),
    "k6v5-g8-vgroup64": dict(context=200, num_q_heads=16, num_kv_heads=2, k_bits=6, v_bits=5, v_group=64),
    "k3v5-kgroup64": dict(context=180, k_bits=3, v_bits=5, k_group=64),
    "k5v6-f32-window": dict(context=160, k_bits=5, v_bits=6, kv_dtype="f32", q_dtype="f32", window=20),
    "k6v3-rotation-window": dict(context=200, k_bits=6, v_bits=3, rotation=True, window=16),
    "k3v3-keys-and-values-rotated": dict(context=250, k_bits=3, v_bits=3, rotation=True, value_rotation=True),
    "k5v1-paged": dict(context=0, var_len=(1, 400), block_size=16, batch=4, k_bits=5, v_bits=1),
    "k1v6-g1": dict(context=150, num_q_heads=8, num_kv_heads=8, k_bits=1, v_bits=6),
    "k6v6-g2-kgroup128": dict(context=140, num_q_heads=16, num_kv_heads=8, k_bits=6, v_bits=6, k_group=128),
    "k5v5-ragged": dict(batch=4, context=0, var_len=(16, 3000), k_bits=5, v_bits=5),
}


@pytest.mark.parametrize("name", list(NPOW2))
def test_non_power_of_two_bits(name):
    wl = small(BASE, config=600 + list(NPOW2).index(name), **NPOW2[name])
    say(f"bit planes {name}: {NPOW2[name]}")
    run = GpuRun(wl, chunk=64)
    for s in range(max(wl.steps, 1)):
        full_check(run, s, out_check_bf16=(s == 0))


WIDTHS = (1, 2, 3, 4, 5, 6, 8)


@pytest.mark.parametrize("kb", WIDTHS)
def test_every_bit_pair(kb):
    """Every (key bits, value bits) instantiation of the split kernel, small: 2 sequences of 70
    tokens (whole pages and a partial one), 4 query heads per kv head."""
    for vb in WIDTHS:
        wl = small(BASE, config=700 + 8 * kb + vb, batch=2, num_q_heads=8, num_kv_heads=2, context=70, k_bits=kb,
                   v_bits=vb)
        say(f"bit pair K{kb}V{vb}")
        run = GpuRun(wl, chunk=64)
        full_check(run, 0, out_check_bf16=False)


# Values rotated before quantization and the output rotated back in the merge: whole pages go
# through the page kernel, the rest through the per-token kernel.
VROT = {
    "values-only": dict(context=300, value_rotation=True),
    "keys-and-values": dict(context=250, rotation=True, value_rotation=True),
    "keys-and-values-g8": dict(context=200, num_q_heads=16, num_kv_heads=2, rotation=True, value_rotation=True),
    "values-g8-vgroup64": dict(context=170, num_q_heads=16, num_kv_heads=2, v_group=64, value_rotation=True),
    "values-f32": dict(context=160, kv_dtype="f32", q_dtype="f32", value_rotation=True),
    "values-paged": dict(context=0, var_len=(1, 300), block_size=16, batch=4, value_rotation=True),
    "values-steps": dict(batch=2, context=700, steps=3, rotation=True, value_rotation=True),
}


@pytest.mark.parametrize("name", list(VROT))
def test_value_rotation(name):
    wl = small(BASE, config=500 + list(VROT).index(name), **VROT[name])
    say(f"value rotation {name}: {VROT[name]}")
    run = GpuRun(wl, chunk=64)
    for s in range(max(wl.steps, 1)):
        full_check(run, s, out_check_bf16=(s == 0))


def test_exact_ties_in_both_append_kernels():
    """Inputs built so that many (x - zero) / scale are exact half-integers (values k/16 with a
    group minimum 0 and maximum 30/16 for 4-bit keys, 3 for 2-bit values): codes must follow
    round-half-to-even bit for bit, both for tokens appended one by one and for whole pages."""
    import oracle as O

    rng = np.random.default_rng(11)
    n = 80
    Kx = rng.integers(0, 31, size=(n, 128)).astype(np.float32) / 16
    Kx[:, 0::32], Kx[:, 1::32] = 0.0, 30.0 / 16
    Vx = rng.integers(0, 49, size=(n, 128)).astype(np.float32) / 16
    Vx[:, 0], Vx[:, 1] = 0.0, 3.0
    prm = K.make_params(128, 1, 1, 4, 32, 2, 128, 0, 0, K.KVQ_BF16, 0)
    cache = K.CacheBuffers(prm, 1, 128)

    def rows(x, t0, t1):
        return torch.from_numpy(W.f32_to_bf16_bits(x[t0:t1]).view(np.int16).reshape(1, t1 - t0, 1, 128)).cuda()

    # 5 tokens one by one (per-token kernel), then 75: 11 single tokens up to the page boundary and
    # 4 whole pages (page kernel)
    for t0, t1 in ((0, 5), (5, 80)):
        before = torch.tensor([t0], dtype=torch.int32, device="cuda")
        K.kvq_quantize_append(prm, cache.struct, before, None, rows(Kx, t0, t1), rows(Vx, t0, t1), t1 - t0)
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    kc = torch.empty((n, 1, 128), dtype=torch.uint8, device="cuda")
    vc = torch.empty((n, 1, 128), dtype=torch.uint8, device="cuda")
    K.kvq_dequantize_debug(prm, cache.struct, lens, 0, 0, n, k_codes=kc, v_codes=vc)
    torch.cuda.synchronize()
    ek, _, _ = O.quantize(Kx.astype(np.float64), 4, 32)
    ev, _, _ = O.quantize(Vx.astype(np.float64), 2, 128)
    ties_k = np.sum(((Kx.astype(np.float64) / 0.125) % 1.0) == 0.5)
    assert ties_k > 1000, ties_k  # the construction does produce exact ties
    assert np.array_equal(kc.cpu().numpy()[:, 0], ek), "key codes differ from the oracle"
    assert np.array_equal(vc.cpu().numpy()[:, 0], ev), "value codes differ from the oracle"


def test_empty_sequences_give_zero():
    wl = small(BASE, context=0, config=300, batch=2)
    say("empty sequences")
    run = GpuRun(wl)
    o = run.decode(0)
    assert np.all(o == 0.0)


def test_constant_groups_scale_zero():
    """Groups with min == max (fp16-exact): scale 0, all codes 0, exact reconstruction."""
    wl = small(BASE, context=40, config=301, batch=1, num_q_heads=4, num_kv_heads=1)
    rng = np.random.default_rng(0)
    Kx = np.full((1, 40, 1, 128), 1.5, dtype=np.float32)
    Vx = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((1, 40, 1, 128)).astype(np.float32)))
    Vx[:, ::3] = -0.75
    q = [W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((1, 4, 128)).astype(np.float32)))]
    say("constant groups")
    run = GpuRun(wl, kv_override=(Kx, Vx), q_override=q)
    full_check(run, 0)


def test_outputs_deterministic_and_split_invariant():
    wl = small(W.WORKLOADS[2], context=2000, config=302)
    say("determinism / split invariance")
    run = GpuRun(wl)
    a = run.decode(0)
    b = run.decode(0)
    assert np.array_equal(a, b)
    old = os.environ.get("KVQ_PAGES_PER_SPLIT")
    try:
        for pps in ("2", "6", "200"):
            os.environ["KVQ_PAGES_PER_SPLIT"] = pps
            c = run.decode(0)
            assert_close(c, a, f"pages/split {pps}")
    finally:
        if old is None:
            os.environ.pop("KVQ_PAGES_PER_SPLIT", None)
        else:
            os.environ["KVQ_PAGES_PER_SPLIT"] = old


@pytest.mark.parametrize("variant", ["window", "value-rotation"])
def test_phase_entry_points_match_attention(variant):
    """kvq_decode_partials + kvq_decode_combine give bit for bit what kvq_decode_attention gives,
    and the workspace rows follow the documented merge rule; with rotated values the merged row
    is in the rotated domain and the normalized Hadamard matrix brings it back."""
    if variant == "window":
        wl = small(W.WORKLOADS[3], batch=2, context=700, steps=1, config=303)
    else:
        wl = small(W.WORKLOADS[3], batch=2, context=700, steps=0, window=0, value_rotation=True, config=305)
    say(f"partials + combine ({variant})")
    run = GpuRun(wl, chunk=256)
    L = run.current_lengths()
    lens = torch.from_numpy(L.astype(np.int32)).cuda()
    q = run._q_dev(0)
    ref = run.attend(lens, int(L.max()), q, "f32")
    wsb = K.kvq_decode_workspace_bytes(run.params, wl.batch, int(L.max()))
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    K.kvq_decode_partials(run.params, run.cache.struct, lens, int(L.max()), q, K.KVQ_BF16, 0.0, ws, wsb)
    K.kvq_decode_combine(run.params, wl.batch, int(L.max()), K.KVQ_BF16, ws, out, K.KVQ_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, ref)
    # merge the rows on the host (fp64) by the documented rule and compare with the kernel's merge
    S = K.kvq_decode_splits(run.params, wl.batch, int(L.max()), K.KVQ_BF16)
    assert S >= 1 and wl.batch * wl.num_q_heads * S * K.KVQ_PART_FLOATS * 4 <= wsb
    blk = ws.view(torch.float32)[: wl.batch * wl.num_q_heads * S * K.KVQ_PART_FLOATS].cpu().numpy()
    blk = blk.astype(np.float64).reshape(wl.batch, wl.num_q_heads, S, K.KVQ_PART_FLOATS)
    # entries [n, S) of a row are not written (n in every written header); empty splits have m = -inf
    n = blk[:, :, :1, 2].astype(np.int64)
    assert np.all(n >= 1) and np.all(n <= S)
    written = np.arange(S)[None, None, :] < n
    assert np.all(blk[..., 2][written] == np.broadcast_to(n, written.shape)[written])
    assert np.all(blk[..., 3][written] == 0.0)
    m, l, acc = np.where(written, blk[..., 0], -np.inf), blk[..., 1], blk[..., 4:]
    empty = np.isneginf(m)
    l = np.where(empty, 0.0, l)
    acc = np.where(empty[..., None], 0.0, acc)
    M = m.max(axis=2, keepdims=True)
    w = np.where(empty, 0.0, np.exp2(np.where(empty, 0.0, m - M)))
    o = (w[..., None] * acc).sum(axis=2) / (w * l).sum(axis=2)[..., None]
    if wl.value_rotation:
        from scipy.linalg import hadamard

        o = o @ (hadamard(128).astype(np.float64) / np.sqrt(128.0))
    assert np.allclose(o, got, rtol=1e-5, atol=2e-6)


def test_graph_replays_match_eager():
    """Decode attention captured in a HIP graph: several replays, with eager work and
    synchronisations between them, each equal bit for bit to the eager result."""
    wl = small(W.WORKLOADS[3], batch=2, context=900, steps=1, config=304)
    say("graph replays")
    run = GpuRun(wl, chunk=256)
    L = run.current_lengths()
    mx = int(L.max())
    lens = torch.from_numpy(L.astype(np.int32)).cuda()
    q = run._q_dev(0)
    eager = run.attend(lens, mx, q, "f32")
    wsb = K.kvq_decode_workspace_bytes(run.params, wl.batch, mx)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.kvq_decode_attention(run.params, run.cache.struct, lens, mx, q, K.KVQ_BF16, out, K.KVQ_F32, 0.0, ws, wsb)
    for r in range(3):
        out.fill_(float("nan"))
        ws.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager), f"replay {r}"
        # eager work between replays
        again = run.attend(lens, mx, q, "f32")
        assert np.array_equal(again, eager)
