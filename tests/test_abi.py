"""Host-only checks of the C ABI: the library loads, exports every symbol the
headers declare, and rejects bad arguments before launching anything (these
calls never reach the GPU, so they run without one)."""
import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K = pytest.importorskip("mixed_precision_kv_kvq_amd")

FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first or no launch happens


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    return sorted(set(re.findall(r"^\s*(?:kvq_status|size_t|const char \*|int32_t|int)\s*\*?\s*(kvq_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = declared("kvq.h")
    assert set(names) == set(K.EXPORTED)
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_generator_exports():
    names = declared("kvq_gen.h")
    assert names == ["kvq_gen_kv", "kvq_gen_q", "kvq_gen_stream_copy", "kvq_gen_stream_read"]
    lib = ctypes.CDLL(os.path.join(ROOT, "workloads", "libkvqgen.so"))
    for n in names:
        assert hasattr(lib, n)


def p(**kw):
    base = dict(head_dim=128, num_q_heads=32, num_kv_heads=8, k_bits=4, k_group=32, v_bits=2, v_group=128, window=0,
                key_rotation=0, kv_dtype=K.KVQ_BF16, block_size=0)
    base.update(kw)
    return K.make_params(**base)


@pytest.mark.parametrize("kb,vb,expect", [(4, 2, 116), (4, 4, 148), (2, 4, 116), (2, 2, 84), (1, 2, 68), (3, 2, 100),
                                          (5, 3, 148), (6, 2, 148), (8, 8, 276)])
def test_record_size_matches_memory_model(kb, vb, expect):
    s = K.kvq_cache_sizes(p(k_bits=kb, v_bits=vb), 2, 100)
    assert s.record_bytes == 16 * expect == 16 * O.bytes_per_token_head(128, kb, 32, vb, 128)
    assert s.pages_bytes == 2 * 7 * 8 * s.record_bytes  # ceil(100/16) pages per sequence
    assert s.window_bytes == 0


def test_sizes_that_do_not_fit_are_rejected():
    out = K.kvq_sizes()
    L = K.lib()
    assert L.kvq_cache_sizes(ctypes.byref(p()), 2 ** 31 - 1, 2 ** 63 - 1, ctypes.byref(out)) == K.KVQ_EINVAL
    assert L.kvq_cache_sizes(ctypes.byref(p(block_size=16)), 1, 2 ** 62, ctypes.byref(out)) == K.KVQ_EINVAL
    assert L.kvq_cache_sizes(ctypes.byref(p()), 1, 2 ** 40, ctypes.byref(out)) == K.KVQ_OK  # 2^36 pages x 8 x 1856 B
    assert out.pages_bytes == (2 ** 36) * 8 * out.record_bytes


def test_window_and_paged_sizes():
    s = K.kvq_cache_sizes(p(window=128), 16, 32832)
    assert s.window_bytes == 16 * 8 * 128 * 128 * 2
    s = K.kvq_cache_sizes(p(block_size=16), 8, 5000)
    assert s.pages_bytes == 5000 * 8 * s.record_bytes


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), K.KVQ_EUNSUPPORTED),
    (dict(k_bits=9), K.KVQ_EUNSUPPORTED),
    (dict(v_bits=7), K.KVQ_EUNSUPPORTED),
    (dict(v_bits=0), K.KVQ_EUNSUPPORTED),
    (dict(k_bits=0), K.KVQ_EUNSUPPORTED),
    (dict(k_group=16), K.KVQ_EUNSUPPORTED),
    (dict(v_group=32), K.KVQ_EUNSUPPORTED),
    (dict(num_q_heads=48, num_kv_heads=8), K.KVQ_EUNSUPPORTED),
    (dict(num_q_heads=30, num_kv_heads=8), K.KVQ_EINVAL),
    (dict(window=-1), K.KVQ_EINVAL),
    (dict(kv_dtype=7), K.KVQ_EINVAL),
    (dict(block_size=32), K.KVQ_EUNSUPPORTED),
    (dict(key_rotation=2), K.KVQ_EINVAL),
    (dict(value_rotation=-1), K.KVQ_EINVAL),
    (dict(value_rotation=1, window=4), K.KVQ_EUNSUPPORTED),
    (dict(num_q_heads=8192, num_kv_heads=1024), K.KVQ_EUNSUPPORTED),  # beyond KVQ_MAX_HEADS
    (dict(window=(1 << 20) + 1), K.KVQ_EUNSUPPORTED),  # beyond KVQ_MAX_WINDOW
])
def test_bad_params_rejected(kw, status):
    out = K.kvq_sizes()
    assert K.lib().kvq_cache_sizes(ctypes.byref(p(**kw)), 1, 16, ctypes.byref(out)) == status


def cache(**kw):
    base = dict(pages=FAKE, k_win=None, v_win=None, block_table=None, batch=2, max_blocks_per_seq=0, capacity=64)
    base.update(kw)
    return K.kvq_cache(**base)


def test_append_validation():
    prm = p()
    L = K.lib()
    assert L.kvq_quantize_append(ctypes.byref(prm), ctypes.byref(cache()), None, None, FAKE, FAKE, 1, None) == K.KVQ_EINVAL
    assert L.kvq_quantize_append(ctypes.byref(prm), ctypes.byref(cache(pages=FAKE + 4)), FAKE, None, FAKE, FAKE, 1,
                                 None) == K.KVQ_EINVAL
    assert L.kvq_quantize_append(ctypes.byref(prm), ctypes.byref(cache()), FAKE, None, FAKE + 2, FAKE, 1,
                                 None) == K.KVQ_EINVAL
    assert L.kvq_quantize_append(ctypes.byref(prm), ctypes.byref(cache()), FAKE, None, FAKE, FAKE, -1,
                                 None) == K.KVQ_EINVAL
    # window without ring buffers, paged without a block table
    assert L.kvq_quantize_append(ctypes.byref(p(window=8)), ctypes.byref(cache()), FAKE, None, FAKE, FAKE, 1,
                                 None) == K.KVQ_EINVAL
    assert L.kvq_quantize_append(ctypes.byref(p(block_size=16)), ctypes.byref(cache()), FAKE, None, FAKE, FAKE, 1,
                                 None) == K.KVQ_EINVAL
    assert L.kvq_quantize_append(ctypes.byref(p(k_bits=9)), ctypes.byref(cache()), FAKE, None, FAKE, FAKE, 1,
                                 None) == K.KVQ_EUNSUPPORTED
    # zero tokens: nothing to do, no launch
    assert L.kvq_quantize_append(ctypes.byref(prm), ctypes.byref(cache()), FAKE, None, None, None, 0, None) == K.KVQ_OK


def test_attention_validation():
    prm = p()
    L = K.lib()
    need = K.kvq_decode_workspace_bytes(prm, 2, 64)
    assert need > 0

    def call(c=None, seq=FAKE, mx=64, q=FAKE, qd=K.KVQ_BF16, out=FAKE, od=K.KVQ_F32, sc=0.0, ws=FAKE, wsb=need,
             prm_=prm):
        return L.kvq_decode_attention(ctypes.byref(prm_), ctypes.byref(c or cache()), seq, mx, q, qd, out, od, sc,
                                      ws, wsb, None)

    assert call(wsb=need - 1) == K.KVQ_ENOSPACE
    assert call(mx=65) == K.KVQ_ENOSPACE  # beyond the capacity of 64 tokens
    assert call(q=None) == K.KVQ_EINVAL
    assert call(out=FAKE + 8) == K.KVQ_EINVAL
    assert call(qd=5) == K.KVQ_EINVAL
    assert call(sc=-1.0) == K.KVQ_EINVAL
    assert call(sc=float("nan")) == K.KVQ_EINVAL
    assert call(seq=None) == K.KVQ_EINVAL
    assert call(prm_=p(head_dim=96)) == K.KVQ_EUNSUPPORTED
    # paged: more pages than the table row holds
    assert call(c=cache(block_table=FAKE, max_blocks_per_seq=3), prm_=p(block_size=16), mx=49,
                wsb=K.kvq_decode_workspace_bytes(p(block_size=16), 2, 49)) == K.KVQ_ENOSPACE
    assert K.kvq_decode_workspace_bytes(p(k_bits=9), 2, 64) == 0
    assert K.kvq_decode_workspace_bytes(p(k_bits=3), 2, 64) > 0
    # value rotation: a flag, and not with a recent window (the window's values are not rotated)
    assert call(prm_=p(value_rotation=2)) == K.KVQ_EINVAL
    assert K.kvq_decode_workspace_bytes(p(value_rotation=1), 2, 64) > 0
    assert K.kvq_decode_workspace_bytes(p(value_rotation=1, window=8), 2, 64) == 0
    assert L.kvq_quantize_append(ctypes.byref(p(value_rotation=1, window=8)), ctypes.byref(cache()), FAKE, None,
                                 FAKE, FAKE, 1, None) == K.KVQ_EUNSUPPORTED


def test_phase_entry_points_validation():
    prm = p()
    L = K.lib()
    need = K.kvq_decode_workspace_bytes(prm, 2, 64)

    def part(mx=64, q=FAKE, qd=K.KVQ_BF16, ws=FAKE, wsb=need, prm_=prm):
        return L.kvq_decode_partials(ctypes.byref(prm_), ctypes.byref(cache()), FAKE, mx, q, qd, 0.0, ws, wsb, None)

    assert part(wsb=need - 1) == K.KVQ_ENOSPACE
    assert part(mx=65) == K.KVQ_ENOSPACE
    assert part(q=None) == K.KVQ_EINVAL
    assert part(ws=FAKE + 4) == K.KVQ_EINVAL
    assert part(qd=7) == K.KVQ_EINVAL
    assert part(prm_=p(v_bits=9)) == K.KVQ_EUNSUPPORTED

    def comb(batch=2, ws=FAKE, out=FAKE, qd=K.KVQ_BF16, od=K.KVQ_F32, prm_=prm):
        return L.kvq_decode_combine(ctypes.byref(prm_), batch, 64, qd, ws, out, od, None)

    assert comb(batch=0) == K.KVQ_EINVAL
    assert comb(ws=None) == K.KVQ_EINVAL
    assert comb(out=FAKE + 8) == K.KVQ_EINVAL
    assert comb(od=9) == K.KVQ_EINVAL
    assert comb(prm_=p(num_q_heads=48)) == K.KVQ_EUNSUPPORTED
    assert K.KVQ_PART_FLOATS == 132


def test_debug_validation():
    prm = p()
    L = K.lib()
    args = [None] * 6
    assert L.kvq_dequantize_debug(ctypes.byref(prm), ctypes.byref(cache()), FAKE, 2, 0, 1, *args, None) == K.KVQ_EINVAL
    assert L.kvq_dequantize_debug(ctypes.byref(prm), ctypes.byref(cache()), FAKE, 0, -1, 1, *args, None) == K.KVQ_EINVAL
    assert L.kvq_dequantize_debug(ctypes.byref(prm), ctypes.byref(cache()), None, 0, 0, 1, *args, None) == K.KVQ_EINVAL
    assert L.kvq_dequantize_debug(ctypes.byref(prm), ctypes.byref(cache()), FAKE, 0, 0, 0, *args, None) == K.KVQ_OK


def test_unfused_baseline_validation():
    prm = p()
    L = K.lib()

    def deq(c=None, seq=FAKE, mx=64, ko=FAKE, vo=FAKE, prm_=prm):
        return L.kvq_dequantize_dense(ctypes.byref(prm_), ctypes.byref(c or cache()), seq, mx, ko, vo, None)

    assert deq(seq=None) == K.KVQ_EINVAL
    assert deq(ko=None) == K.KVQ_EINVAL
    assert deq(vo=FAKE + 2) == K.KVQ_EINVAL
    assert deq(mx=-1) == K.KVQ_EINVAL
    assert deq(mx=1 << 31) == K.KVQ_EINVAL
    assert deq(c=cache(pages=FAKE + 8)) == K.KVQ_EINVAL
    assert deq(prm_=p(k_bits=12)) == K.KVQ_EUNSUPPORTED

    need = K.kvq_dense_workspace_bytes(prm, 2, 600)
    assert need == 2 * 32 * 3 * K.KVQ_PART_FLOATS * 4  # three splits of 256 positions
    assert K.kvq_dense_workspace_bytes(prm, 2, 0) == 2 * 32 * 1 * K.KVQ_PART_FLOATS * 4
    assert K.kvq_dense_workspace_bytes(p(k_bits=9), 2, 600) == 0

    def att(b=2, k=FAKE, v=FAKE, seq=FAKE, mx=600, q=FAKE, qd=K.KVQ_BF16, out=FAKE, od=K.KVQ_F32, sc=0.0, ws=FAKE,
            wsb=need):
        return L.kvq_dense_decode_attention(ctypes.byref(prm), b, k, v, seq, mx, q, qd, out, od, sc, ws, wsb, None)

    assert att(wsb=need - 1) == K.KVQ_ENOSPACE
    assert att(b=0) == K.KVQ_EINVAL
    assert att(k=None) == K.KVQ_EINVAL
    assert att(v=FAKE + 4) == K.KVQ_EINVAL
    assert att(qd=3) == K.KVQ_EINVAL
    assert att(od=9) == K.KVQ_EINVAL
    assert att(sc=float("inf")) == K.KVQ_EINVAL
    assert att(seq=None) == K.KVQ_EINVAL


def test_error_budget_validation():
    L = K.lib()
    need = K.kvq_error_budget_workspace_bytes(p(), 2, 64)

    def call(prm_=None, c=None, seq=FAKE, mx=64, kr=FAKE, vr=FAKE, q=FAKE, qd=K.KVQ_BF16, sc=0.0, hs=FAKE, us=FAKE,
             ws=FAKE, wsb=need):
        return L.kvq_error_budget(ctypes.byref(prm_ or p()), ctypes.byref(c or cache()), seq, mx, kr, vr, q, qd, sc,
                                  hs, us, ws, wsb, None)

    assert call(seq=None) == K.KVQ_EINVAL
    assert call(kr=None) == K.KVQ_EINVAL
    assert call(vr=FAKE + 2) == K.KVQ_EINVAL
    assert call(hs=FAKE + 4) == K.KVQ_EINVAL
    assert call(us=None) == K.KVQ_EINVAL
    assert call(ws=None) == K.KVQ_EINVAL
    assert call(ws=FAKE + 8) == K.KVQ_EINVAL
    assert call(wsb=need - 4) == K.KVQ_ENOSPACE
    assert call(qd=4) == K.KVQ_EINVAL
    assert call(sc=-2.0) == K.KVQ_EINVAL
    assert call(mx=-1) == K.KVQ_EINVAL
    assert call(prm_=p(v_group=32)) == K.KVQ_EUNSUPPORTED


def test_error_budget_workspace_plan():
    # one item per (sequence, kv head, group of up to 4 query heads, range of pages); about two
    # workgroups per CU, at least one page per wave of a range
    # and both fp32 scores of every (sequence, query head, position)
    item = 4 * 2112  # 32 + 4 x 4 x 128 + 4 + 4 floats, padded to whole 128-byte lines
    units = 2 * 8  # batch 2 x 8 kv heads, 4 query heads per kv head: one head group
    for length, ranges in [(0, 1), (1, 1), (128, 1), (129, 2), (16 * 8 * 16, 16), (32768, 32)]:
        rows = -(-length // 16) * 16  # score rows padded to whole 16-position pages
        assert K.kvq_error_budget_workspace_bytes(p(), 2, length) == units * ranges * item + 2 * 32 * rows * 8, length
    # 8 query heads per kv head: two head groups
    assert K.kvq_error_budget_workspace_bytes(p(num_q_heads=64), 2, 32768) == 2 * units * 16 * item + 2 * 64 * 32768 * 8
    # batch 16 x 8 kv heads: 128 items, four ranges each
    assert K.kvq_error_budget_workspace_bytes(p(), 16, 32768) == 128 * 4 * item + 16 * 32 * 32768 * 8
    assert K.kvq_error_budget_workspace_bytes(p(k_bits=9), 2, 600) == 0
    assert K.kvq_error_budget_workspace_bytes(p(), 0, 600) == 0
    assert K.kvq_error_budget_workspace_bytes(p(), 2, -1) == 0


def test_status_strings():
    for s in range(6):
        assert K.kvq_status_str(s)
    assert "device" in K.kvq_status_str(K.KVQ_EDEVICE)
    assert "unknown" in K.kvq_status_str(99)


def test_workspace_grows_with_length_and_split_override(monkeypatch):
    prm = p()
    a = K.kvq_decode_workspace_bytes(prm, 16, 32768)
    b = K.kvq_decode_workspace_bytes(prm, 16, 131072)
    assert 0 < a <= b
    monkeypatch.setenv("KVQ_PAGES_PER_SPLIT", "2")
    c = K.kvq_decode_workspace_bytes(prm, 16, 32768)
    assert c > a


@pytest.mark.parametrize("window,batch,heads", [(0, 1, 8), (128, 16, 8), (40, 3, 2), (16, 64, 8)])
def test_workspace_is_monotone_in_length(window, batch, heads, monkeypatch):
    """A workspace sized for a maximum length serves every shorter length: the size never drops as the
    length grows (the split count of a shorter length can exceed that of a longer one, the size covers both)."""
    prm = p(window=window, num_kv_heads=heads, num_q_heads=4 * heads)
    for env in (None, "6"):
        if env:
            monkeypatch.setenv("KVQ_PAGES_PER_SPLIT", env)
        prev = 0
        for L in list(range(0, 3000)) + list(range(3000, 300000, 997)):
            w = K.kvq_decode_workspace_bytes(prm, batch, L)
            assert w >= prev, (L, w, prev)
            prev = w


def test_package_shares_torchs_hip_runtime():
    """Importing the package first must not map a second HIP runtime beside torch's (a second
    runtime finds no device).  Checked in a fresh interpreter, where the import order is ours."""
    import subprocess
    import sys

    code = ("import mixed_precision_kv_kvq_amd, workloads.device, torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_bound_call_marshals_once_and_raises():
    prm = p()
    call = K.bound_call("kvq_decode_combine", prm, 0, 64, K.KVQ_BF16, FAKE, FAKE, K.KVQ_F32, stream=0)
    with pytest.raises(K.KvqError) as e:
        call()
    assert e.value.status == K.KVQ_EINVAL
    ok = K.bound_call("kvq_quantize_append", prm, cache(), FAKE, None, None, None, 0, stream=0)
    ok()  # zero tokens: validated, nothing launched


def test_noalloc_validation():
    """The allocation-free entry point rejects calls whose partial rows exceed its device array
    (before touching the device), and bad arguments as kvq_decode_attention does."""
    L = K.lib()
    prm = p(num_q_heads=64, key_rotation=1)
    assert K.kvq_decode_workspace_bytes(prm, 512, 131072) > K.KVQ_NOALLOC_SCRATCH_BYTES
    cs = K.kvq_cache(FAKE, None, None, None, 512, 0, 131072)
    st = L.kvq_decode_attention_noalloc(ctypes.byref(prm), ctypes.byref(cs), FAKE, 131072, FAKE, K.KVQ_BF16, FAKE,
                                        K.KVQ_F32, 0.0, None)
    assert st == K.KVQ_ENOSPACE
    assert L.kvq_decode_attention_noalloc(ctypes.byref(p(k_bits=9)), ctypes.byref(cs), FAKE, 16, FAKE, K.KVQ_BF16,
                                          FAKE, K.KVQ_F32, 0.0, None) == K.KVQ_EUNSUPPORTED
    assert L.kvq_decode_attention_noalloc(ctypes.byref(prm), None, FAKE, 16, FAKE, K.KVQ_BF16, FAKE, K.KVQ_F32, 0.0,
                                          None) == K.KVQ_EINVAL


def test_device_status_validation():
    """kvq_device_status needs an error word and an output; a misaligned error word is rejected by
    every entry point that takes the cache (host checks only: nothing is launched)."""
    L = K.lib()
    flags = ctypes.c_uint32(0)
    cs = K.kvq_cache(FAKE, None, None, None, 1, 0, 16)
    assert L.kvq_device_status(ctypes.byref(cs), ctypes.byref(flags), None) == K.KVQ_EINVAL
    assert L.kvq_device_status(None, ctypes.byref(flags), None) == K.KVQ_EINVAL
    cs.error_flags = FAKE
    assert L.kvq_device_status(ctypes.byref(cs), None, None) == K.KVQ_EINVAL
    cs.error_flags = FAKE + 2  # not 4-byte aligned
    assert L.kvq_quantize_append(ctypes.byref(p()), ctypes.byref(cs), FAKE, None, FAKE, FAKE, 1, None) == K.KVQ_EINVAL
    assert L.kvq_decode_attention(ctypes.byref(p()), ctypes.byref(cs), FAKE, 16, FAKE, K.KVQ_BF16, FAKE, K.KVQ_F32,
                                  0.0, FAKE, 1 << 30, None) == K.KVQ_EINVAL
