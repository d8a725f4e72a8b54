"""kvq_decode_attention_noalloc (partial rows in the library's own device array) against
kvq_decode_attention (caller workspace): same kernels and split plan, so the outputs must be
identical bit for bit.  Two calls in a row, the second on a smaller input, so that the second
call reuses the array the first one filled; the first case is also checked against the oracle."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import mixed_precision_kv_kvq_amd as K  # noqa: E402
import workloads as W  # noqa: E402
from kvq_harness import GpuRun, assert_close, oracle_heads, oracle_unit, small  # noqa: E402


def say(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def _both(run: GpuRun, step: int, out_dtype: int):
    """Output of the workspace entry point and of the allocation-free one on the same state."""
    wl = run.wl
    L = run.current_lengths()
    seq_lens = torch.from_numpy(L.astype(np.int32)).cuda()
    q = run._q_dev(step)
    qd = K.KVQ_F32 if wl.q_dtype == "f32" else K.KVQ_BF16
    odt = torch.float32 if out_dtype == K.KVQ_F32 else torch.int16
    ws_bytes = K.kvq_decode_workspace_bytes(run.params, wl.batch, int(L.max()))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    ref = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=odt, device="cuda")
    got = torch.full_like(ref, 7)
    K.kvq_decode_attention(run.params, run.cache.struct, seq_lens, int(L.max()), q, qd, ref, out_dtype, 0.0, ws,
                           ws_bytes)
    K.kvq_decode_attention_noalloc(run.params, run.cache.struct, seq_lens, int(L.max()), q, qd, got, out_dtype, 0.0)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    # first call: 32k-token batch of 4 with a recent window (several splits per unit)
    big = small(W.WORKLOADS[3], batch=4, context=3000, steps=1)
    say(f"noalloc call 1: {big.name} B=4 L=3001")
    run = GpuRun(big, device_gen=True)
    run.decode(0)  # one decode step (append + attention through the workspace entry point)
    ref, got = _both(run, 0, K.KVQ_F32)
    assert np.array_equal(ref, got), "first call differs from kvq_decode_attention"
    cache, _, _ = oracle_unit(run, 1, 3)
    g = big.group_q
    assert_close(got[1, 3 * g:4 * g], oracle_heads(run, cache, 1, 3, 0), "noalloc vs oracle")
    del run
    torch.cuda.synchronize()

    # second call: smaller batch and length, bf16 output, reusing the array the first call filled
    little = small(W.WORKLOADS[2], batch=2, context=700)
    say(f"noalloc call 2: {little.name} B=2 L=700 bf16 output")
    run2 = GpuRun(little, device_gen=False)
    ref2, got2 = _both(run2, 0, K.KVQ_BF16)
    assert np.array_equal(ref2, got2), "second (smaller) call differs from kvq_decode_attention"


def test_noalloc_rejects_beyond_the_array():
    # batch 512 x 64 query heads at 131072 tokens needs far more than 16 MiB of partial rows
    prm = K.make_params(128, 64, 8, 4, 32, 2, 128, 0, 1, K.KVQ_BF16, 0)
    need = K.kvq_decode_workspace_bytes(prm, 512, 131072)
    assert need > K.KVQ_NOALLOC_SCRATCH_BYTES
    cs = K.kvq_cache(0x100000, None, None, None, 512, 0, 131072)
    st = K.kvq_decode_attention_noalloc(prm, cs, 0x100000, 131072, 0x100000, K.KVQ_BF16, 0x100000, K.KVQ_F32, 0.0,
                                        check=False)
    assert st == K.KVQ_ENOSPACE
