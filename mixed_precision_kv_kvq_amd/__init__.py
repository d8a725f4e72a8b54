"""Python binding of libkvq.so: decode attention over a group-wise quantized KV cache.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkvq.so.  Functions keep the C names of include/kvq.h and accept
torch tensors (device pointers are taken with ``data_ptr()``) or raw integer
addresses.  Streams default to torch's current stream.  Importing this package
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint8, c_uint16, c_void_p

# torch first: libkvq.so resolves its HIP runtime by soname (libamdhip64.so.7), which then binds
# to the copy torch has already loaded.  Loaded before torch, the library would pull in a second
# HIP runtime next to torch's own, and that second runtime finds no device.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KVQ_LIB") or os.path.join(_HERE, "libkvq.so")

KVQ_OK, KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_ENOSPACE, KVQ_EHIP, KVQ_EDEVICE = range(6)
KVQ_DEV_TABLE_ENTRY, KVQ_DEV_CAPACITY, KVQ_DEV_LENGTH, KVQ_DEV_COUNT = 1, 2, 4, 8
KVQ_F32, KVQ_BF16 = 0, 1
KVQ_ROT_NONE, KVQ_ROT_WHT = 0, 1
KVQ_PART_FLOATS = 132  # floats per (row, split) of the decode workspace: m, l, 0, 0, acc[128]

EXPORTED = [
    "kvq_cache_sizes",
    "kvq_quantize_append",
    "kvq_decode_workspace_bytes",
    "kvq_decode_attention",
    "kvq_decode_splits",
    "kvq_decode_partials",
    "kvq_decode_combine",
    "kvq_decode_attention_noalloc",
    "kvq_decode_step",
    "kvq_decode_step_partials",
    "kvq_dequantize_debug",
    "kvq_dequantize_dense",
    "kvq_dense_workspace_bytes",
    "kvq_dense_decode_attention",
    "kvq_error_budget_workspace_bytes",
    "kvq_error_budget",
    "kvq_device_status",
    "kvq_status_str",
]


class kvq_params(ctypes.Structure):
    _fields_ = [
        ("head_dim", c_int32),
        ("num_q_heads", c_int32),
        ("num_kv_heads", c_int32),
        ("k_bits", c_int32),
        ("k_group", c_int32),
        ("v_bits", c_int32),
        ("v_group", c_int32),
        ("window", c_int32),
        ("key_rotation", c_int32),
        ("kv_dtype", c_int32),
        ("block_size", c_int32),
        ("value_rotation", c_int32),
    ]


class kvq_cache(ctypes.Structure):
    _fields_ = [
        ("pages", c_void_p),
        ("k_win", c_void_p),
        ("v_win", c_void_p),
        ("block_table", c_void_p),
        ("batch", c_int32),
        ("max_blocks_per_seq", c_int32),
        ("capacity", c_int64),
        ("error_flags", c_void_p),
    ]


class kvq_sizes(ctypes.Structure):
    _fields_ = [("record_bytes", c_size_t), ("pages_bytes", c_size_t), ("window_bytes", c_size_t)]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kvq_status_str(status)} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python mixed_precision_kv_kvq_amd/build.py` "
            "(or __graft_entry__.build()); there is no fallback path."
        )
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    lib.kvq_cache_sizes.argtypes = [P(kvq_params), c_int32, c_int64, P(kvq_sizes)]
    lib.kvq_cache_sizes.restype = c_int32
    lib.kvq_quantize_append.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                        c_void_p]
    lib.kvq_quantize_append.restype = c_int32
    lib.kvq_decode_workspace_bytes.argtypes = [P(kvq_params), c_int32, c_int64]
    lib.kvq_decode_workspace_bytes.restype = c_size_t
    lib.kvq_decode_attention.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int64, c_void_p, c_int32, c_void_p,
                                         c_int32, c_float, c_void_p, c_size_t, c_void_p]
    lib.kvq_decode_attention.restype = c_int32
    lib.kvq_decode_splits.argtypes = [P(kvq_params), c_int32, c_int64, c_int32]
    lib.kvq_decode_splits.restype = c_int32
    lib.kvq_decode_partials.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int64, c_void_p, c_int32, c_float,
                                        c_void_p, c_size_t, c_void_p]
    lib.kvq_decode_partials.restype = c_int32
    lib.kvq_decode_combine.argtypes = [P(kvq_params), c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int32,
                                       c_void_p]
    lib.kvq_decode_combine.restype = c_int32
    lib.kvq_decode_attention_noalloc.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int64, c_void_p, c_int32,
                                                 c_void_p, c_int32, c_float, c_void_p]
    lib.kvq_decode_attention_noalloc.restype = c_int32
    lib.kvq_decode_step.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_void_p, c_void_p, c_int64, c_void_p,
                                    c_int32, c_void_p, c_int32, c_float, c_void_p, c_size_t, c_void_p]
    lib.kvq_decode_step.restype = c_int32
    lib.kvq_decode_step_partials.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_void_p, c_void_p, c_int64,
                                             c_void_p, c_int32, c_float, c_void_p, c_size_t, c_void_p]
    lib.kvq_decode_step_partials.restype = c_int32
    lib.kvq_dequantize_debug.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int32, c_int64, c_int64, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.kvq_dequantize_debug.restype = c_int32
    lib.kvq_dequantize_dense.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int64, c_void_p, c_void_p,
                                         c_void_p]
    lib.kvq_dequantize_dense.restype = c_int32
    lib.kvq_dense_workspace_bytes.argtypes = [P(kvq_params), c_int32, c_int64]
    lib.kvq_dense_workspace_bytes.restype = c_size_t
    lib.kvq_dense_decode_attention.argtypes = [P(kvq_params), c_int32, c_void_p, c_void_p, c_void_p, c_int64,
                                               c_void_p, c_int32, c_void_p, c_int32, c_float, c_void_p, c_size_t,
                                               c_void_p]
    lib.kvq_dense_decode_attention.restype = c_int32
    lib.kvq_error_budget_workspace_bytes.argtypes = [P(kvq_params), c_int32, c_int64]
    lib.kvq_error_budget_workspace_bytes.restype = c_size_t
    lib.kvq_error_budget.argtypes = [P(kvq_params), P(kvq_cache), c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
                                     c_int32, c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.kvq_error_budget.restype = c_int32
    lib.kvq_device_status.argtypes = [P(kvq_cache), P(ctypes.c_uint32), c_void_p]
    lib.kvq_device_status.restype = c_int32
    lib.kvq_status_str.argtypes = [c_int32]
    lib.kvq_status_str.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib():
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st, where):
    if st != KVQ_OK:
        raise KvqError(st, where)


def bound_call(name: str, *args, stream=None):
    """A zero-argument callable that calls C entry point `name` with these arguments, marshalled
    once here (structs by reference, tensors as device pointers, the stream as a handle), and
    raises KvqError on a non-OK status.  For tight launch loops where per-call marshalling shows."""
    fn = getattr(_lib, name)
    conv = [ctypes.byref(a) if isinstance(a, ctypes.Structure) else _ptr(a) if hasattr(a, "data_ptr") else a
            for a in args]
    if name in ("kvq_quantize_append", "kvq_decode_attention", "kvq_decode_partials", "kvq_decode_combine",
                "kvq_decode_attention_noalloc", "kvq_decode_step", "kvq_decode_step_partials",
                "kvq_dequantize_dense", "kvq_dense_decode_attention", "kvq_error_budget"):
        conv.append(_stream(stream))
    conv = tuple(conv)

    def call():
        st = fn(*conv)
        if st != KVQ_OK:
            raise KvqError(st, name)

    return call


def kvq_device_status(cache, stream=None):
    """(status, flags): waits for the stream, reads the cache's device error word."""
    flags = ctypes.c_uint32(0)
    st = _lib.kvq_device_status(ctypes.byref(cache), ctypes.byref(flags), _stream(stream))
    return st, int(flags.value)


def kvq_status_str(status: int) -> str:
    return _lib.kvq_status_str(int(status)).decode()


def kvq_cache_sizes(params: kvq_params, batch: int, capacity: int) -> kvq_sizes:
    out = kvq_sizes()
    _check(_lib.kvq_cache_sizes(ctypes.byref(params), batch, capacity, ctypes.byref(out)), "kvq_cache_sizes")
    return out


def kvq_quantize_append(params, cache, seq_lens_before, n_new_per_seq, k_new, v_new, n_new, stream=None, check=True):
    st = _lib.kvq_quantize_append(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens_before),
                                  _ptr(n_new_per_seq), _ptr(k_new), _ptr(v_new), int(n_new), _stream(stream))
    if check:
        _check(st, "kvq_quantize_append")
    return st


def kvq_decode_workspace_bytes(params, batch: int, max_seq_len: int) -> int:
    return int(_lib.kvq_decode_workspace_bytes(ctypes.byref(params), batch, max_seq_len))


def kvq_decode_attention(params, cache, seq_lens, max_seq_len, q, q_dtype, out, out_dtype, softmax_scale, workspace,
                         workspace_bytes, stream=None, check=True):
    st = _lib.kvq_decode_attention(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens), int(max_seq_len),
                                   _ptr(q), int(q_dtype), _ptr(out), int(out_dtype), float(softmax_scale),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "kvq_decode_attention")
    return st


def kvq_decode_splits(params, batch: int, max_seq_len: int, q_dtype: int) -> int:
    return int(_lib.kvq_decode_splits(ctypes.byref(params), int(batch), int(max_seq_len), int(q_dtype)))


def kvq_decode_partials(params, cache, seq_lens, max_seq_len, q, q_dtype, softmax_scale, workspace, workspace_bytes,
                        stream=None, check=True):
    st = _lib.kvq_decode_partials(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens), int(max_seq_len),
                                  _ptr(q), int(q_dtype), float(softmax_scale), _ptr(workspace),
                                  int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "kvq_decode_partials")
    return st


def kvq_decode_combine(params, batch, max_seq_len, q_dtype, workspace, out, out_dtype, stream=None, check=True):
    st = _lib.kvq_decode_combine(ctypes.byref(params), int(batch), int(max_seq_len), int(q_dtype), _ptr(workspace),
                                 _ptr(out), int(out_dtype), _stream(stream))
    if check:
        _check(st, "kvq_decode_combine")
    return st


def kvq_decode_step(params, cache, seq_lens_before, k_new, v_new, max_seq_len, q, q_dtype, out, out_dtype,
                    softmax_scale, workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvq_decode_step(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens_before), _ptr(k_new),
                              _ptr(v_new), int(max_seq_len), _ptr(q), int(q_dtype), _ptr(out), int(out_dtype),
                              float(softmax_scale), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "kvq_decode_step")
    return st


def kvq_decode_step_partials(params, cache, seq_lens_before, k_new, v_new, max_seq_len, q, q_dtype, softmax_scale,
                             workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvq_decode_step_partials(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens_before), _ptr(k_new),
                                       _ptr(v_new), int(max_seq_len), _ptr(q), int(q_dtype), float(softmax_scale),
                                       _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "kvq_decode_step_partials")
    return st


KVQ_NOALLOC_SCRATCH_BYTES = 16 << 20  # device array behind kvq_decode_attention_noalloc


def kvq_decode_attention_noalloc(params, cache, seq_lens, max_seq_len, q, q_dtype, out, out_dtype, softmax_scale,
                                 stream=None, check=True):
    st = _lib.kvq_decode_attention_noalloc(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens),
                                           int(max_seq_len), _ptr(q), int(q_dtype), _ptr(out), int(out_dtype),
                                           float(softmax_scale), _stream(stream))
    if check:
        _check(st, "kvq_decode_attention_noalloc")
    return st


def kvq_dequantize_debug(params, cache, seq_lens, seq, t0, n, k_codes=None, v_codes=None, k_meta=None, v_meta=None,
                         k_hat=None, v_hat=None, stream=None, check=True):
    st = _lib.kvq_dequantize_debug(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens), int(seq), int(t0),
                                   int(n), _ptr(k_codes), _ptr(v_codes), _ptr(k_meta), _ptr(v_meta), _ptr(k_hat),
                                   _ptr(v_hat), _stream(stream))
    if check:
        _check(st, "kvq_dequantize_debug")
    return st


def kvq_dequantize_dense(params, cache, seq_lens, max_seq_len, k_out, v_out, stream=None, check=True):
    st = _lib.kvq_dequantize_dense(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens), int(max_seq_len),
                                   _ptr(k_out), _ptr(v_out), _stream(stream))
    if check:
        _check(st, "kvq_dequantize_dense")
    return st


def kvq_dense_workspace_bytes(params, batch: int, max_seq_len: int) -> int:
    return int(_lib.kvq_dense_workspace_bytes(ctypes.byref(params), int(batch), int(max_seq_len)))


def kvq_dense_decode_attention(params, batch, k, v, seq_lens, max_seq_len, q, q_dtype, out, out_dtype, softmax_scale,
                               workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvq_dense_decode_attention(ctypes.byref(params), int(batch), _ptr(k), _ptr(v), _ptr(seq_lens),
                                         int(max_seq_len), _ptr(q), int(q_dtype), _ptr(out), int(out_dtype),
                                         float(softmax_scale), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "kvq_dense_decode_attention")
    return st


KVQ_EB_HEAD = 8  # per (sequence, query head) error statistics
KVQ_EB_UNIT = 8  # per (sequence, kv head) reconstruction statistics


def kvq_error_budget_workspace_bytes(params, batch: int, max_seq_len: int) -> int:
    return int(_lib.kvq_error_budget_workspace_bytes(ctypes.byref(params), batch, max_seq_len))


def kvq_error_budget(params, cache, seq_lens, max_seq_len, k_ref, v_ref, q, q_dtype, softmax_scale, head_stats,
                     unit_stats, workspace, workspace_bytes, stream=None, check=True):
    st = _lib.kvq_error_budget(ctypes.byref(params), ctypes.byref(cache), _ptr(seq_lens), int(max_seq_len),
                               _ptr(k_ref), _ptr(v_ref), _ptr(q), int(q_dtype), float(softmax_scale),
                               _ptr(head_stats), _ptr(unit_stats), _ptr(workspace), int(workspace_bytes),
                               _stream(stream))
    if check:
        _check(st, "kvq_error_budget")
    return st


# --------------------------------------------------------------------------
# Plumbing: device buffers for one cache, allocated with torch.
# --------------------------------------------------------------------------
def make_params(head_dim=128, num_q_heads=32, num_kv_heads=8, k_bits=4, k_group=32, v_bits=2, v_group=128, window=0,
                key_rotation=0, kv_dtype=KVQ_BF16, block_size=0, value_rotation=0) -> kvq_params:
    return kvq_params(head_dim, num_q_heads, num_kv_heads, k_bits, k_group, v_bits, v_group, window, key_rotation,
                      kv_dtype, block_size, value_rotation)


class CacheBuffers:
    """Torch-owned device buffers of one cache and the matching kvq_cache struct."""

    def __init__(self, params: kvq_params, batch: int, capacity: int, block_table=None, device="cuda"):
        import torch

        sizes = kvq_cache_sizes(params, batch, capacity)
        self.params = params
        self.sizes = sizes
        self.pages = torch.empty(max(int(sizes.pages_bytes), 16), dtype=torch.uint8, device=device)
        if params.window > 0:
            self.k_win = torch.empty(int(sizes.window_bytes), dtype=torch.uint8, device=device)
            self.v_win = torch.empty(int(sizes.window_bytes), dtype=torch.uint8, device=device)
        else:
            self.k_win = self.v_win = None
        self.block_table = block_table
        mbps = int(block_table.shape[1]) if block_table is not None else 0
        # device error word (KVQ_DEV_* flags), zero until a kernel meets a bad device-side input
        self.error_word = torch.zeros(4, dtype=torch.int32, device=device)
        self.struct = kvq_cache(_ptr(self.pages), _ptr(self.k_win), _ptr(self.v_win), _ptr(block_table), batch, mbps,
                                capacity, _ptr(self.error_word))

    def device_errors(self) -> int:
        """KVQ_DEV_* flags the kernels have raised on this cache so far (synchronizes)."""
        return kvq_device_status(self.struct)[1]

    def clear_device_errors(self) -> None:
        self.error_word.zero_()
