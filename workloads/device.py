"""Device-side generation of the seeded inputs (wrapper of workloads/libkvqgen.so).

Produces, on the GPU, exactly the values that workloads.Workload produces on
the host (a test checks bit equality on samples).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import TENSOR_K, TENSOR_Q, TENSOR_V, Workload, normal_table, stream_key

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvqgen.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build with `python mixed_precision_kv_kvq_amd/build.py`")
        lib = ctypes.CDLL(path)
        lib.kvq_gen_kv.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
        lib.kvq_gen_kv.restype = ctypes.c_int
        lib.kvq_gen_q.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.kvq_gen_q.restype = ctypes.c_int
        lib.kvq_gen_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p]
        lib.kvq_gen_stream_read.restype = ctypes.c_int
        lib.kvq_gen_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.kvq_gen_stream_copy.restype = ctypes.c_int
        _LIB = lib
    return _LIB


class DeviceGenerator:
    """Holds the device copies of the quantile table and channel std of one workload."""

    def __init__(self, wl: Workload, device="cuda"):
        self.wl = wl
        self.device = device
        self.table = torch.from_numpy(normal_table()).to(device)
        self.sig_k = torch.from_numpy(wl.key_sigma()).to(device).contiguous()
        self.sig_v = torch.from_numpy(wl.value_sigma()).to(device).contiguous()

    def kv(self, tensor: int, t0: int, n: int, out: torch.Tensor | None = None) -> torch.Tensor:
        """[B][n][Hkv][d] rows of K or V for tokens [t0, t0+n) (bf16 stored as int16, or fp32)."""
        wl = self.wl
        f32 = wl.kv_dtype == "f32"
        shape = (wl.batch, n, wl.num_kv_heads, wl.head_dim)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32 if f32 else torch.int16, device=self.device)
        sig = self.sig_k if tensor == TENSOR_K else self.sig_v
        rc = _lib().kvq_gen_kv(out.data_ptr(), int(f32), stream_key(wl.seed, wl.config, tensor), sig.data_ptr(),
                               self.table.data_ptr(), wl.batch, n, wl.num_kv_heads, t0, wl.head_dim,
                               torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"kvq_gen_kv failed: hip error {rc}")
        return out

    def q(self, step: int, out: torch.Tensor | None = None) -> torch.Tensor:
        wl = self.wl
        f32 = wl.q_dtype == "f32"
        if out is None:
            out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim), dtype=torch.float32 if f32 else torch.int16,
                              device=self.device)
        rc = _lib().kvq_gen_q(out.data_ptr(), int(f32), stream_key(wl.seed, wl.config, TENSOR_Q),
                              self.table.data_ptr(), wl.batch, wl.num_q_heads, wl.head_dim, step,
                              torch.cuda.current_stream().cuda_stream)
        if rc:
            raise RuntimeError(f"kvq_gen_q failed: hip error {rc}")
        return out


def stream_read_call(buf: torch.Tensor, nbytes: int, sink: torch.Tensor, blocks: int, nontemporal: bool, stream):
    """A zero-argument callable launching the read-only streaming kernel over nbytes of buf."""
    fn = _lib().kvq_gen_stream_read
    args = (buf.data_ptr(), int(nbytes), sink.data_ptr(), int(blocks), int(nontemporal), stream.cuda_stream)

    def call():
        rc = fn(*args)
        if rc:
            raise RuntimeError(f"kvq_gen_stream_read failed: hip error {rc}")

    return call


def stream_copy(dst: torch.Tensor, src: torch.Tensor, nbytes: int, stream):
    """Launch the plain copy kernel over nbytes (a kernel of known traffic, for counter calibration)."""
    assert dst.numel() * dst.element_size() >= nbytes and src.numel() * src.element_size() >= nbytes
    rc = _lib().kvq_gen_stream_copy(dst.data_ptr(), src.data_ptr(), int(nbytes), stream.cuda_stream)
    if rc:
        raise RuntimeError(f"kvq_gen_stream_copy failed: hip error {rc}")
