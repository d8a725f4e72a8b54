"""Seeded synthetic inputs for the quantized-KV decode-attention workloads.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds no arithmetic of the method (no quantization, no
rotation, no attention): it only produces the bytes that both sides receive.

Generator (counter based, so any element can be produced on its own):

* Each (seed, config, tensor) stream has a 64-bit key ``stream_key``.
* Element ``idx`` of that stream takes the 64-bit output of SplitMix64
  (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014) at state ``key + (idx + 1) * 0x9E3779B97F4A7C15``.
* The top 16 bits select an entry of a 65536-entry table of standard-normal
  quantiles, ``ndtri((i + 0.5) / 65536)`` rounded to fp32.
* The value is ``fp32(sigma[channel] * z)``, then rounded to bf16 with
  round-to-nearest-even for bf16 tensors.

The same generator is implemented in HIP (``workloads/gen.hip``) so that the
multi-gigabyte caches of the long-context workloads can be produced on the
device; a test checks that both implementations agree bit for bit.

Element index of a K/V element (b, kvh, t, c): ``((b*Hkv + kvh) * T_STRIDE + t) * d + c``
with ``T_STRIDE = 2**24`` so that indices do not depend on the context length.
Element index of a query element (step, b, h, c): ``((step*B + b) * Hq + h) * d + c``.
"""
from __future__ import annotations

import dataclasses
import functools
from typing import Optional

import numpy as np

GOLDEN_GAMMA = 0x9E3779B97F4A7C15
M64 = (1 << 64) - 1
T_STRIDE = 1 << 24

TENSOR_K, TENSOR_V, TENSOR_Q = 1, 2, 3


# --------------------------------------------------------------------------
# SplitMix64
# --------------------------------------------------------------------------
def _mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(0xBF58476D1CE4E5B9)
        z ^= z >> np.uint64(27)
        z *= np.uint64(0x94D049BB133111EB)
        z ^= z >> np.uint64(31)
    return z


def stream_key(seed: int, config: int, tensor: int) -> int:
    """64-bit key of one (seed, config, tensor) stream."""
    s = ((seed & 0xFFFFFFFF) << 32) | ((config & 0xFFFF) << 16) | (tensor & 0xFFFF)
    return _mix64_int(s + GOLDEN_GAMMA)


def splitmix_u64(key: int, idx: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs at element indices ``idx`` of the stream with ``key``."""
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + (idx + np.uint64(1)) * np.uint64(GOLDEN_GAMMA)
    return _mix64_np(state)


@functools.lru_cache(maxsize=1)
def normal_table() -> np.ndarray:
    """65536 standard-normal quantiles at cell midpoints, as fp32."""
    from scipy.special import ndtri

    p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(p).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(key: int, idx: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """fp32 values ``sigma * z`` (sigma broadcast against idx)."""
    u = splitmix_u64(key, idx)
    z = normal_table()[(u >> np.uint64(48)).astype(np.int64)]
    return (np.asarray(sigma, dtype=np.float32) * z).astype(np.float32)


# --------------------------------------------------------------------------
# Workload definitions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and structure of one synthetic workload (one attention layer)."""

    config: int
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context: int  # tokens in the cache before decoding (fixed-length workloads)
    window: int  # most recent tokens kept unquantized
    steps: int  # decode steps that each append one token, then attend; 0 = one attention over the context
    kv_dtype: str  # "f32" or "bf16"
    q_dtype: str
    k_bits: int
    k_group: int
    v_bits: int
    v_group: int
    rotation: bool  # key-only 128-point normalized Walsh-Hadamard rotation
    block_size: int  # 0 = contiguous per-sequence storage, else tokens per page
    key_outliers: int  # outlier channels per kv head
    key_outlier_mult: float
    key_lognormal_sigma: float  # 0 = unit channel std
    var_len: Optional[tuple] = None  # (lo, hi) inclusive uniform context lengths
    seed: int = 0
    value_rotation: bool = False  # the same rotation applied to the values (no recent window)

    @property
    def group_q(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def with_bits(self, k_bits: int, v_bits: int) -> "Workload":
        return dataclasses.replace(self, k_bits=k_bits, v_bits=v_bits)

    def context_lengths(self) -> np.ndarray:
        """Per-sequence context length before the first decode step."""
        if self.var_len is None:
            return np.full(self.batch, self.context, dtype=np.int64)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, self.config, 101])))
        lo, hi = self.var_len
        return rng.integers(lo, hi + 1, size=self.batch).astype(np.int64)

    def key_sigma(self) -> np.ndarray:
        """Per (kv head, channel) key standard deviation, fp32 [Hkv][d]."""
        d, H = self.head_dim, self.num_kv_heads
        sig = np.ones((H, d), dtype=np.float64)
        for h in range(H):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, self.config, TENSOR_K, h])))
            if self.key_lognormal_sigma > 0:
                sig[h] = rng.lognormal(0.0, self.key_lognormal_sigma, size=d)
            if self.key_outliers:
                ch = rng.choice(d, size=self.key_outliers, replace=False)
                sig[h, ch] *= self.key_outlier_mult
        return sig.astype(np.float32)

    def value_sigma(self) -> np.ndarray:
        return np.ones((self.num_kv_heads, self.head_dim), dtype=np.float32)

    # ---- element generation (host) --------------------------------------
    def kv_f32(self, tensor: int, b: int, kvh: int, t0: int, n: int) -> np.ndarray:
        """fp32 values of K or V for one (sequence, kv head), tokens [t0, t0+n): [n][d].

        For bf16 workloads the values are already rounded to bf16 (returned as fp32).
        """
        d = self.head_dim
        sig = (self.key_sigma() if tensor == TENSOR_K else self.value_sigma())[kvh]
        t = np.arange(t0, t0 + n, dtype=np.uint64)[:, None]
        c = np.arange(d, dtype=np.uint64)[None, :]
        idx = ((np.uint64(b * self.num_kv_heads + kvh) * np.uint64(T_STRIDE) + t) * np.uint64(d)) + c
        x = draw(stream_key(self.seed, self.config, tensor), idx, sig[None, :])
        if self.kv_dtype == "bf16":
            x = bf16_bits_to_f32(f32_to_bf16_bits(x))
        return x

    def kv_batch_f32(self, tensor: int, t0: int, n: int) -> np.ndarray:
        """K or V for all sequences and kv heads, tokens [t0, t0+n): [B][n][Hkv][d] fp32."""
        out = np.empty((self.batch, n, self.num_kv_heads, self.head_dim), dtype=np.float32)
        for b in range(self.batch):
            for h in range(self.num_kv_heads):
                out[b, :, h, :] = self.kv_f32(tensor, b, h, t0, n)
        return out

    def q_f32(self, step: int) -> np.ndarray:
        """Queries of one decode step: [B][Hq][d] fp32 (bf16-rounded for bf16 workloads)."""
        B, Hq, d = self.batch, self.num_q_heads, self.head_dim
        idx = (np.uint64(step * B) * np.uint64(Hq) * np.uint64(d)) + np.arange(B * Hq * d, dtype=np.uint64)
        x = draw(stream_key(self.seed, self.config, TENSOR_Q), idx, np.float32(1.0)).reshape(B, Hq, d)
        if self.q_dtype == "bf16":
            x = bf16_bits_to_f32(f32_to_bf16_bits(x))
        return x

    def block_table(self, max_blocks: Optional[int] = None):
        """Seeded random page assignment for paged workloads.

        Returns (table [B][max_blocks] int32 with -1 padding, pool_pages).
        Capacity covers the context plus the decode steps.
        """
        L = self.context_lengths() + self.steps
        nb = -(-L // self.block_size)
        pool = int(nb.sum())
        if max_blocks is None:
            max_blocks = int(nb.max())
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([self.seed, self.config, 202])))
        perm = rng.permutation(pool).astype(np.int32)
        table = np.full((self.batch, max_blocks), -1, dtype=np.int32)
        o = 0
        for b in range(self.batch):
            table[b, : nb[b]] = perm[o : o + nb[b]]
            o += nb[b]
        return table, pool


def _w(**kw) -> Workload:
    base = dict(head_dim=128, steps=0, kv_dtype="bf16", q_dtype="bf16", k_bits=4, k_group=32, v_bits=2,
                v_group=128, rotation=False, block_size=0, key_outliers=3, key_outlier_mult=10.0,
                key_lognormal_sigma=0.5, window=0)
    base.update(kw)
    return Workload(**base)


# The five workloads: shapes, bit widths, structure (see the design doc for the recipe).
WORKLOADS = {
    1: _w(config=1, name="1head-d128-L512-f32", batch=1, num_q_heads=1, num_kv_heads=1, context=512,
          kv_dtype="f32", q_dtype="f32", key_outliers=4, key_outlier_mult=8.0, key_lognormal_sigma=0.0),
    2: _w(config=2, name="b1-gqa32x8-L4096", batch=1, num_q_heads=32, num_kv_heads=8, context=4096),
    3: _w(config=3, name="b16-gqa32x8-L32768-win128-64steps", batch=16, num_q_heads=32, num_kv_heads=8,
          context=32768, window=128, steps=64),
    4: _w(config=4, name="b8-gqa32x8-L1k-16k-paged16", batch=8, num_q_heads=32, num_kv_heads=8, context=0,
          var_len=(1024, 16384), block_size=16),
    5: _w(config=5, name="b64-gqa64x8-L131072-wht", batch=64, num_q_heads=64, num_kv_heads=8, context=131072,
          rotation=True, key_outlier_mult=20.0),
}

# Bit-width sweep of the paged workload (key bits, value bits).
SWEEP_BITS = [(4, 4), (4, 2), (2, 4), (2, 2), (1, 2)]
# Widths between the powers of two on the same paged workload: K3V3 at the payload of K4V2 and
# K2V4 (6 bits per key-value pair), and K3V2, K5V3, K6V2.
PLANE_BITS = [(3, 3), (3, 2), (5, 3), (6, 2)]
