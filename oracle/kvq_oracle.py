"""CPU oracle for decode attention over a group-wise quantized KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in ``oracle/``.
The product path (the HIP library and its Python binding) never calls it and
shares no code with it.

Plain, slow, numpy fp64.  Each function cites the passage it follows.  Sources:

* [P1] nalar.dev, "Kuantisasi KV cache mengganggu attention melalui key dan
  value tersimpan" (KV-cache quantization disturbs attention through the stored
  keys and values).  Sections used: "Error pada key masuk sebelum softmax"
  (the attention equations and the key-error identity), "Error pada value masuk
  setelah bobot attention terbentuk" (the value-error identity), "Granularitas
  kuantisasi menentukan nilai yang berbagi scale" (groups sharing a scale and a
  zero point / offset), "Pertumbuhan cache mengubah trade pada serving"
  (memory accounting; recent tokens kept at higher precision).
* [P2] nalar.dev tag index "Kuantisasi on Nalar", item "Outlier Aktivasi Dapat
  Menentukan Skala untuk Seluruh Grup Kuantisasi" (one outlier widens the
  group's scale).
* [P3] gist.science technical summary of arXiv 2502.15075, "Quantize What
  Counts: More for Keys, Less for Values".  Sections "Methodologie" and
  "Resultaten" (key-only rotation, group sizes 32 for keys and 64/128 for
  values), "Belangrijkste Bijdragen" (K4V2, 25% memory saving vs K4V4).

Readings taken where the pages leave a step open (all listed in the design doc):

* Groups are runs of G consecutive channels of one token's vector of one kv
  head.
* The zero point is the real value of code 0 (an offset): x_hat = zero + c*scale.
* fp16 metadata with directed rounding: zero = RD16(min), scale =
  RU16((max - zero) / (2^b - 1)), bumped one fp16 ulp if zero + (2^b-1)*scale
  still falls short of max; min and max are taken after adding +0.0 (so -0
  becomes +0).
* Codes: round half to even of (x - zero)/scale in fp64, clamped to
  [0, 2^b - 1]; all codes 0 when scale is 0.
* Sliding recent window: token t of a sequence of length L is stored
  unquantized iff t >= L - R.
* Key rotation: 128-point normalized Sylvester Walsh-Hadamard transform,
  butterflies in stage order h = 1, 2, ..., d/2 on fp64, then a multiply by
  c = RN64(2^-3.5).  Window keys stay raw and are scored with the raw query.
* Value rotation (a variant): the same transform on the values before they are
  quantized; the attention output over the quantized tokens is transformed back
  (the normalized Sylvester matrix is symmetric and orthogonal, its own inverse).
* GQA: query head h reads kv head floor(h / g), g = Hq / Hkv.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
F16 = np.float16

# RN_fp64(2**-3.5) = RN_fp64(1/sqrt(128)); 1/sqrt(128.0) in fp64 is one ulp low.
WHT_C = float.fromhex("0x1.6a09e667f3bcdp-4")


# --------------------------------------------------------------------------
# fp16 directed rounding of fp64 values  ([P1] "Granularitas ...": the scale
# and zero point are stored at some precision; fp16 is the precision fixed here)
# --------------------------------------------------------------------------
def fp16_round_down(x: np.ndarray) -> np.ndarray:
    """Largest fp16 value <= x (x finite, |x| < 65504).  Returns float16."""
    x = np.asarray(x, dtype=F64)
    h = x.astype(F16)  # round to nearest even
    over = h.astype(F64) > x
    return np.where(over, np.nextafter(h, F16(-np.inf)), h).astype(F16)


def fp16_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest fp16 value >= x (x finite, |x| < 65504).  Returns float16."""
    x = np.asarray(x, dtype=F64)
    h = x.astype(F16)
    under = h.astype(F64) < x
    return np.where(under, np.nextafter(h, F16(np.inf)), h).astype(F16)


def f16_bits(h: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(h, dtype=F16).view(np.uint16)


# --------------------------------------------------------------------------
# Group-wise asymmetric quantizer  ([P1] "Granularitas kuantisasi menentukan
# nilai yang berbagi scale"; group sizes and K/V bit split from [P3]
# "Resultaten" and "Belangrijkste Bijdragen")
# --------------------------------------------------------------------------
def group_metadata(xg: np.ndarray, bits: int):
    """Scale and zero point of each group.

    xg: [..., G] fp64 values of the groups.  Returns (scale, zero) as float16
    arrays of shape [...].
    """
    qmax = float((1 << bits) - 1)
    m = xg.min(axis=-1) + 0.0
    M = xg.max(axis=-1) + 0.0
    zero = fp16_round_down(m)
    zf = zero.astype(F64)
    scale = fp16_round_up((M - zf) / qmax)
    sf = scale.astype(F64)
    short = (zf + qmax * sf) < M  # coverage fix-up: one fp16 ulp up
    scale = np.where(short, np.nextafter(scale, F16(np.inf)), scale).astype(F16)
    return scale, zero


def group_codes(xg: np.ndarray, scale: np.ndarray, zero: np.ndarray, bits: int) -> np.ndarray:
    """Integer codes of each element: RNE((x - zero) / scale), clamped."""
    qmax = float((1 << bits) - 1)
    sf = scale.astype(F64)[..., None]
    zf = zero.astype(F64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = (xg - zf) / sf
    c = np.clip(np.rint(y), 0.0, qmax)
    c = np.where(sf == 0.0, 0.0, c)
    return c.astype(np.uint8)


def quantize(x: np.ndarray, bits: int, group: int):
    """Quantize vectors along the last axis in groups of ``group`` channels.

    x: [..., d] values (exactly representable in fp64).
    Returns codes uint8 [..., d], scale float16 [..., d/group], zero float16 [..., d/group].
    """
    x = np.asarray(x, dtype=F64)
    d = x.shape[-1]
    if d % group:
        raise ValueError("group must divide the vector length")
    xg = x.reshape(*x.shape[:-1], d // group, group)
    scale, zero = group_metadata(xg, bits)
    codes = group_codes(xg, scale, zero, bits)
    return codes.reshape(x.shape), scale, zero


def dequantize(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, group: int) -> np.ndarray:
    """x_hat = zero + c * scale in fp64 ([P1] "Granularitas ...": offset convention)."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    cg = codes.reshape(*codes.shape[:-1], d // group, group).astype(F64)
    xh = zero.astype(F64)[..., None] + cg * scale.astype(F64)[..., None]
    return xh.reshape(codes.shape)


# --------------------------------------------------------------------------
# Key-only rotation  ([P3] "Methodologie", "Belangrijkste Bijdragen" and
# "Resultaten": rotation applied to keys only, to spread key outliers)
# --------------------------------------------------------------------------
def wht_rotate(x: np.ndarray) -> np.ndarray:
    """Normalized Walsh-Hadamard transform along the last axis (fp64).

    Butterfly stages h = 1, 2, 4, ...: (a, b) -> (a + b, a - b) on index pairs
    (i, i + h) with (i & h) == 0, then every element times WHT_C.  This is the
    Sylvester-ordered Hadamard matrix divided by sqrt(128) for d = 128.
    """
    y = np.array(x, dtype=F64, copy=True)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("rotation needs a power-of-two length")
    if d != 128:
        raise ValueError("the normalization constant is fixed for d = 128")
    h = 1
    while h < d:
        idx = np.arange(d)
        lo = idx[(idx & h) == 0]
        a = y[..., lo].copy()
        b = y[..., lo + h].copy()
        y[..., lo] = a + b
        y[..., lo + h] = a - b
        h *= 2
    return y * WHT_C


# --------------------------------------------------------------------------
# Recent-token window  ([P1] "Pertumbuhan cache mengubah trade pada serving")
# --------------------------------------------------------------------------
def quantized_mask(L: int, R: int) -> np.ndarray:
    """True for the tokens of a length-L sequence that are stored quantized."""
    return np.arange(L) < (L - R)


# --------------------------------------------------------------------------
# Cache of one (sequence, kv head)
# --------------------------------------------------------------------------
def build_unit_cache(K: np.ndarray, V: np.ndarray, L: int, wl_params: dict):
    """Quantized cache state of one (sequence, kv head) after L tokens.

    K, V: [L][d] raw values (exactly representable in fp64).
    wl_params: k_bits, k_group, v_bits, v_group, window, rotation and optionally
    value_rotation.
    Returns a dict with the codes and fp16 metadata of the quantized tokens,
    the dequantized keys and values (rotated domain when the respective
    rotation is on), and the raw window tokens.
    """
    R = wl_params["window"]
    nq = max(0, L - R)
    Kq = np.asarray(K[:nq], dtype=F64)
    if wl_params["rotation"]:
        Kq = wht_rotate(Kq)
    Vq = np.asarray(V[:nq], dtype=F64)
    v_rot = bool(wl_params.get("value_rotation", False))
    if v_rot:
        Vq = wht_rotate(Vq)
    kc, ks, kz = quantize(Kq, wl_params["k_bits"], wl_params["k_group"])
    vc, vs, vz = quantize(Vq, wl_params["v_bits"], wl_params["v_group"])
    return dict(
        nq=nq,
        k_rotated=bool(wl_params["rotation"]),
        v_rotated=v_rot,
        k_codes=kc, k_scale=ks, k_zero=kz,
        v_codes=vc, v_scale=vs, v_zero=vz,
        k_hat=dequantize(kc, ks, kz, wl_params["k_group"]),
        v_hat=dequantize(vc, vs, vz, wl_params["v_group"]),
        k_win=np.asarray(K[nq:L], dtype=F64),
        v_win=np.asarray(V[nq:L], dtype=F64),
    )


# --------------------------------------------------------------------------
# Attention  ([P1] "Error pada key masuk sebelum softmax": s = q K^T / sqrt(d),
# a = softmax(s), o = a V)
# --------------------------------------------------------------------------
def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=F64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """One head: q [d], K [T][d], V [T][d] -> o [d]."""
    s = (np.asarray(K, dtype=F64) @ np.asarray(q, dtype=F64)) * scale
    return softmax(s) @ np.asarray(V, dtype=F64)


def unit_scores(q: np.ndarray, cache: dict, scale: float, rotation: bool) -> np.ndarray:
    """Scores of one query head against one unit cache: quantized tokens then window."""
    q = np.asarray(q, dtype=F64)
    qk = wht_rotate(q) if rotation else q
    s_q = cache["k_hat"] @ qk
    s_w = cache["k_win"] @ q
    return np.concatenate([s_q, s_w]) * scale


def unit_attention(q: np.ndarray, cache: dict, scale: float, rotation: bool) -> np.ndarray:
    """Decode attention of one query head over one (sequence, kv head) cache.

    With value rotation the quantized tokens' values are in the rotated domain:
    their weighted sum is transformed back before the window tokens are added.
    """
    s = unit_scores(q, cache, scale, rotation)
    a = softmax(s)
    nq = cache["nq"]
    if cache.get("v_rotated", False):
        return wht_rotate(a[:nq] @ cache["v_hat"]) + a[nq:] @ cache["v_win"]
    Vall = np.concatenate([cache["v_hat"], cache["v_win"]], axis=0)
    return a @ Vall


def decode_attention(q: np.ndarray, caches: list, num_kv_heads: int, scale: float, rotation: bool) -> np.ndarray:
    """All query heads of one sequence: q [Hq][d], caches[kvh] -> o [Hq][d] fp64.

    Query head h reads kv head floor(h / g).
    """
    Hq = q.shape[0]
    g = Hq // num_kv_heads
    out = np.empty(q.shape, dtype=F64)
    for h in range(Hq):
        out[h] = unit_attention(q[h], caches[h // g], scale, rotation)
    return out


# --------------------------------------------------------------------------
# Error budgets  ([P1] "Error pada key masuk sebelum softmax": a key error E_K
# moves the scores by q E_K^T / sqrt(d) before the softmax; "Error pada value
# masuk setelah bobot attention terbentuk": with the weights fixed, a value
# error moves the output by a E_V; "Evaluasi harus sesuai ...": judge the
# attention quantities, not only reconstruction error; [P2] entries on
# separate key and value error budgets)
# --------------------------------------------------------------------------
def error_budget(q: np.ndarray, K: np.ndarray, V: np.ndarray, cache: dict, scale: float):
    """Error statistics of one query head against one unit cache.

    K, V: the original [L][d] rows; cache: build_unit_cache of the same rows.
    Window positions are stored exactly, so their reconstruction is the row.
    Reconstructions of rotated tensors are rotated back first (the transform is
    its own inverse): every error is taken in the original domain.
    Returns (head, unit):
      head = [max |s' - s|, rms (s' - s), TV(a', a), |a V_hat - a V|,
              |a' V - a V|, |a' V_hat - a V|, |a V|, 0]
        with s = scale K q, s' = scale K_hat q, a = softmax(s), a' = softmax(s');
        the fourth entry is the value error alone (a E_V), the fifth the key
        error alone, the sixth both; TV is half the L1 distance.
      unit = [sum E_K^2, sum E_V^2, max |E_K|, max |E_V|, sum K^2, sum V^2,
              number of quantized positions, 0] over the quantized positions.
    An empty sequence gives zeros.
    """
    nq = cache["nq"]
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    L = K.shape[0]
    k_hat = wht_rotate(cache["k_hat"]) if cache.get("k_rotated", False) else cache["k_hat"]
    v_hat = wht_rotate(cache["v_hat"]) if cache.get("v_rotated", False) else cache["v_hat"]
    EK = k_hat - K[:nq]
    EV = v_hat - V[:nq]
    unit = np.array([np.sum(EK * EK), np.sum(EV * EV),
                     np.max(np.abs(EK)) if nq else 0.0, np.max(np.abs(EV)) if nq else 0.0,
                     np.sum(K[:nq] ** 2), np.sum(V[:nq] ** 2), float(nq), 0.0])
    if L == 0:
        return np.zeros(8), unit
    K_hat = np.concatenate([k_hat, K[nq:]])
    V_hat = np.concatenate([v_hat, V[nq:]])
    q = np.asarray(q, dtype=F64)
    s = (K @ q) * scale
    s_q = (K_hat @ q) * scale
    a = softmax(s)
    a_q = softmax(s_q)
    o = a @ V
    ds = s_q - s
    head = np.array([
        np.max(np.abs(ds)),
        np.sqrt(np.mean(ds * ds)),
        0.5 * np.sum(np.abs(a_q - a)),
        np.linalg.norm(a @ V_hat - o),
        np.linalg.norm(a_q @ V - o),
        np.linalg.norm(a_q @ V_hat - o),
        np.linalg.norm(o),
        0.0,
    ])
    return head, unit


# --------------------------------------------------------------------------
# Memory accounting  ([P1] "Pertumbuhan cache ...": payload plus metadata;
# [P3] "Belangrijkste Bijdragen": K4V2 vs K4V4)
# --------------------------------------------------------------------------
def bytes_per_token_head(d: int, k_bits: int, k_group: int, v_bits: int, v_group: int, meta_bytes: int = 4) -> float:
    """Stored bytes of one quantized token of one kv head: codes + (scale, zero) per group."""
    return d * k_bits / 8 + (d // k_group) * meta_bytes + d * v_bits / 8 + (d // v_group) * meta_bytes


def payload_bits_per_element_pair(k_bits: int, v_bits: int) -> int:
    return k_bits + v_bits
