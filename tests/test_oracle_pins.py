"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own code path: exact rational
arithmetic, a brute-force search over all fp16 values or all codes, high
precision decimal attention, a textbook library routine, closed forms, or
hand-derived fixtures in tests/golden/.  ``test_oracle_mutations.py`` plants
mistakes in the oracle and shows that these checks catch them.
"""
import json
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

# ---------------------------------------------------------------------------
# Independent helpers (no oracle code)
# ---------------------------------------------------------------------------
_ALL_F16 = None


def all_finite_fp16_sorted():
    """All finite fp16 values as sorted fp64 (with -0 and +0 both present)."""
    global _ALL_F16
    if _ALL_F16 is None:
        v = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
        v = v[np.isfinite(v)]
        _ALL_F16 = np.unique(v)  # sorted, -0 and +0 collapse to one entry (0.0)
    return _ALL_F16


def rd16_brute(x):
    """Largest fp16 <= x by search over all fp16 values (comparisons exact in fp64)."""
    t = all_finite_fp16_sorted()
    i = np.searchsorted(t, x, side="right") - 1
    return t[i]


def ru16_brute(x):
    t = all_finite_fp16_sorted()
    i = np.searchsorted(t, x, side="left")
    return t[i]


def exact_group_quant(xs, bits):
    """Exact-rational quantizer of one group: returns zero, scale (Fractions) and codes.

    zero: largest fp16 <= min; scale: smallest fp16 s with zero + (2^b-1)s >= max;
    code: nearest integer to (x - zero)/scale in exact arithmetic, ties to even.
    """
    qmax = (1 << bits) - 1
    m, M = min(xs), max(xs)
    zero = Fraction(float(rd16_brute(m)))
    cand = all_finite_fp16_sorted()
    need = (Fraction(M) - zero) / qmax
    # smallest fp16 >= need
    s = None
    for v in cand[np.searchsorted(cand, float(need) * (1 - 1e-12) if need > 0 else 0.0, side="left"):]:
        if Fraction(float(v)) >= need:
            s = Fraction(float(v))
            break
    codes = []
    near_tie = []
    for x in xs:
        if s == 0:
            codes.append(0)
            near_tie.append(False)
            continue
        y = (Fraction(x) - zero) / s
        fl = int(np.floor(float(y)))
        # exact floor around the float estimate
        while Fraction(fl) > y:
            fl -= 1
        while Fraction(fl + 1) <= y:
            fl += 1
        frac = y - fl
        if frac > Fraction(1, 2):
            c = fl + 1
        elif frac < Fraction(1, 2):
            c = fl
        else:
            c = fl if fl % 2 == 0 else fl + 1
        codes.append(min(max(c, 0), qmax))
        # within fp64 rounding of the division of a tie: both neighbours acceptable
        near_tie.append(abs(frac - Fraction(1, 2)) <= abs(y) * Fraction(1, 2 ** 51) and frac != Fraction(1, 2))
    return zero, s, codes, near_tie


def dec_attention(q, K, V, scale):
    """High-precision (50 digit) softmax attention of one head, returns floats."""
    getcontext().prec = 50
    qd = [Decimal(float(v)) for v in q]
    s = []
    for row in K:
        s.append(sum(Decimal(float(a)) * b for a, b in zip(row, qd)) * Decimal(scale))
    mx = max(s)
    e = [(x - mx).exp() for x in s]
    Z = sum(e)
    out = []
    for c in range(len(V[0])):
        out.append(float(sum(e[t] * Decimal(float(V[t][c])) for t in range(len(V))) / Z))
    return np.array(out)


def random_bf16_like(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    u = x.view(np.uint32)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Check functions (also used by the mutation tests)
# ---------------------------------------------------------------------------
def check_fp16_directed(O_):
    rng = np.random.default_rng(1)
    xs = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 4, 4000),
        all_finite_fp16_sorted()[::97],
        np.array([0.0, -0.0, 0.1, -0.1, 65504.0, -65504.0, 2.0 ** -24, 3 * 2.0 ** -26, 2.0 ** -30]),
    ])
    xs = xs[np.abs(xs) < 65504]
    rd = O_.fp16_round_down(xs).astype(np.float64)
    ru = O_.fp16_round_up(xs).astype(np.float64)
    assert np.array_equal(rd, rd16_brute(xs)), "RD16 differs from brute force"
    assert np.array_equal(ru, ru16_brute(xs)), "RU16 differs from brute force"


def check_golden(O_):
    with open(os.path.join(HERE, "golden", "quant_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], dtype=np.float64)
        codes, scale, zero = O_.quantize(x, c["bits"], len(x))
        assert int(O_.f16_bits(zero)[0]) == int(c["zero_bits"], 16), c["name"]
        assert int(O_.f16_bits(scale)[0]) == int(c["scale_bits"], 16), c["name"]
        assert codes.tolist() == c["codes"], c["name"]
        xh = O_.dequantize(codes, scale, zero, len(x))
        assert xh.tolist() == [float(Fraction(v)) for v in c["x_hat"]], c["name"]


def check_group_invariants(O_, bits, G, n=600, seed=0):
    rng = np.random.default_rng(seed + bits)
    x = random_bf16_like(rng, (n, G), 1.0)
    x[: n // 4] *= 10.0 ** rng.integers(-6, 3, (n // 4, 1))
    x[n // 4: n // 4 + 8, 3] += 300.0  # outliers
    codes, scale, zero = O_.quantize(x, bits, G)
    qmax = (1 << bits) - 1
    assert codes.max() <= qmax
    sf, zf = scale.astype(np.float64), zero.astype(np.float64)
    m, M = x.min(-1, keepdims=True), x.max(-1, keepdims=True)
    # coverage and minimality (pins the directed rounding exactly)
    assert np.all(zf <= m)
    nxt = np.nextafter(zero, np.float16(np.inf)).astype(np.float64)
    assert np.all(nxt > m), "zero is not the largest fp16 <= min"
    assert np.all(zf + qmax * sf >= M)
    prev = np.nextafter(scale, np.float16(-np.inf)).astype(np.float64)
    ok_min = (sf == 0) | (zf + qmax * prev < M)
    assert np.all(ok_min), "scale is not the smallest covering fp16"
    # reconstruction bound |x - x_hat| <= scale * (1/2 + qmax * 2^-53)
    xh = O_.dequantize(codes, scale, zero, G)
    err = np.abs(x - xh)
    assert np.all(err <= sf[:, 0:1] * (0.5 + qmax * 2.0 ** -53) + 0.0)


def check_brute_force_codes(O_, bits, G=8, n=300, seed=3):
    rng = np.random.default_rng(seed + 7 * bits)
    x = random_bf16_like(rng, (n, G), 2.0)
    # constructed exact ties: x - zero = (k + 1/2) * scale with dyadic values
    ties = np.array([[0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.0]]) * 1.0
    ties = ties[:, :G] if G <= 8 else np.pad(ties, ((0, 0), (0, G - 8)))
    x = np.concatenate([x, ties * (2 ** bits - 1) / 3.0])
    codes, scale, zero = O_.quantize(x, bits, G)
    for i in range(x.shape[0]):
        z, s, c, near = exact_group_quant([float(v) for v in x[i]], bits)
        assert Fraction(float(zero[i, 0])) == z, i
        assert Fraction(float(scale[i, 0])) == s, i
        for j in range(G):
            if not near[j]:
                assert codes[i, j] == c[j], (i, j)
        # dequantization is exact
        xh = O_.dequantize(codes[i], scale[i], zero[i], G)
        for j in range(G):
            assert Fraction(float(xh[j])) == z + int(codes[i, j]) * s


def check_wht(O_):
    from scipy.linalg import hadamard

    getcontext().prec = 60
    c_exact = Decimal(2) ** Decimal("-3.5")
    assert O_.WHT_C == float(c_exact)  # float(Decimal) rounds to nearest
    H = hadamard(128).astype(np.float64) / np.sqrt(128.0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((20, 128))
    y = O_.wht_rotate(x)
    assert np.max(np.abs(y - x @ H.T)) < 1e-14
    assert np.max(np.abs(O_.wht_rotate(y) - x)) < 1e-14
    E = np.eye(128)
    HE = O_.wht_rotate(E)
    assert np.all(np.abs(np.abs(HE) - O_.WHT_C) == 0.0)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    assert abs(O_.wht_rotate(q) @ O_.wht_rotate(k) - q @ k) < 1e-12


def check_attention_library(O_):
    import torch

    rng = np.random.default_rng(11)
    for T in (1, 7, 300):
        q = rng.standard_normal(128)
        K = rng.standard_normal((T, 128)) * 2.0
        V = rng.standard_normal((T, 128))
        o = O_.attention(q, K, V, 1.0 / np.sqrt(128.0))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q).view(1, 1, 1, 128), torch.tensor(K).view(1, 1, T, 128), torch.tensor(V).view(1, 1, T, 128)
        ).view(128).numpy()
        assert np.max(np.abs(o - ref)) < 1e-12


def check_attention_decimal(O_):
    rng = np.random.default_rng(12)
    for d, T in ((2, 1), (4, 3), (8, 5)):
        q = rng.standard_normal(d)
        K = rng.standard_normal((T, d)) * 3
        V = rng.standard_normal((T, d))
        sc = 1.0 / np.sqrt(d)
        o = O_.attention(q, K, V, sc)
        ref = dec_attention(q, K, V, sc)
        assert np.max(np.abs(o - ref)) < 1e-13


def _params(R=0, rot=False, kb=4, vb=2):
    return dict(k_bits=kb, k_group=32, v_bits=vb, v_group=128, window=R, rotation=rot)


def check_end_to_end_exact(O_):
    """Tiny unit: quantize with exact rationals, attend in 50-digit decimal."""
    rng = np.random.default_rng(21)
    L, d, R = 6, 128, 2
    K = random_bf16_like(rng, (L, d), 1.0)
    K[:, 5] *= 10.0
    V = random_bf16_like(rng, (L, d), 1.0)
    q = random_bf16_like(rng, (d,), 1.0)
    cache = O_.build_unit_cache(K, V, L, _params(R=R))
    o = O_.unit_attention(q, cache, 1.0 / np.sqrt(d), False)
    Kh = np.array(K)
    Vh = np.array(V)
    for t in range(L - R):
        for gi in range(d // 32):
            z, s, c, _ = exact_group_quant(list(K[t, 32 * gi: 32 * gi + 32]), 4)
            Kh[t, 32 * gi: 32 * gi + 32] = [float(z + ci * s) for ci in c]
        z, s, c, _ = exact_group_quant(list(V[t]), 2)
        Vh[t] = [float(z + ci * s) for ci in c]
    ref = dec_attention(q, Kh, Vh, 1.0 / np.sqrt(d))
    assert np.max(np.abs(o - ref)) < 1e-13


def check_error_identities(O_):
    """Key error enters before the softmax, value error after it ([P1])."""
    rng = np.random.default_rng(31)
    L, d = 40, 128
    K = random_bf16_like(rng, (L, d), 1.0)
    V = random_bf16_like(rng, (L, d), 1.0)
    q = random_bf16_like(rng, (d,), 1.0)
    sc = 1.0 / np.sqrt(d)
    cache = O_.build_unit_cache(K, V, L, _params())
    # key path: s' = s + q E_K^T / sqrt(d)
    s_prime = O_.unit_scores(q, cache, sc, False)
    E_K = cache["k_hat"] - K
    assert np.max(np.abs(s_prime - ((K @ q) * sc + (E_K @ q) * sc))) < 1e-12
    # value path with exact keys: o' = o + a E_V
    a = O_.softmax((K @ q) * sc)
    c2 = dict(cache)
    c2["k_hat"] = K.copy()
    o_prime = O_.unit_attention(q, c2, sc, False)
    E_V = cache["v_hat"] - V
    assert np.max(np.abs(o_prime - (a @ V + a @ E_V))) < 1e-12


def check_window(O_):
    rng = np.random.default_rng(41)
    L, d = 50, 128
    K = random_bf16_like(rng, (L, d), 1.0)
    V = random_bf16_like(rng, (L, d), 1.0)
    q = random_bf16_like(rng, (d,), 1.0)
    sc = 1.0 / np.sqrt(d)
    # R >= L: nothing quantized -> exact attention
    full = O_.build_unit_cache(K, V, L, _params(R=L))
    assert full["nq"] == 0
    assert np.max(np.abs(O_.unit_attention(q, full, sc, False) - O_.attention(q, K, V, sc))) < 1e-13
    # ring-buffer simulation of appends gives the same quantized set
    for R in (0, 1, 7, 16, 49, 50, 64):
        ring = [None] * max(R, 1)
        quantized = set()
        for t in range(L):
            if R == 0:
                quantized.add(t)
                continue
            old = ring[t % R]
            if old is not None:
                quantized.add(old)
            ring[t % R] = t
        mask = O_.quantized_mask(L, R)
        assert set(np.nonzero(mask)[0].tolist()) == quantized, R


def check_gqa(O_):
    d, Hkv, g = 128, 4, 3
    rng = np.random.default_rng(51)
    caches = []
    for kvh in range(Hkv):
        L = 5
        K = random_bf16_like(rng, (L, d), 1.0)
        V = np.full((L, d), float(kvh + 1))  # constant value per kv head
        caches.append(O_.build_unit_cache(K, V, L, _params(R=L)))
    q = rng.standard_normal((Hkv * g, d))
    o = O_.decode_attention(q, caches, Hkv, 1.0 / np.sqrt(d), False)
    for h in range(Hkv * g):
        assert np.allclose(o[h], h // g + 1, atol=1e-13, rtol=0)


def check_rotation_special_case(O_):
    """Rotation on with nothing quantized equals the unrotated result (H orthonormal)."""
    rng = np.random.default_rng(61)
    L, d = 30, 128
    K = random_bf16_like(rng, (L, d), 1.0)
    V = random_bf16_like(rng, (L, d), 1.0)
    q = random_bf16_like(rng, (d,), 1.0)
    sc = 1.0 / np.sqrt(d)
    cache = O_.build_unit_cache(K, V, L, _params(R=L, rot=True))
    assert np.max(np.abs(O_.unit_attention(q, cache, sc, True) - O_.attention(q, K, V, sc))) < 1e-13
    # quantized rotated keys: scores equal (H q) . k_hat_rot
    cache = O_.build_unit_cache(K, V, L, _params(R=0, rot=True))
    s = O_.unit_scores(q, cache, sc, True)
    from scipy.linalg import hadamard
    H = hadamard(128) / np.sqrt(128.0)
    assert np.max(np.abs(s - (cache["k_hat"] @ (H @ q)) * sc)) < 1e-12


def check_value_rotation(O_):
    """Value rotation (a variant): the output over the quantized tokens is the Hadamard matrix
    (scipy's, normalized — a route independent of the oracle's butterflies) applied to the
    weighted dequantized rotated values; and, with the same quantized keys, it stays within the
    value quantization error of attention over the raw values: the rotation back is orthogonal,
    so |o - o_raw|_2 <= max_t |v_hat_t - v_t|_2 <= sqrt(128) * max scale / 2."""
    from scipy.linalg import hadamard

    H = hadamard(128) / np.sqrt(128.0)
    rng = np.random.default_rng(91)
    L, d = 40, 128
    K = random_bf16_like(rng, (L, d), 1.0)
    V = random_bf16_like(rng, (L, d), 1.0)
    V[:, 3] *= 12.0  # an outlier channel, which the rotation spreads
    q = random_bf16_like(rng, (d,), 1.0)
    sc = 1.0 / np.sqrt(d)
    for vb in (2, 4, 8):
        prm = dict(_params(R=0, kb=4, vb=vb), value_rotation=True)
        cache = O_.build_unit_cache(K, V, L, prm)
        o = O_.unit_attention(q, cache, sc, False)
        a = O_.softmax(cache["k_hat"] @ q * sc)
        assert np.max(np.abs(o - H @ (a @ cache["v_hat"]))) < 1e-12
        o_raw = a @ V.astype(np.float64)
        bound = np.sqrt(128.0) * np.max(cache["v_scale"].astype(np.float64)) / 2
        assert np.linalg.norm(o - o_raw) <= bound * (1 + 1e-12)
        # the rotated values really are what was quantized: codes of H v, not of v
        c, _, _ = O_.quantize(V.astype(np.float64) @ H, vb, 128)
        assert np.array_equal(cache["v_codes"], c)


def check_memory_model(O_):
    expect = {(4, 2): 116, (4, 4): 148, (2, 4): 116, (2, 2): 84, (1, 2): 68,
              (3, 2): 100, (5, 3): 148, (6, 2): 148, (3, 3): 116, (7, 1): 148}
    for (kb, vb), b in expect.items():
        assert O_.bytes_per_token_head(128, kb, 32, vb, 128) == b
    # payload only: K4V2 vs K4V4 is 6/8 = 75% -> the 25% saving of [P3]
    assert Fraction(O_.payload_bits_per_element_pair(4, 2), O_.payload_bits_per_element_pair(4, 4)) == Fraction(3, 4)


def check_group_size_monotone(O_):
    rng = np.random.default_rng(71)
    x = random_bf16_like(rng, (400, 128), 1.0)
    x[:, 7] *= 15.0
    for bits in range(1, 9):
        _, s32, _ = O_.quantize(x, bits, 32)
        _, s128, _ = O_.quantize(x, bits, 128)
        assert np.all(s32.astype(np.float64) <= s128.astype(np.float64)[:, 0:1])


def check_outlier(O_):
    rng = np.random.default_rng(81)
    x = random_bf16_like(rng, (200, 32), 1.0)
    for bits in (2, 3, 4, 5, 6):
        for delta in (10.0, 100.0):
            y = x.copy()
            others = np.delete(y, 5, axis=1)
            y[:, 5] = others.min(-1) + delta  # the group minimum stays where it was
            _, s, _ = O_.quantize(y, bits, 32)
            assert np.all(s.astype(np.float64)[:, 0] >= delta / ((1 << bits) - 1))


def check_error_budget(O_):
    """Error budgets, pinned by what the definitions force rather than by retyping them:
    * an exact cache gives zero errors and |a V| equal to scipy-softmax attention's norm;
    * keys shifted by one common vector u move every score by scale q.u: the max and rms score
      errors equal |scale q.u|, while the weights, and so TV and the key-only output error, do
      not move (softmax is shift invariant);
    * on a real quantization, the value-only output error equals |a E_V| with a from scipy's
      softmax ([P1]'s o' = o + a E_V), TV equals half the L1 distance of scipy softmaxes, and
      the key-only and joint errors equal the distances between attention outputs; window
      positions carry no error and the unit statistics cover exactly the L - R quantized ones."""
    from scipy.special import softmax as sp_softmax

    rng = np.random.default_rng(101)
    L, d = 50, 128
    K = random_bf16_like(rng, (L, d), 1.0)
    K[:, 9] *= 10.0
    V = random_bf16_like(rng, (L, d), 1.0)
    q = random_bf16_like(rng, (d,), 1.0)
    sc = 1.0 / np.sqrt(d)
    exact = dict(nq=L, k_hat=K.copy(), v_hat=V.copy(), k_win=K[L:], v_win=V[L:])
    head, unit = O_.error_budget(q, K, V, exact, sc)
    o_ref = sp_softmax(K @ q * sc) @ V
    assert np.all(head[:6] == 0) and np.all(unit[:4] == 0)
    assert abs(head[6] - np.linalg.norm(o_ref)) < 1e-12 and unit[6] == L
    u = random_bf16_like(rng, (d,), 0.3)
    shifted = dict(exact, k_hat=K + u)
    head, unit = O_.error_budget(q, K, V, shifted, sc)
    shift = abs(sc * float(q @ u))
    assert shift > 1e-3
    assert abs(head[0] - shift) < 1e-9 and abs(head[1] - shift) < 1e-9
    assert head[2] < 1e-12 and head[4] < 1e-9 and head[3] == 0
    assert abs(unit[0] - L * float(u @ u)) < 1e-8 * L * float(u @ u)
    for kb, vb, R in ((4, 2, 0), (2, 4, 7), (1, 1, 12)):
        prm = _params(R=R, kb=kb, vb=vb)
        cache = O_.build_unit_cache(K, V, L, prm)
        head, unit = O_.error_budget(q, K, V, cache, sc)
        nq = L - R
        Kh = np.concatenate([cache["k_hat"], K[nq:]])
        Vh = np.concatenate([cache["v_hat"], V[nq:]])
        a = sp_softmax(K @ q * sc)
        a_q = sp_softmax(Kh @ q * sc)
        assert abs(head[3] - np.linalg.norm(a @ (Vh - V))) < 1e-12
        assert abs(head[2] - 0.5 * np.abs(a_q - a).sum()) < 1e-12
        assert abs(head[4] - np.linalg.norm(a_q @ V - a @ V)) < 1e-12
        assert abs(head[5] - np.linalg.norm(a_q @ Vh - a @ V)) < 1e-12
        assert unit[6] == nq
        assert abs(unit[1] - np.sum((Vh - V) ** 2)) < 1e-12 * max(1.0, unit[1])
        assert unit[2] == np.max(np.abs(Kh - K)) and head[0] == np.max(np.abs((Kh - K) @ q * sc))
        assert head[3] > 0 and head[4] > 0
    # rotated caches: the same statistics as an unrotated cache holding the hats rotated back
    # with scipy's (normalized) Hadamard matrix, a route independent of the oracle's butterflies
    from scipy.linalg import hadamard
    H = hadamard(128) / np.sqrt(128.0)
    for rot, vrot in ((True, False), (False, True), (True, True)):
        prm = dict(_params(R=0, rot=rot, kb=4, vb=2), value_rotation=vrot)
        cache = O_.build_unit_cache(K, V, L, prm)
        plain = dict(nq=L, k_hat=cache["k_hat"] @ H if rot else cache["k_hat"],
                     v_hat=cache["v_hat"] @ H if vrot else cache["v_hat"], k_win=K[L:], v_win=V[L:])
        head, unit = O_.error_budget(q, K, V, cache, sc)
        head_p, unit_p = O_.error_budget(q, K, V, plain, sc)
        assert np.allclose(head, head_p, rtol=1e-10, atol=1e-12) and np.allclose(unit, unit_p, rtol=1e-10, atol=1e-12)
        assert head[3] > 0 and head[4] > 0
    empty = O_.build_unit_cache(K[:0], V[:0], 0, _params())
    head, unit = O_.error_budget(q, K[:0], V[:0], empty, sc)
    assert np.all(head == 0) and np.all(unit == 0)


def check_one_bit_range_limit(O_):
    """1-bit groups at the edge of the fp16 range.  A group spanning [-32767.5, 32767.5] has
    zero = -32768 and needs a scale >= 65535.5: no finite fp16 reaches it (brute force over all of
    them), so the smallest fp16 >= the need is +inf, every code is 0 (x / inf rounds to 0) and the
    reconstruction is NaN.  The widest bf16 group below 2^15, [-32640, 32640], stays finite and
    agrees with the exact-rational quantizer."""
    xs = [-32767.5, -10.0, 0.0, 32767.5]
    zero = Fraction(float(rd16_brute(min(xs))))
    assert zero == -32768
    need = Fraction(max(xs)) - zero
    assert all(Fraction(float(v)) < need for v in all_finite_fp16_sorted()), "a finite fp16 covers the group"
    codes, scale, z = O_.quantize(np.array(xs), 1, len(xs))
    assert int(O_.f16_bits(scale)[0]) == 0x7C00, "scale is not +inf"
    assert Fraction(float(z[0])) == zero
    assert codes.tolist() == [0, 0, 0, 0]
    assert np.all(np.isnan(O_.dequantize(codes, scale, z, len(xs))))
    xs = [-32640.0, -3.0, 5.0, 32640.0]
    zero, sc, ref_codes, _ = exact_group_quant(xs, 1)
    codes, scale, z = O_.quantize(np.array(xs), 1, len(xs))
    assert np.isfinite(float(scale[0])) and Fraction(float(scale[0])) == sc and Fraction(float(z[0])) == zero
    assert codes.tolist() == ref_codes


ALL_CHECKS = [
    check_fp16_directed, check_golden, check_wht, check_attention_library, check_attention_decimal,
    check_end_to_end_exact, check_error_identities, check_window, check_gqa, check_rotation_special_case,
    check_memory_model, check_group_size_monotone, check_outlier, check_value_rotation, check_error_budget,
    check_one_bit_range_limit,
]


# ---------------------------------------------------------------------------
# Tests
# ---------------------------------------------------------------------------
def test_fp16_directed_rounding_matches_brute_force():
    check_fp16_directed(O)


def test_golden_hand_derived_examples():
    check_golden(O)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("G", [32, 128])
def test_group_invariants(bits, G):
    check_group_invariants(O, bits, G)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6])
def test_codes_match_exact_rational_brute_force(bits):
    check_brute_force_codes(O, bits)


def test_wht_closed_forms():
    check_wht(O)


def test_attention_equals_torch_sdpa_fp64():
    check_attention_library(O)


def test_attention_equals_decimal_brute_force():
    check_attention_decimal(O)


def test_end_to_end_exact_rational_and_decimal():
    check_end_to_end_exact(O)


def test_key_and_value_error_identities():
    check_error_identities(O)


def test_window_semantics():
    check_window(O)


def test_gqa_mapping():
    check_gqa(O)


def test_rotation_special_cases():
    check_rotation_special_case(O)


def test_memory_model_closed_form():
    check_memory_model(O)


def test_group_size_monotone():
    check_group_size_monotone(O)


def test_outlier_widens_scale():
    check_outlier(O)


def test_value_rotation_variant():
    check_value_rotation(O)


def test_bf16_rounding_helper_of_the_parity_tests():
    """The fp64 -> bf16 round-to-nearest-even used to state expected dense values, against exact
    rational rounding: random values, and exact ties between neighbours (which go to even)."""
    from fractions import Fraction

    import workloads as W
    from kvq_harness import bf16_bits_rne_f64

    def exact(x):
        if x == 0:
            return 0 if np.copysign(1.0, x) > 0 else 0x8000
        fx = Fraction(x)
        a = abs(fx)
        e = 0
        while a >= 2:
            a /= 2
            e += 1
        while a < 1:
            a *= 2
            e -= 1
        m = a * 128  # 8 significant bits: 128 <= m < 256
        r = int(m)
        frac = m - r
        if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and r % 2 == 1):
            r += 1
        val = Fraction(r, 128) * Fraction(2) ** e * (1 if fx > 0 else -1)
        return int(W.f32_to_bf16_bits(np.array([float(val)], dtype=np.float32))[0])

    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(300) * np.exp2(rng.integers(-30, 30, 300)))
    # exact ties: a bf16 value plus half its unit in the last place, both parities
    for m in (128, 129, 200, 255):
        for e in (-20, 0, 13):
            xs += [(m + 0.5) * 2.0 ** (e - 7), -(m + 0.5) * 2.0 ** (e - 7)]
    xs += [0.0, 1.0, -3.0]
    got = bf16_bits_rne_f64(np.array(xs))
    want = np.array([exact(x) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_error_budget_definitions():
    check_error_budget(O)


def test_one_bit_range_limit():
    check_one_bit_range_limit(O)
