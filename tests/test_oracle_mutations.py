"""Plant plausible mistakes in a private copy of the oracle and show the pins catch them.

Each mutation replaces one function of a freshly loaded copy of
``oracle/kvq_oracle.py`` (the real module is untouched) and runs every pin
check; at least one must fail.
"""
import importlib.util
import os

import numpy as np
import pytest

import test_oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kvq_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("kvq_oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def mut_zero_round_nearest(M):
    def group_metadata(xg, bits):
        qmax = float((1 << bits) - 1)
        m = xg.min(axis=-1) + 0.0
        Mx = xg.max(axis=-1) + 0.0
        zero = m.astype(np.float16)  # mistake: nearest instead of down
        scale = M.fp16_round_up((Mx - zero.astype(np.float64)) / qmax)
        return scale, zero
    M.group_metadata = group_metadata


def mut_scale_round_nearest(M):
    orig = M.fp16_round_up
    M.fp16_round_up = lambda x: np.asarray(x, dtype=np.float64).astype(np.float16)  # mistake
    M._orig = orig


def mut_round_half_up(M):
    def group_codes(xg, scale, zero, bits):
        qmax = float((1 << bits) - 1)
        sf = scale.astype(np.float64)[..., None]
        zf = zero.astype(np.float64)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            y = (xg - zf) / sf
        c = np.clip(np.floor(y + 0.5), 0.0, qmax)  # mistake: ties away from even
        return np.where(sf == 0.0, 0.0, c).astype(np.uint8)
    M.group_codes = group_codes


def mut_dequant_sign(M):
    def dequantize(codes, scale, zero, group):
        d = codes.shape[-1]
        cg = codes.reshape(*codes.shape[:-1], d // group, group).astype(np.float64)
        return (zero.astype(np.float64)[..., None] - cg * scale.astype(np.float64)[..., None]).reshape(codes.shape)
    M.dequantize = dequantize


def mut_dequant_group_index(M):
    def dequantize(codes, scale, zero, group):
        d = codes.shape[-1]
        cg = codes.reshape(*codes.shape[:-1], d // group, group).astype(np.float64)
        s = scale.astype(np.float64)[..., ::-1]  # mistake: groups paired with the wrong metadata
        z = zero.astype(np.float64)[..., ::-1]
        return (z[..., None] + cg * s[..., None]).reshape(codes.shape)
    M.dequantize = dequantize


def mut_attention_no_scale(M):
    orig = M.attention
    M.attention = lambda q, K, V, scale: orig(q, K, V, 1.0)  # mistake: softmax scale dropped
    orig_s = M.unit_scores
    M.unit_scores = lambda q, cache, scale, rotation: orig_s(q, cache, 1.0, rotation)


def mut_attention_reversed_values(M):
    def attention(q, K, V, scale):
        s = (np.asarray(K, dtype=np.float64) @ np.asarray(q, dtype=np.float64)) * scale
        return M.softmax(s) @ np.asarray(V, dtype=np.float64)[::-1]  # mistake: weights/values misaligned
    M.attention = attention

    def unit_attention(q, cache, scale, rotation):
        s = M.unit_scores(q, cache, scale, rotation)
        Vall = np.concatenate([cache["v_hat"], cache["v_win"]], axis=0)
        return M.softmax(s) @ Vall[::-1]
    M.unit_attention = unit_attention


def mut_gqa_modulo(M):
    def decode_attention(q, caches, num_kv_heads, scale, rotation):
        out = np.empty(q.shape)
        for h in range(q.shape[0]):
            out[h] = M.unit_attention(q[h], caches[h % num_kv_heads], scale, rotation)  # mistake
        return out
    M.decode_attention = decode_attention


def mut_window_off_by_one(M):
    M.quantized_mask = lambda L, R: np.arange(L) <= (L - R)  # mistake


def mut_wht_no_normalization(M):
    orig = M.wht_rotate
    M.wht_rotate = lambda x: orig(x) / M.WHT_C  # mistake: unnormalized Hadamard


def mut_wht_constant_low(M):
    M.WHT_C = 1.0 / np.sqrt(128.0)  # one ulp low


def mut_softmax_no_max_shift_wrong_axis(M):
    def softmax(s):
        e = np.exp(np.asarray(s, dtype=np.float64))
        return e / e.sum()  * (1.0 + 1e-9)  # mistake: normalization off
    M.softmax = softmax


def mut_value_rotation_not_undone(M):
    orig = M.unit_attention

    def unit_attention(q, cache, scale, rotation):
        if not cache.get("v_rotated", False):
            return orig(q, cache, scale, rotation)
        a = M.softmax(M.unit_scores(q, cache, scale, rotation))
        nq = cache["nq"]
        return a[:nq] @ cache["v_hat"] + a[nq:] @ cache["v_win"]  # mistake: output left in the rotated domain
    M.unit_attention = unit_attention


def mut_error_budget_weights_from_quantized_keys(M):
    orig = M.error_budget

    def error_budget(q, K, V, cache, scale):
        head, unit = orig(q, K, V, cache, scale)
        nq = cache["nq"]
        K_hat = np.concatenate([cache["k_hat"], np.asarray(K, dtype=np.float64)[nq:]])
        V_hat = np.concatenate([cache["v_hat"], np.asarray(V, dtype=np.float64)[nq:]])
        if len(K_hat):
            a_q = M.softmax(K_hat @ q * scale)
            head[3] = np.linalg.norm(a_q @ V_hat - a_q @ V)  # mistake: value error under the quantized weights
        return head, unit
    M.error_budget = error_budget


def mut_error_budget_rotated_domain(M):
    orig = M.error_budget

    def error_budget(q, K, V, cache, scale):
        c = dict(cache, k_rotated=False)  # mistake: rotated keys compared in the rotated domain
        return orig(q, K, V, c, scale)
    M.error_budget = error_budget


MUTATIONS = [
    mut_error_budget_rotated_domain, mut_error_budget_weights_from_quantized_keys, mut_value_rotation_not_undone, mut_zero_round_nearest, mut_scale_round_nearest, mut_round_half_up, mut_dequant_sign,
    mut_dequant_group_index, mut_attention_no_scale, mut_attention_reversed_values, mut_gqa_modulo,
    mut_window_off_by_one, mut_wht_no_normalization, mut_wht_constant_low, mut_softmax_no_max_shift_wrong_axis,
]


def run_all_checks(M):
    failures = []
    checks = list(P.ALL_CHECKS) + [
        lambda m: P.check_group_invariants(m, 2, 32, n=200),
        lambda m: P.check_brute_force_codes(m, 2, n=60),
    ]
    for chk in checks:
        try:
            chk(M)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failures.append((getattr(chk, "__name__", "lambda"), type(e).__name__))
    return failures


def test_unmutated_copy_passes():
    assert run_all_checks(fresh_oracle()) == []


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__)
def test_mutation_is_caught(mutation):
    M = fresh_oracle()
    mutation(M)
    assert run_all_checks(M), f"{mutation.__name__} was not caught by any pin"
