"""Pins of the oracle's 4-bit KV cache quantizer and of its decode attention
over that cache, against a worked example, exact bounds, closed forms and
invariants.  (QFactory notes 2.1: the asymmetric form x ~ (code - zero) *
scale; QServe talk summary: 4-bit keys and values with per-token scales and
zero points, read by the attention kernel.)"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e7_kv4_rows.json")
D = 128


def f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def kv(codes, s_bits, z):
    return {"codes": np.asarray(codes, np.uint8), "s": np.asarray(s_bits, np.uint16), "z": np.asarray(z, np.uint8)}


# --------------------------------------------------------------------------
# Quantizer
# --------------------------------------------------------------------------
def test_e7_worked_rows():
    g = json.load(open(GOLD))
    assert g["D"] == D
    x = np.zeros((len(g["rows"]), D), np.float16)
    for i, r in enumerate(g["rows"]):
        if "fill" in r:
            x[i] = r["fill"]
        for k, v in r.get("nonzero", {}).items():
            x[i, int(k)] = v
    q = orc.quantize_kv4(x)
    for i, r in enumerate(g["rows"]):
        assert int(q["s"][i]) == r["s_bits"], i
        assert int(q["z"][i]) == r["z"], i
        n = len(r["codes_head"])
        assert list(q["codes"][i, :n]) == r["codes_head"], i
        assert np.all(q["codes"][i, n:] == r["codes_rest"]), i


def random_rows(seed, n=4000):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, D)) * np.exp(rng.uniform(-6, 6, (n, 1)))
    x += rng.uniform(-3, 3, (n, 1)) * np.abs(x).mean(axis=1, keepdims=True) * (rng.random((n, 1)) < 0.3)
    x[rng.random((n, D)) < 0.02] *= 20.0                  # outlier channels
    return np.clip(x, -60000, 60000).astype(np.float16)


@pytest.mark.parametrize("seed", [1, 2])
def test_round_trip_error_bound(seed):
    """For every element: |x - (code - zero) s| <= s/2 + 15 |s - (hi - lo)/15| + 2^-18 s.
    Codes that do not clamp give rint(x/s) s (error s/2); only the top can clamp, and
    only by what rounding the scale down lost."""
    x = random_rows(seed)
    q = orc.quantize_kv4(x)
    xd = x.astype(np.float64)
    lo = np.minimum(0, xd.min(axis=1))
    hi = np.maximum(0, xd.max(axis=1))
    s = f16v(q["s"])
    assert np.all(s > 0)
    err = np.abs(xd - orc.kv4_dequant(q))
    bound = s / 2 + 15 * np.abs(s - (hi - lo) / 15) + 2.0 ** -18 * s
    assert np.all(err <= bound[:, None])
    # the scale is the fp16 rounding of the range over 15: within half an fp16 step
    assert np.all(np.abs(s - (hi - lo) / 15) <= 2.0 ** -11 * (hi - lo) / 15 + 2.0 ** -25)


def test_zero_is_exact_and_ranges():
    x = random_rows(3, 1000)
    x[:, 5] = 0
    q = orc.quantize_kv4(x)
    assert np.all(q["codes"] <= 15) and np.all(q["z"] <= 15)
    assert np.array_equal(q["codes"][:, 5], q["z"])                 # 0 -> the zero point
    assert np.all(orc.kv4_dequant(q)[:, 5] == 0)


def test_codes_monotone_in_x():
    x = random_rows(4, 500)
    q = orc.quantize_kv4(x)
    order = np.argsort(x.astype(np.float64), axis=1, kind="stable")
    sc = np.take_along_axis(q["codes"].astype(int), order, axis=1)
    assert np.all(np.diff(sc, axis=1) >= 0)


def test_sign_flip_mirrors_the_codes():
    """Negating a row swaps lo and hi: the scale is the same and code' = 15 - code
    wherever no tie or clamp intervenes."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, D))).astype(np.float16)
    x[:, 0] = np.abs(x).max(axis=1)                  # make the range symmetric: lo = -hi
    x[:, 1] = -x[:, 0]
    a, b = orc.quantize_kv4(x), orc.quantize_kv4(-x)
    assert np.array_equal(a["s"], b["s"])
    s = f16v(a["s"])
    t = np.abs(x.astype(np.float64) / s[:, None])
    clean = np.abs(t - np.floor(t) - 0.5) > 1e-3     # away from ties
    za, zb = a["z"].astype(int), b["z"].astype(int)
    # with lo = -hi the zero point is rint(hi/s) = rint(7.5 (1 + d)) for both signs
    assert np.array_equal(za, zb)
    ca = a["codes"].astype(int) - za[:, None]
    cb = b["codes"].astype(int) - zb[:, None]
    inner = clean & (a["codes"] > 0) & (a["codes"] < 15) & (b["codes"] > 0) & (b["codes"] < 15)
    assert np.array_equal(ca[inner], -cb[inner])


# --------------------------------------------------------------------------
# Decode attention
# --------------------------------------------------------------------------
def rand_cache(rng, B, Hkv, S):
    x = rng.standard_normal((B, Hkv, S, D)).astype(np.float16)
    return orc.quantize_kv4(x)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(6)
    k, v = rand_cache(rng, 2, 2, 8), rand_cache(rng, 2, 2, 8)
    q = rng.standard_normal((2, 2, D)).astype(np.float16)
    r = orc.kv4_attention(q, k, v, np.array([1, 1], np.int32), 0.088)
    vd = orc.kv4_dequant(v)
    assert np.array_equal(r["out"], vd[:, :, 0, :])
    assert np.array_equal(r["absout"], np.abs(vd[:, :, 0, :]))


def test_zero_query_gives_the_mean_value():
    rng = np.random.default_rng(7)
    k, v = rand_cache(rng, 1, 1, 40), rand_cache(rng, 1, 1, 40)
    q = np.zeros((1, 1, D), np.float16)
    L = 37
    r = orc.kv4_attention(q, k, v, np.array([L], np.int32), 0.088)
    vd = orc.kv4_dequant(v)[0, 0]
    for d in range(0, D, 9):
        exact = sum(Fraction(float(vd[t, d])) for t in range(L)) / L
        assert abs(Fraction(r["out"][0, 0, d]) - exact) <= Fraction(L, 2 ** 50) * max(1, abs(exact))


def two_token_case(a, kd0, kd1, sm):
    """q = a at channel 0; keys dequantize to kd0, kd1 at channel 0 and 0 elsewhere."""
    q = np.zeros((1, 1, D), np.float16)
    q[0, 0, 0] = a
    kc = np.full((1, 1, 2, D), 7, np.uint8)
    kc[0, 0, 0, 0] = 7 + kd0
    kc[0, 0, 1, 0] = 7 + kd1
    k = kv(kc, np.full((1, 1, 2), 0x3C00, np.uint16), np.full((1, 1, 2), 7, np.uint8))   # scale 1, zero 7
    return q, k


def test_two_tokens_follow_the_logistic_closed_form():
    rng = np.random.default_rng(8)
    v = rand_cache(rng, 1, 1, 2)
    vd = orc.kv4_dequant(v)[0, 0]
    for a, kd0, kd1, sm in [(1.5, 3, -2, 0.25), (-0.75, 8, 1, 0.088), (2.0, -7, 6, 1.0)]:
        q, k = two_token_case(a, kd0, kd1, sm)
        r = orc.kv4_attention(q, k, v, np.array([2], np.int32), sm)
        delta = sm * a * (kd0 - kd1)
        w0 = 1.0 / (1.0 + math.exp(-delta))
        want = w0 * vd[0] + (1 - w0) * vd[1]
        assert np.allclose(r["out"][0, 0], want, rtol=1e-13, atol=1e-13)
        assert r["score"][0, 0, 0] == sm * a * kd0 and r["score"][0, 0, 1] == sm * a * kd1
        assert r["absscore"][0, 0, 0] == abs(sm * a * kd0)


def test_a_large_gap_selects_one_token_exactly():
    """Scores 1000 apart: exp of the gap underflows to 0 in double, so the output is
    exactly that token's value (and a softmax without the max would overflow)."""
    rng = np.random.default_rng(9)
    v = rand_cache(rng, 1, 1, 2)
    q, k = two_token_case(100.0, 6, -6, 1.0)   # scores +600 and -600
    r = orc.kv4_attention(q, k, v, np.array([2], np.int32), 1.0)
    assert np.array_equal(r["out"][0, 0], orc.kv4_dequant(v)[0, 0, 0])


def test_tokens_past_the_length_do_not_matter():
    rng = np.random.default_rng(10)
    k, v = rand_cache(rng, 2, 1, 50), rand_cache(rng, 2, 1, 50)
    q = rng.standard_normal((2, 1, D)).astype(np.float16)
    lens = np.array([33, 50], np.int32)
    a = orc.kv4_attention(q, k, v, lens, 0.088)
    k2 = {n: t.copy() for n, t in k.items()}
    v2 = {n: t.copy() for n, t in v.items()}
    for t in (k2, v2):
        t["codes"][0, :, 33:] = 15 - t["codes"][0, :, 33:]
        t["s"][0, :, 33:] = 0x7BFF                  # 65504
        t["z"][0, :, 33:] = 0
    b = orc.kv4_attention(q, k2, v2, lens, 0.088)
    assert np.array_equal(a["out"][0], b["out"][0])
    # an empty sequence gives zeros
    c = orc.kv4_attention(q, k, v, np.array([0, 50], np.int32), 0.088)
    assert np.all(c["out"][0] == 0) and np.array_equal(c["out"][1], a["out"][1])


def test_token_order_does_not_matter():
    rng = np.random.default_rng(11)
    k, v = rand_cache(rng, 1, 2, 64), rand_cache(rng, 1, 2, 64)
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    perm = rng.permutation(64)
    a = orc.kv4_attention(q, k, v, np.array([64], np.int32), 0.088)
    kp = {"codes": k["codes"][:, :, perm], "s": k["s"][:, :, perm], "z": k["z"][:, :, perm]}
    vp = {"codes": v["codes"][:, :, perm], "s": v["s"][:, :, perm], "z": v["z"][:, :, perm]}
    b = orc.kv4_attention(q, kp, vp, np.array([64], np.int32), 0.088)
    assert np.allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)


def test_grouped_query_heads_share_consecutive_kv_heads():
    """Hq = 8 query heads on Hkv = 2 kv heads: heads 0-3 read kv head 0, heads 4-7 kv head 1."""
    rng = np.random.default_rng(12)
    k, v = rand_cache(rng, 1, 2, 4), rand_cache(rng, 1, 2, 4)
    q = rng.standard_normal((1, 8, D)).astype(np.float16)
    r = orc.kv4_attention(q, k, v, np.array([1], np.int32), 0.088)
    vd = orc.kv4_dequant(v)
    for h in range(8):
        assert np.array_equal(r["out"][0, h], vd[0, h // 4, 0])


def test_scale_of_query_and_softmax_scale_commute():
    rng = np.random.default_rng(13)
    k, v = rand_cache(rng, 1, 1, 30), rand_cache(rng, 1, 1, 30)
    q = rng.standard_normal((1, 1, D)).astype(np.float16)
    a = orc.kv4_attention(q, k, v, np.array([30], np.int32), 0.5)
    b = orc.kv4_attention((q.astype(np.float32) * 2).astype(np.float16), k, v, np.array([30], np.int32), 0.25)
    assert np.allclose(a["out"], b["out"], rtol=1e-14, atol=1e-14)
