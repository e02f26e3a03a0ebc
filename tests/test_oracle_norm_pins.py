"""Pins of the oracle's fused normalization + INT8 quantizer against things
other than itself: hand-worked examples (tests/golden/e5, e6), exact rational
arithmetic for the statistics, invariances the definition implies, and
special cases that reduce to the plain quantizer.

The step is the QServe talk summary's activation quantization fusion
("Precision Data Flow and Activation Quantization Fusion"): the layer before
a linear layer (LayerNorm there) writes the 8-bit activations directly.
"""
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

from conftest import load_golden
from oracle import oracle as orc


def f32_bits(v):
    return "0x%08x" % struct.unpack("<I", struct.pack("<f", np.float32(v)))[0]


def rows(seed, M, K, outliers=True):
    """fp16 rows with a spread of magnitudes (and a few large channels)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, size=(M, 1)))
    if outliers:
        x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 50
    return x.astype(np.float16)


def gam(K, seed=1):
    rng = np.random.default_rng(seed)
    return (1 + 0.1 * rng.standard_normal(K)).astype(np.float16)


def test_layernorm_worked_example():
    g = load_golden("e5_layernorm_token.json")
    out = orc.norm_quantize_act(np.array([g["x"]], np.float16), np.array(g["gamma"], np.float16),
                                np.array(g["beta"], np.float16), eps=g["eps"], rms=g["rms"])
    assert out["mean"][0] == g["mean"] and out["r"][0] == g["r"]
    assert out["h"][0].view(np.float16).astype(np.float64).tolist() == g["h"]
    assert f32_bits(out["s_a"][0]) == g["s_a_bits"]
    assert out["qx"][0].tolist() == g["qx"]


def test_rmsnorm_worked_example():
    g = load_golden("e6_rmsnorm_token.json")
    out = orc.norm_quantize_act(np.array([g["x"]], np.float16), np.array(g["gamma"], np.float16),
                                None, eps=g["eps"], rms=g["rms"])
    assert out["mean"][0] == g["mean"]
    assert f32_bits(np.float32(out["r"][0])) == g["rstd_bits"]
    assert ["0x%04x" % v for v in out["h"][0]] == g["h_bits"]
    assert f32_bits(out["s_a"][0]) == g["s_a_bits"]
    assert out["qx"][0].tolist() == g["qx"]


@pytest.mark.parametrize("K", [8, 96, 1000])
def test_mean_is_the_exact_mean_rounded_once(K):
    x = rows(10 + K, 6, K)
    out = orc.norm_quantize_act(x, gam(K), None, eps=1e-5, rms=False)
    for m in range(x.shape[0]):
        exact = sum(Fraction(float(v)) for v in x[m].astype(np.float64)) / K
        assert out["mean"][m] == float(exact)          # Fraction -> float rounds to nearest


@pytest.mark.parametrize("rms", [False, True])
@pytest.mark.parametrize("K", [8, 96, 1000])
def test_rstd_matches_exact_arithmetic(K, rms):
    getcontext().prec = 60
    x = rows(20 + K, 5, K)
    eps = 1e-5
    out = orc.norm_quantize_act(x, gam(K), None, eps=eps, rms=rms)
    for m in range(x.shape[0]):
        v = [Fraction(float(t)) for t in x[m].astype(np.float64)]
        mu = Fraction(0) if rms else Fraction(out["mean"][m])   # the double mean, as used
        var = sum((t - mu) ** 2 for t in v) / K
        ve = Decimal(var.numerator) / Decimal(var.denominator) + Decimal(float(np.float32(eps)))
        exact = 1 / ve.sqrt()
        got = Decimal(float(out["r"][m]))
        # rounded double sum of K non-negative terms: relative error below K * 2^-52
        assert abs(got - exact) <= exact * Decimal(K) * Decimal(2) ** -50


@pytest.mark.parametrize("rms", [False, True])
def test_scale_by_power_of_two_leaves_everything_unchanged(rms):
    x = rows(3, 8, 256, outliers=False) * np.float16(0.25)
    g = gam(256)
    a = orc.norm_quantize_act(x, g, None, eps=0.0, rms=rms)
    b = orc.norm_quantize_act((x.astype(np.float32) * 8).astype(np.float16), g, None, eps=0.0, rms=rms)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["qx"], b["qx"])
    assert np.array_equal(a["s_a"], b["s_a"])


def test_layernorm_ignores_an_exact_shift():
    rng = np.random.default_rng(4)
    x = rng.integers(-40, 40, size=(6, 128)).astype(np.float16)      # integers: x + 7 is exact
    g = gam(128)
    a = orc.norm_quantize_act(x, g, None, eps=1e-3, rms=False)
    b = orc.norm_quantize_act(x + np.float16(7), g, None, eps=1e-3, rms=False)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["qx"], b["qx"])
    assert np.array_equal(a["r"], b["r"])


def test_rmsnorm_of_unit_rows_is_the_plain_quantizer():
    rng = np.random.default_rng(5)
    x = rng.choice(np.array([-1.0, 1.0], np.float16), size=(7, 384))
    out = orc.norm_quantize_act(x, np.ones(384, np.float16), None, eps=0.0, rms=True)
    assert np.all(out["r"] == 1.0)
    assert np.array_equal(out["h"].view(np.float16), x)
    qx, sa = orc.quantize_act(x)
    assert np.array_equal(out["qx"], qx) and np.array_equal(out["s_a"], sa)


@pytest.mark.parametrize("rms", [False, True])
def test_one_hot_gamma_selects_one_feature(rms):
    K, j = 64, 37
    x = rows(6, 3, K, outliers=False)
    g = np.zeros(K, np.float16)
    g[j] = 1
    out = orc.norm_quantize_act(x, g, None, eps=1e-4, rms=rms)
    h = out["h"].view(np.float16).astype(np.float32)
    assert np.all(h[:, np.arange(K) != j] == 0)
    mu32 = out["mean"].astype(np.float32)
    rstd = out["r"].astype(np.float32)
    want = ((x[:, j].astype(np.float32) - mu32) * rstd).astype(np.float16)
    assert np.array_equal(h[:, j].astype(np.float16), want)


def test_beta_alone():
    K = 40
    x = rows(7, 2, K)
    out = orc.norm_quantize_act(x, np.zeros(K, np.float16), np.full(K, -0.75, np.float16), eps=1e-5)
    assert np.all(out["h"].view(np.float16) == np.float16(-0.75))
    assert np.all(out["qx"] == -127)
    assert np.all(out["s_a"] == np.float32(0.75) / np.float32(127))


def test_zero_rows():
    K = 32
    x = np.zeros((2, K), np.float16)
    out = orc.norm_quantize_act(x, np.ones(K, np.float16), None, eps=1e-5, rms=False)
    assert np.all(out["qx"] == 0) and np.all(out["s_a"] == 0) and np.all(out["h"] == 0)
    # eps = 0: var + eps = 0, the scale factor is taken as 0 and only beta is left
    out = orc.norm_quantize_act(x, np.ones(K, np.float16), np.full(K, 2.0, np.float16), eps=0.0, rms=True)
    assert np.all(np.isinf(out["r"])) and np.all(out["qx"] == 127)
    assert np.all(out["s_a"] == np.float32(2.0) / np.float32(127))


def test_near_midpoint_flag():
    f = np.float32(0.3)
    nxt = np.nextafter(f, np.float32(1))
    mid = (float(f) + float(nxt)) / 2
    flags = orc.rstd_near_midpoint(np.array([mid, float(f), np.inf, mid * (1 + 2.0 ** -30)]))
    assert flags.tolist() == [True, False, False, False]
