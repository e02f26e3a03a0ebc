"""Pins of the oracle's W4A16 product (fp16 activations times the two-level
weights dequantized as r * s0, QFactory notes 2.1: w = (w_quant - zero) *
scale) against closed forms and exact rational arithmetic."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as orc


def f16(bits):
    return np.array(bits, np.uint16).view(np.float16).astype(np.float64)


def weights(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    wq = orc.quantize_weights(w)
    r, bad = orc.dequant_i8(wq["q4"], wq["s1"], wq["z"])
    assert bad == 0
    return r, wq["s0"]


def test_one_hot_rows_pick_one_dequantized_weight():
    N, K = 32, 256
    r, s0 = weights(N, K, 1)
    for k in (0, 37, 128, 255):
        x = np.zeros((2, K), np.float16)
        x[0, k] = 1.0
        x[1, k] = -0.25
        ref, absref = orc.gemm_w4a16(x, r, s0)
        want = r[:, k].astype(np.float64) * f16(s0)
        assert np.array_equal(ref[0], want) and np.array_equal(ref[1], -0.25 * want)
        assert np.array_equal(absref[0], np.abs(want))


def test_exact_rational_sum():
    N, K = 16, 128
    r, s0 = weights(N, K, 2)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((3, K)).astype(np.float16)
    ref, absref = orc.gemm_w4a16(x, r, s0)
    for m in range(3):
        for n in range(N):
            exact = sum(Fraction(float(x[m, k])) * int(r[n, k]) for k in range(K)) * Fraction(float(f16(s0[n])))
            aexact = sum(abs(Fraction(float(x[m, k])) * int(r[n, k])) for k in range(K)) * abs(Fraction(float(f16(s0[n]))))
            # K rounded double additions: relative error below K * 2^-53 of the absolute sum
            assert abs(Fraction(ref[m, n]) - exact) <= aexact * Fraction(K, 2 ** 53)
            assert abs(Fraction(absref[m, n]) - aexact) <= aexact * Fraction(K, 2 ** 53)


def test_small_integer_inputs_are_exact_and_linear():
    """Integer activations and a power-of-two scale: every partial sum is exact,
    so the product is linear in x exactly (catches index and transpose slips)."""
    N, K = 16, 256
    rng = np.random.default_rng(4)
    r = rng.integers(-127, 128, (N, K)).astype(np.int8)
    s0 = np.full(N, 0x1800, np.uint16)            # 2^-9
    x1 = rng.integers(-3, 4, (2, K)).astype(np.float16)
    x2 = rng.integers(-3, 4, (2, K)).astype(np.float16)
    a, _ = orc.gemm_w4a16(x1, r, s0)
    b, _ = orc.gemm_w4a16(x2, r, s0)
    c, _ = orc.gemm_w4a16((x1.astype(np.float32) + x2).astype(np.float16), r, s0)
    assert np.array_equal(a + b, c)
    want = x1.astype(np.int64) @ r.astype(np.int64).T * 2.0 ** -9
    assert np.array_equal(a, want)


@pytest.mark.parametrize("K", [128, 512])
def test_matches_the_w4a8_weights_in_double(K):
    """The dequantized weight is the W4A8 path's INT8 weight times s0: the
    product equals x @ (r * s0)^T computed by numpy in double."""
    N = 24
    r, s0 = weights(N, K, 5 + K)
    x = np.random.default_rng(6).standard_normal((4, K)).astype(np.float16)
    ref, absref = orc.gemm_w4a16(x, r, s0)
    w = r.astype(np.float64) * f16(s0)[:, None]
    want = x.astype(np.float64) @ w.T
    assert np.allclose(ref, want, rtol=0, atol=1e-12 * absref.max())
