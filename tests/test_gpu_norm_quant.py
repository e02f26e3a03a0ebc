"""GPU parity of the fused normalization + per-token INT8 quantizer
(norm_quantize_act_i8) against the oracle, through the C ABI.

qx and s_a are compared bit for bit.  The one order-dependent step is the
double sum of squares: a token whose double 1/sqrt lies within 2^-36
(relative) of a midpoint between two floats may round to the other float in
another order, so the oracle flags those tokens (a few per ten thousand) and
they are checked to be valid instead: s_a within one part in a million and
every code within one step.
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import dev, say, to_dev, to_host
from w4a8_quantized_linear_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a8_quantized_linear_amd import _lib
    _lib.load()           # raises if the HIP library is not built: no fallback
    yield


def gamma_beta(K, seed):
    rng = np.random.default_rng(seed)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    b = (0.05 * rng.standard_normal(K)).astype(np.float16)
    return g, b


def check(x, g, b, eps, rms, where, x_dev=None):
    from w4a8_quantized_linear_amd import norm_quantize_act_i8
    say(where)
    xt = to_dev(x) if x_dev is None else x_dev
    qx, sa = norm_quantize_act_i8(xt, to_dev(g), None if b is None else to_dev(b), eps=eps, rms=rms)
    qx, sa = to_host(qx), to_host(sa)
    ref = orc.norm_quantize_act(np.ascontiguousarray(x), g, b, eps=eps, rms=rms)
    flag = orc.rstd_near_midpoint(ref["r"])
    ok = ~flag
    bad_s = np.nonzero(ok & (sa.view(np.uint32) != ref["s_a"].view(np.uint32)))[0]
    assert bad_s.size == 0, "%s: s_a differs at tokens %s" % (where, bad_s[:8])
    bad_q = np.nonzero(ok & np.any(qx != ref["qx"], axis=1))[0]
    assert bad_q.size == 0, "%s: qx differs at tokens %s" % (where, bad_q[:8])
    if flag.any():
        rel = np.abs(sa[flag].astype(np.float64) - ref["s_a"][flag]) / np.maximum(ref["s_a"][flag], 1e-30)
        assert np.all(rel <= 1e-6), where
        assert np.all(np.abs(qx[flag].astype(np.int32) - ref["qx"][flag]) <= 1), where
    assert flag.mean() < 0.01, "%s: %d of %d tokens flagged" % (where, flag.sum(), flag.size)
    return qx, sa


CASES = [(0, 16, 512, 512), (1, 1, 4096, 4096), (1, 32, 11008, 4096), (2, 256, 4096, 11008),
         (3, 4096, 4096, 11008), (3, 4096, 11008, 4096), (4, 512, 8192, 10240), (4, 64, 28672, 8192)]


@pytest.mark.parametrize("rms", [False, True], ids=["layernorm", "rmsnorm"])
@pytest.mark.parametrize("family,M,K,N", CASES)
def test_norm_quant_config_shapes(family, M, K, N, rms):
    x = workloads.activations(family, M, K, N)
    g, b = gamma_beta(K, K + M)
    check(x, g, None if rms else b, 1e-5, rms, "norm quant %s family=%d M=%d K=%d"
          % ("rms" if rms else "layer", family, M, K))


@pytest.mark.parametrize("rms", [False, True], ids=["layernorm", "rmsnorm"])
@pytest.mark.parametrize("M,K", [(3, 128), (5, 40960), (8, 65536), (1100, 1152), (2000, 8320)])
def test_norm_quant_ragged_and_long_rows(M, K, rms):
    """Rows shorter than a wave's chunks, rows that fill the registers only
    partly, rows longer than the registers (re-read from cache), and both
    the four-waves-per-token and one-wave-per-token layouts."""
    rng = np.random.default_rng(M * 7 + K)
    x = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-2, 2, (M, 1)))).astype(np.float16)
    g, b = gamma_beta(K, K)
    check(x, g, b, 1e-6, rms, "norm quant ragged M=%d K=%d rms=%d" % (M, K, rms))


def test_norm_quant_edges_stride_and_determinism():
    import torch
    from w4a8_quantized_linear_amd import norm_quantize_act_i8
    K = 256
    x = np.zeros((9, K), np.float16)
    x[1, 7] = -3.0                                   # single non-zero
    x[2] = np.float16(0.75)                          # constant row: variance 0
    x[3, :4] = [1, 3, 1, 3]                          # the worked example's row
    x[4] = np.float16(60000.0)
    x[4, ::3] = np.float16(-60000.0)                 # large values
    x[5, ::2] = np.float16(2.0 ** -24)               # subnormals
    x[6] = np.arange(K, dtype=np.float16)
    x[7] = np.float16(1.0)
    x[7, ::2] = np.float16(-1.0)
    g, b = gamma_beta(K, 3)
    for rms in (False, True):
        check(x, g, b, 1e-5, rms, "norm quant edges rms=%d" % rms)
        check(x, g, None, 0.0, rms, "norm quant edges eps=0 rms=%d" % rms)   # zero rows: rstd 0
    # row stride larger than K
    wide = workloads.activations(0, 16, 1024, 512)
    t = to_dev(wide)[:, :512]
    assert t.stride(0) == 1024
    g2, b2 = gamma_beta(512, 5)
    check(np.ascontiguousarray(wide[:, :512]), g2, b2, 1e-5, False, "norm quant ldx=1024", x_dev=t)
    # M = 0 is a no-op; repeated calls are bit-identical
    norm_quantize_act_i8(torch.empty((0, 128), dtype=torch.float16, device=dev()),
                         to_dev(np.ones(128, np.float16)))
    x3 = workloads.activations(3, 777, 4096, 11008)
    g3, b3 = gamma_beta(4096, 9)
    a = [norm_quantize_act_i8(to_dev(x3), to_dev(g3), to_dev(b3)) for _ in range(2)]
    assert torch.equal(a[0][0], a[1][0]) and torch.equal(a[0][1], a[1][1])


def test_norm_quant_feeds_the_gemm():
    """The fused producer's outputs are the GEMM's inputs: the INT32
    accumulators of gemm_w4a8 on them match the oracle's contraction."""
    import torch
    from gpu_helpers import gpu_weights
    from w4a8_quantized_linear_amd import gemm_w4a8, norm_quantize_act_i8
    M, K, N = 64, 4096, 4096
    x = workloads.activations(1, M, K, N)
    w = workloads.weights(1, K, N)
    g, b = gamma_beta(K, 11)
    say("norm quant -> gemm M=%d K=%d N=%d" % (M, K, N))
    qx, sa = norm_quantize_act_i8(to_dev(x), to_dev(g), to_dev(b))
    wq = gpu_weights(w)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev())
    gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
    ref = orc.norm_quantize_act(x, g, b, eps=1e-5)
    keep = ~orc.rstd_near_midpoint(ref["r"])
    wref = orc.quantize_weights(w)
    r, bad = orc.dequant_i8(wref["q4"], wref["s1"], wref["z"])
    assert bad == 0
    acc_ref, _ = orc.gemm_acc(ref["qx"], r)
    assert np.array_equal(to_host(acc)[keep], acc_ref[keep])
