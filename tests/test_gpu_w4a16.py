"""GPU parity of the W4A16 GEMM (gemm_w4a16) against the oracle, through the C ABI.

The GPU sums exact products x*r in fp32 in its own order, scales by s0 and
rounds to fp16; the oracle sums the same products in double.  The bound used
follows from that arithmetic: |y - ref| <= K 2^-24 absref (fp32 summation of
terms whose absolute sum is absref) + 2^-10 |ref| (the product with s0 and the
fp16 rounding) + 2^-24 (fp16 subnormal spacing).  One-hot activations make
every sum exact, and there the result is bit-exact: y = fp16(r s0), which pins
the operand layout k by k.
"""
import os

import numpy as np
import pytest

import oracle as orc
from gpu_helpers import dev, gpu_weights, say, to_dev, to_host
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


def ref_of(x, w):
    wq = orc.quantize_weights(w)
    r, bad = orc.dequant_i8(wq["q4"], wq["s1"], wq["z"])
    assert bad == 0
    return orc.gemm_w4a16(x, r, wq["s0"]), r, wq["s0"]


def check(y_bits, ref, absref, K, where):
    y = y_bits.view(np.float16).astype(np.float64)
    tol = K * 2.0 ** -24 * absref + 2.0 ** -10 * np.abs(ref) + 2.0 ** -24
    err = np.abs(y - ref)
    bad = err > tol
    assert not bad.any(), "%s: %d outputs outside the bound, worst excess %g" % (where, bad.sum(), (err - tol).max())


CASES = [(0, 16, 512, 512), (1, 1, 4096, 4096), (1, 8, 4096, 12288), (1, 32, 4096, 22016),
         (1, 16, 11008, 4096), (2, 5, 4096, 11008), (4, 1, 8192, 10240), (4, 17, 28672, 8192),
         (2, 12, 1024, 8208)]      # four tiles per workgroup with a one-tile tail


@pytest.mark.parametrize("family,M,K,N", CASES)
def test_w4a16_config_shapes(family, M, K, N):
    from w4a8_quantized_linear_amd import gemm_w4a16
    say("w4a16 family=%d M=%d K=%d N=%d" % (family, M, K, N))
    w = workloads.weights(family, K, N)
    x = workloads.activations(family, M, K, N)
    wq = gpu_weights(w)
    y = gemm_w4a16(to_dev(x), wq["wpacked"], wq["s0"], N)
    (ref, absref), _, _ = ref_of(x, w)
    check(to_host(y).view(np.uint16), ref, absref, K, "w4a16 M=%d K=%d N=%d" % (M, K, N))


def test_w4a16_one_hot_is_exact():
    """x = one-hot rows: the sum is one exact product, so y = fp16(r[n,k] s0[n])."""
    from w4a8_quantized_linear_amd import gemm_w4a16
    K, N = 256, 48
    w = workloads.weights(1, K, N)
    ks = [0, 1, 7, 8, 15, 16, 31, 63, 64, 72, 100, 127, 128, 200, 255]
    x = np.zeros((len(ks), K), np.float16)
    x[np.arange(len(ks)), ks] = 1.0
    say("w4a16 one-hot K=%d N=%d" % (K, N))
    wq = gpu_weights(w)
    y = to_host(gemm_w4a16(to_dev(x), wq["wpacked"], wq["s0"], N))
    (ref, _), r, s0 = ref_of(x, w)
    want = ref.astype(np.float16)          # ref = r * s0 exactly here; one rounding to fp16
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


def test_w4a16_stride_tails_and_determinism():
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a16
    K, N = 1152, 272                         # 9 groups (waves get 2 or 3), 17 tiles (a tail tile)
    w = workloads.weights(0, K, N)
    wide = workloads.activations(0, 21, 2048, N)
    t = to_dev(wide)[:, :K]
    assert t.stride(0) == 2048
    say("w4a16 ldx=2048 K=%d N=%d M=21" % (K, N))
    wq = gpu_weights(w)
    y1 = gemm_w4a16(t, wq["wpacked"], wq["s0"], N)
    y2 = gemm_w4a16(t, wq["wpacked"], wq["s0"], N)
    assert torch.equal(y1, y2)
    x = np.ascontiguousarray(wide[:, :K])
    (ref, absref), _, _ = ref_of(x, w)
    check(to_host(y1).view(np.uint16), ref, absref, K, "w4a16 strided")
    # K of one group (three of the four waves have nothing to add), M = 0
    w1 = workloads.weights(0, 128, 64)
    x1 = workloads.activations(0, 3, 128, 64)
    wq1 = gpu_weights(w1)
    y = gemm_w4a16(to_dev(x1), wq1["wpacked"], wq1["s0"], 64)
    (ref, absref), _, _ = ref_of(x1, w1)
    check(to_host(y).view(np.uint16), ref, absref, 128, "w4a16 K=128")
    gemm_w4a16(torch.empty((0, 128), dtype=torch.float16, device=dev()), wq1["wpacked"], wq1["s0"], 64)


@pytest.mark.parametrize("nt", ["1", "2", "4"])
def test_w4a16_two_token_tiles_match_one(nt):
    """Two 16-token tiles per workgroup (each rebuilt weight feeds two MFMAs)
    give the same bits as one: every token's sum is the same MFMA sequence.
    M = 37 leaves a partly filled second pair of tiles; N = 272 a tail tile."""
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a16
    K, N, M = 1152, 272, 37
    w = workloads.weights(2, K, N)
    x = workloads.activations(2, M, K, N)
    say("w4a16 MT=2 vs MT=1 NT=%s M=%d K=%d N=%d" % (nt, M, K, N))
    wq = gpu_weights(w)
    keys = ("W4A8_W16_NT", "W4A8_W16_MT")
    old = {k: os.environ.get(k) for k in keys}
    try:
        os.environ["W4A8_W16_NT"] = nt
        out = {}
        for mt in ("1", "2"):
            os.environ["W4A8_W16_MT"] = mt
            out[mt] = gemm_w4a16(to_dev(x), wq["wpacked"], wq["s0"], N)
        torch.cuda.synchronize()
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    assert torch.equal(out["1"], out["2"])
    (ref, absref), _, _ = ref_of(x, w)
    check(to_host(out["2"]).view(np.uint16), ref, absref, K, "w4a16 MT=2")
