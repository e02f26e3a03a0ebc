"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact on every integer result (qx, s_a, s0, s1, z, the packed codes read
back through w4a8_unpack_weights, and the INT32 accumulators of the real GEMM
main loop); the fp16 outputs within |dy| <= 1e-2 + 1e-3 |y_ref|.  Every
case, the full workload sizes included, is compared element by element: all
M x N GEMM outputs, every channel of the quantized weights.
"""
import os

import numpy as np
import pytest

import oracle as orc
from gpu_helpers import (assert_y_close, case_inputs, dev, f16_bits, gpu_weights,
                         oracle_weights_rows, say, to_dev, to_host)
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


KN_ALL = sorted({(K, N) for fam in workloads.FAMILIES for (K, N) in fam.kns})
FAMILY_OF = {}
for fam in workloads.FAMILIES:
    for kn in fam.kns:
        FAMILY_OF.setdefault(kn, fam.index)


# ---------------------------------------------------------------------------
# activation quantizer
# ---------------------------------------------------------------------------
ACT_CASES = [(0, 16, 512, 512), (1, 1, 4096, 4096), (1, 8, 4096, 12288), (1, 32, 11008, 4096),
             (2, 256, 4096, 11008), (3, 4096, 4096, 11008), (3, 4096, 11008, 4096),
             (4, 512, 28672, 8192), (4, 64, 8192, 57344)]


@pytest.mark.parametrize("family,M,K,N", ACT_CASES)
def test_act_quant_bit_exact(family, M, K, N):
    from w4a8_quantized_linear_amd import quantize_act_per_token_i8
    say("act quant family=%d M=%d K=%d" % (family, M, K))
    x = workloads.activations(family, M, K, N)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    qx_ref, sa_ref = orc.quantize_act(x)
    assert np.array_equal(to_host(qx), qx_ref)
    assert np.array_equal(to_host(sa).view(np.uint32), sa_ref.view(np.uint32))


def test_act_quant_edges_and_row_stride():
    import torch
    from w4a8_quantized_linear_amd import quantize_act_per_token_i8
    K = 256
    x = np.zeros((6, K), np.float16)
    x[1, 7] = -3.0                                   # single non-zero
    x[2, :5] = [3, -1.5, 0.75, -0.375, 1]            # worked-example token (ties)
    x[3, :8] = [127, -63.5, 31.25, 0.5, -0.5, 1.5, -127, 2.5]
    x[4] = np.float16(65504.0)                       # largest fp16
    x[5, ::2] = np.float16(2.0 ** -24)               # smallest subnormal
    say("act quant edges")
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    qx_ref, sa_ref = orc.quantize_act(x)
    assert np.array_equal(to_host(qx), qx_ref)
    assert np.array_equal(to_host(sa).view(np.uint32), sa_ref.view(np.uint32))
    # row stride larger than K: quantize the left 512 columns of a 1024-wide buffer
    wide = workloads.activations(0, 16, 1024, 512)
    t = to_dev(wide)[:, :512]
    assert t.stride(0) == 1024
    qx2, sa2 = quantize_act_per_token_i8(t)
    qx2_ref, sa2_ref = orc.quantize_act(np.ascontiguousarray(wide[:, :512]))
    assert np.array_equal(to_host(qx2), qx2_ref)
    assert np.array_equal(to_host(sa2).view(np.uint32), sa2_ref.view(np.uint32))
    # M = 0 is a no-op
    e = torch.empty((0, 128), dtype=torch.float16, device=dev())
    quantize_act_per_token_i8(e)


@pytest.mark.parametrize("waves", ["1", "4"])
@pytest.mark.parametrize("M,K", [(2048, 4096), (1100, 11008), (4096, 1152)])
def test_act_quant_both_layouts(waves, M, K):
    """The two register layouts of the quantizer -- one wave per token (rows
    held by one wave, tokens walked with a row prefetch) and four waves per
    token -- forced in turn, on rows with outlier channels, exact ties and a
    zero row, bit-exact against the oracle."""
    from w4a8_quantized_linear_amd import quantize_act_per_token_i8
    say("act quant layout waves=%s M=%d K=%d" % (waves, M, K))
    x = workloads.activations(1, M, K, 4096)
    x[3] = 0
    x[5, :8] = [127, -63.5, 31.25, 0.5, -0.5, 1.5, -127, 2.5]
    x[5, 8:] = 0
    old = os.environ.get("W4A8_ACT_WAVES")
    os.environ["W4A8_ACT_WAVES"] = waves
    try:
        qx, sa = quantize_act_per_token_i8(to_dev(x))
        qx_h, sa_h = to_host(qx), to_host(sa)
    finally:
        if old is None:
            os.environ.pop("W4A8_ACT_WAVES", None)
        else:
            os.environ["W4A8_ACT_WAVES"] = old
    qx_ref, sa_ref = orc.quantize_act(x)
    assert np.array_equal(sa_h.view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(qx_h, qx_ref)


@pytest.mark.parametrize("M", [64, 1100])
def test_act_quant_every_half_value(M):
    """Each row holds every finite fp16 value up to its absmax (the rest 0),
    under scales that make exact ties (absmax 127, 63.5, 254: s_a = 1, 0.5, 2)
    and random ones: every quotient the division can meet for that scale,
    including those within rounding distance of a half-integer.  M spans the
    launch shapes of the four-waves-per-token layout the row length needs."""
    from w4a8_quantized_linear_amd import quantize_act_per_token_i8
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    vals = vals[np.isfinite(vals)]
    K = vals.size                                    # 63488 = 496 groups of 128
    assert K % 128 == 0
    rng = np.random.default_rng(20261202 + M)
    amax = rng.uniform(-24, 15.99, size=M)
    amax = np.exp2(amax).astype(np.float16)
    amax[:6] = [127, 63.5, 254, 65504, 2.0 ** -24, 1]
    x = np.where(np.abs(vals)[None, :] <= amax[:, None], vals[None, :], np.float16(0))
    x = np.ascontiguousarray(x.astype(np.float16))
    say("act quant every fp16 value M=%d K=%d" % (M, K))
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    qx_ref, sa_ref = orc.quantize_act(x)
    assert np.array_equal(to_host(sa).view(np.uint32), sa_ref.view(np.uint32))
    assert np.array_equal(to_host(qx), qx_ref)


# ---------------------------------------------------------------------------
# weight quantizer + packing (read back through the unpack entry point)
# ---------------------------------------------------------------------------
def _check_weights(w, wq, rows, where):
    from w4a8_quantized_linear_amd import w4a8_unpack_weights
    import torch
    N, K = w.shape
    ref = oracle_weights_rows(w, rows)
    q4c, s1u, zu = w4a8_unpack_weights(wq["wpacked"], N, K)
    idx = torch.from_numpy(rows).to(dev())
    assert np.array_equal(f16_bits(wq["s0"][idx]), ref["s0"]), where + " s0"
    assert np.array_equal(to_host(wq["s1"][idx]), ref["s1"]), where + " s1"
    assert np.array_equal(to_host(wq["z"][idx]), ref["z"]), where + " z"
    assert np.array_equal(to_host(s1u[idx]), ref["s1"]), where + " unpacked s1"
    assert np.array_equal(to_host(zu[idx]), ref["z"]), where + " unpacked z"
    assert np.array_equal(to_host(q4c[idx]), orc.pack_q4(ref["q4"])), where + " codes"


@pytest.mark.parametrize("K,N", KN_ALL)
def test_weight_quant_bit_exact(K, N):
    import torch
    fam = FAMILY_OF[(K, N)]
    say("weight quant family=%d K=%d N=%d" % (fam, K, N))
    w = workloads.weights(fam, K, N)
    wq = gpu_weights(w)
    _check_weights(w, wq, np.arange(N), "K=%d N=%d" % (K, N))
    del wq
    torch.cuda.empty_cache()


def test_weight_quant_edges():
    say("weight quant edges")
    K = 384                                          # three groups (odd group count)
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((48, K)) * 0.02).astype(np.float32)
    w[0] = 0                                         # zero channel
    w[1] = np.abs(w[1])                              # one-signed channels
    w[2] = -np.abs(w[2])
    w[3, :128] = (np.arange(128) - 119) * 2.0 ** -10  # worked example row (group 0)
    w[4] *= 0.05                                     # subnormal fp16 channel scale
    w[5, 128:256] = 0                                # an all-zero group
    w[6] = 0
    w[6, 200] = 1.0                                  # a single non-zero weight
    wq = gpu_weights(w)
    _check_weights(w, wq, np.arange(48), "edges")


# ---------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------
def _gemm_case(family, M, K, N, wq=None, w=None):
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a8, quantize_act_per_token_i8
    say("gemm family=%d M=%d K=%d N=%d" % (family, M, K, N))
    if w is None:
        w = workloads.weights(family, K, N)
    x = workloads.activations(family, M, K, N)
    if wq is None:
        wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    acc = torch.empty((M, N), dtype=torch.int32, device=dev())
    y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
    torch.cuda.synchronize()
    # oracle: every token row against every channel
    out = orc.linear(x, orc.quantize_weights(w))
    acc_g = to_host(acc)
    assert np.array_equal(acc_g, out["acc"]), "INT32 accumulators differ (%d of %d)" % (
        (acc_g != out["acc"]).sum(), acc_g.size)
    assert_y_close(f16_bits(y), out["y"], "M=%d K=%d N=%d" % (M, K, N))
    return y, acc


def test_gemm_tiny_family0():
    _gemm_case(0, 16, 512, 512)


@pytest.mark.parametrize("M", [1, 8, 32])
@pytest.mark.parametrize("K,N", workloads.FAMILIES[1].kns)
def test_gemm_7b_decode(M, K, N):
    _gemm_case(1, M, K, N)


def test_gemm_batched_decode_m256():
    _gemm_case(2, 256, 4096, 11008)


@pytest.mark.parametrize("K,N", workloads.FAMILIES[3].kns)
def test_gemm_prefill_m4096(K, N):
    _gemm_case(3, 4096, K, N)


@pytest.mark.parametrize("K,N", workloads.FAMILIES[4].kns)
def test_gemm_70b_layers(K, N):
    import torch
    w = workloads.weights(4, K, N)
    wq = gpu_weights(w)
    for M in workloads.FAMILIES[4].ms:
        _gemm_case(4, M, K, N, wq=wq, w=w)
    del wq
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M,K,N,tm,ranges", [
    (768, 11008, 4096, 8, 192),     # TM 4 tiles fill the CUs: TM 8, each of 96 tiles in two ranges
    (384, 11008, 4096, 4, 192),     # 96 TM 4 tiles, two ranges each
    (160, 8192, 10240, 4, 240),     # 120 TM 4 tiles (the last m-block ragged), two ranges each
])
def test_gemm_prefill_split_tiles_full(M, K, N, tm, ranges):
    """The default plans of long-K layers whose tiles fit one round split
    every tile into equal K ranges (no range straddles two tiles); compared
    in full."""
    from w4a8_quantized_linear_amd import gemm_w4a8_plan
    p = gemm_w4a8_plan(M, N, K)
    assert p["kind"] == 1 and p["mt"] == tm and p["splitk"] == ranges and p["ws_bytes"] > 0, p
    _gemm_case(3, M, K, N)


def test_gemm_without_workspace_long_k():
    """ws == NULL at K = 28672, N = 8192, M = 64 (the 70B down projection):
    the default plan splits K over an N-split kernel whose unsplit LDS would
    not fit, so the call takes a launchable unsplit plan; compared in full
    against the oracle and against the split call."""
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a8, gemm_w4a8_plan_detail, quantize_act_per_token_i8
    M, K, N = 64, 28672, 8192
    d = gemm_w4a8_plan_detail(M, N, K, False)
    assert d["ws_bytes"] == 0 and d["lds_bytes"] <= 128 * 1024, d
    say("gemm ws=NULL M=%d K=%d N=%d plan %s" % (M, K, N, d))
    w = workloads.weights(4, K, N)
    x = workloads.activations(4, M, K, N)
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    acc0 = torch.empty((M, N), dtype=torch.int32, device=dev())
    acc1 = torch.empty((M, N), dtype=torch.int32, device=dev())
    y0 = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc0, use_workspace=False)
    y1 = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc1)
    torch.cuda.synchronize()
    out = orc.linear(x, orc.quantize_weights(w))
    assert np.array_equal(to_host(acc0), out["acc"])
    assert_y_close(f16_bits(y0), out["y"], "ws=NULL")
    assert np.array_equal(to_host(acc1), out["acc"])
    assert np.array_equal(f16_bits(y0), f16_bits(y1))


EDGE = [(1, 128, 16), (5, 128, 48), (17, 384, 48), (33, 256, 80), (63, 640, 32), (65, 384, 16),
        (100, 512, 144), (16, 384, 4096)]


@pytest.mark.parametrize("M,K,N", EDGE)
def test_gemm_edge_shapes(M, K, N):
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a8, quantize_act_per_token_i8
    say("gemm edge M=%d K=%d N=%d" % (M, K, N))
    rng = np.random.default_rng(M * 1000 + K + N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    x[M // 2] = 0                                      # an all-zero token
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    acc = torch.empty((M, N), dtype=torch.int32, device=dev())
    y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
    out = orc.linear(x, orc.quantize_weights(w))
    assert np.array_equal(to_host(acc), out["acc"])
    assert_y_close(f16_bits(y), out["y"], "edge")
    assert not to_host(acc)[M // 2].any()


def _with_plan(plan, fn):
    old = os.environ.get("W4A8_DECODE_PLAN")
    os.environ["W4A8_DECODE_PLAN"] = plan
    try:
        return fn()
    finally:
        if old is None:
            del os.environ["W4A8_DECODE_PLAN"]
        else:
            os.environ["W4A8_DECODE_PLAN"] = old


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_splitk_equals_no_splitk_and_is_deterministic(M):
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, quantize_act_per_token_i8
    K, N = 4096, 4096
    say("split-k equality M=%d" % M)
    w = workloads.weights(1, K, N)
    x = workloads.activations(1, M, K, N)
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    mt = 1 if M <= 16 else (2 if M <= 32 else 4)
    results = []
    plans = ["%d,2,1" % mt, "%d,2,4" % mt, "%d,1,16" % mt, "%d,4,3" % mt, "%d,2,4" % mt,
             "%d,1,1,8,2" % mt, "%d,1,2,4,2" % mt]
    if mt == 1:
        plans += ["1,1,1,4,4,1", "1,2,1,4,2,1", "1,1,3,8,2,1", "1,2,2,4,4,1", "1,1,1,4,4,0"]
    for plan in plans:
        def run():
            acc = torch.empty((M, N), dtype=torch.int32, device=dev())
            y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
            torch.cuda.synchronize()
            return f16_bits(y), to_host(acc)
        results.append(_with_plan(plan, run))
    for y, acc in results[1:]:
        assert np.array_equal(acc, results[0][1])
        assert np.array_equal(y, results[0][0])
    # the workspace's counters are left zeroed (the partial slots are scratch)
    ws = _lib._ws_cache.get(torch.device(dev()))
    if ws is not None:
        assert int(ws[:65536].count_nonzero()) == 0


def test_workspace_reuse_with_smaller_second_call():
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, quantize_act_per_token_i8
    K, N = 4096, 4096
    w = workloads.weights(1, K, N)
    wq = gpu_weights(w)
    ref_w = orc.quantize_weights(w)
    for M in (32, 1, 8):
        say("workspace reuse M=%d" % M)
        x = workloads.activations(1, M, K, N)
        qx, sa = quantize_act_per_token_i8(to_dev(x))
        acc = torch.empty((M, N), dtype=torch.int32, device=dev())
        gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
        out = orc.linear(x, ref_w)
        assert np.array_equal(to_host(acc), out["acc"])
    ws = _lib._ws_cache.get(torch.device(dev()))
    assert ws is None or int(ws[:65536].count_nonzero()) == 0


@pytest.mark.parametrize("plan", ["1,2,1", "1,4,2", "2,4,1", "4,2,3", "1,2,1,4,4,1", "1,2,2,8,2,1"])
def test_gemm_n_tail_tiles(plan):
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a8, quantize_act_per_token_i8
    M, K, N = 20, 768, 48          # 3 n-tiles: the last workgroup's tile group is partial
    say("gemm n-tail plan=%s" % plan)
    rng = np.random.default_rng(99)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    acc = torch.zeros((M, N), dtype=torch.int32, device=dev())

    def run():
        y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
        torch.cuda.synchronize()
        return y
    y = _with_plan(plan, run)
    out = orc.linear(x, orc.quantize_weights(w))
    assert np.array_equal(to_host(acc), out["acc"])
    assert_y_close(f16_bits(y), out["y"], "n-tail")


def _with_env(name, value, fn):
    old = os.environ.get(name)
    os.environ[name] = value
    try:
        return fn()
    finally:
        if old is None:
            del os.environ[name]
        else:
            os.environ[name] = old


# Shapes for the many-token kernel (16 TM x 256 workgroup tiles, TM in
# {4, 8, 16}; weight rings of 4 or 6 groups, unrolled by 4 or 12): ragged M
# and N tails, K with a group count below, at and past the ring depth and the
# unroll and not a multiple of them, and enough m-blocks to fill more than
# one band of four.
@pytest.mark.parametrize("tm", ["4", "8", "16"])
@pytest.mark.parametrize("M,K,N", [(300, 384, 272), (17, 256, 48), (512, 1024, 512),
                                   (1100, 640, 304), (257, 1152, 1040), (90, 1664, 256)])
def test_prefill_ragged(tm, M, K, N):
    import torch
    from w4a8_quantized_linear_amd import gemm_w4a8, quantize_act_per_token_i8
    say("prefill TM=%s M=%d K=%d N=%d" % (tm, M, K, N))
    rng = np.random.default_rng(M + 7 * K + 13 * N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    x[M // 3] = 0
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    acc = torch.zeros((M, N), dtype=torch.int32, device=dev())

    def run():
        y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
        torch.cuda.synchronize()
        return y
    y = _with_env("W4A8_PREFILL_TM", tm, run)
    out = orc.linear(x, orc.quantize_weights(w))
    assert np.array_equal(to_host(acc), out["acc"])
    assert_y_close(f16_bits(y), out["y"], "prefill")


# Stream-K: (tile, group) units split into P ranges, tiles finished by their
# last contributor.  P from 1 (one workgroup does everything) to more ranges
# than groups per tile (every tile split many ways); results are bit-exact
# and deterministic, and the workspace counters are left at zero.
@pytest.mark.parametrize("tm", ["4", "8"])
@pytest.mark.parametrize("P", ["1", "5", "37", "256"])
@pytest.mark.parametrize("M,K,N", [(300, 384, 272), (1100, 640, 304), (257, 1152, 1040)])
def test_prefill_stream_k(tm, P, M, K, N):
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, quantize_act_per_token_i8
    say("prefill stream-K TM=%s P=%s M=%d K=%d N=%d" % (tm, P, M, K, N))
    rng = np.random.default_rng(3 * M + 5 * K + N)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    out = orc.linear(x, orc.quantize_weights(w))
    old = {k: os.environ.get(k) for k in ("W4A8_PREFILL_TM", "W4A8_PREFILL_P")}
    os.environ["W4A8_PREFILL_TM"] = tm
    os.environ["W4A8_PREFILL_P"] = P
    try:
        need = _lib.gemm_w4a8_workspace_bytes(M, N, K)
        assert need > 0
        ws = torch.zeros(need, dtype=torch.uint8, device=dev())
        accs = []
        for rep in range(2):
            acc = torch.full((M, N), 7, dtype=torch.int32, device=dev())
            y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc, ws=ws)
            torch.cuda.synchronize()
            accs.append(to_host(acc))
            assert np.array_equal(accs[-1], out["acc"]), "rep %d" % rep
            assert_y_close(f16_bits(y), out["y"], "stream-K")
        assert int(to_host(ws[:65536]).astype(np.int64).sum()) == 0, "counters not reset"
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def test_workspace_shared_across_shapes_and_kernels():
    """One workspace buffer serves calls of different shapes and both split
    kernels in turn (stream-K prefill, split-K decode): the partial slots are
    scratch, only the counters must stay zero, and every call is bit-exact."""
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, quantize_act_per_token_i8
    cases = [  # (M, K, N, env)
        (1100, 640, 304, {"W4A8_PREFILL_TM": "4", "W4A8_PREFILL_P": "37"}),
        (300, 1024, 2048, {"W4A8_PREFILL_TM": "8", "W4A8_PREFILL_P": "200"}),
        (24, 1024, 2048, {"W4A8_DECODE_PLAN": "2,1,3"}),
        (257, 1152, 1040, {"W4A8_PREFILL_TM": "8", "W4A8_PREFILL_P": "64"}),
        (9, 1024, 512, {"W4A8_DECODE_PLAN": "1,2,4"}),
        (1100, 640, 304, {"W4A8_PREFILL_TM": "4", "W4A8_PREFILL_P": "37"}),
    ]
    keys = ("W4A8_PREFILL_TM", "W4A8_PREFILL_P", "W4A8_DECODE_PLAN")
    saved = {k: os.environ.get(k) for k in keys}
    ws = None
    try:
        for (M, K, N, env) in cases:
            say("shared workspace M=%d K=%d N=%d %s" % (M, K, N, env))
            for k in keys:
                os.environ.pop(k, None)
            os.environ.update(env)
            need = _lib.gemm_w4a8_workspace_bytes(M, N, K)
            assert need > 0, env
            if ws is None or ws.numel() < need:
                old_ws = ws
                ws = torch.zeros(max(need, 64 << 20), dtype=torch.uint8, device=dev())
                if old_ws is not None:   # carry the scratch over: it must not matter
                    ws[:old_ws.numel()] = old_ws
            rng = np.random.default_rng(M + K + N)
            w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
            x = rng.standard_normal((M, K)).astype(np.float16)
            wq = gpu_weights(w)
            qx, sa = quantize_act_per_token_i8(to_dev(x))
            acc = torch.empty((M, N), dtype=torch.int32, device=dev())
            y = gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc, ws=ws)
            torch.cuda.synchronize()
            out = orc.linear(x, orc.quantize_weights(w))
            assert np.array_equal(to_host(acc), out["acc"]), env
            assert_y_close(f16_bits(y), out["y"], "shared workspace")
            assert int(to_host(ws[:65536]).astype(np.int64).sum()) == 0, "counters not reset"
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("M,K,N", [(96, 4096, 11008), (128, 11008, 4096), (113, 8192, 10240),
                                   (256, 11008, 4096), (200, 8192, 2048), (137, 4096, 4096), (160, 4096, 768),
                                   (232, 4096, 4096), (160, 28672, 2048), (200, 28672, 2048), (160, 8192, 6144),
                                   (252, 24192, 1152), (80, 4096, 1536), (100, 8192, 768), (128, 2048, 2048),
                                   (128, 11008, 8448), (229, 2176, 5376), (131, 2048, 12544), (384, 8192, 2048),
                                   (512, 4096, 1024), (449, 6144, 2048), (1024, 4096, 1024), (700, 2048, 1024),
                                   (448, 28672, 2048)])
def test_gemm_mid_m_takes_the_decode_kernels(M, K, N):
    """65..128 tokens on layers whose 64 x 256 prefill tiles would leave more
    than half of the CUs idle, and 129..1024 tokens on layers with at most
    2^20 outputs (2^21 for small weights), run on the decode kernels; every
    row compared."""
    from w4a8_quantized_linear_amd import gemm_w4a8_plan
    assert gemm_w4a8_plan(M, N, K)["kind"] == 0
    _gemm_case(4, M, K, N)


@pytest.mark.parametrize("M,K,N", [(5, 1152, 272), (24, 3072, 1040), (40, 2048, 528), (100, 1152, 272),
                                   (233, 1152, 272), (497, 1152, 272), (1000, 1152, 272)])
def test_every_decode_candidate_is_exact(M, K, N):
    """Every plan the learned selector may pick (gemm_w4a8_decode_candidates)
    runs, and gives the oracle's INT32 accumulators bit for bit."""
    import torch
    from w4a8_quantized_linear_amd import (gemm_w4a8, gemm_w4a8_decode_candidates, gemm_w4a8_plan,
                                           quantize_act_per_token_i8)
    rng = np.random.default_rng(M * 7 + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float16)
    wq = gpu_weights(w)
    qx, sa = quantize_act_per_token_i8(to_dev(x))
    want = orc.linear(x, orc.quantize_weights(w))["acc"]
    cands = gemm_w4a8_decode_candidates(M, N, K)
    assert len(cands) >= 40
    for c in cands:
        plan = ",".join(str(v) for v in c)
        say("decode candidate M=%d K=%d N=%d plan=%s" % (M, K, N, plan))

        def run():
            got = gemm_w4a8_plan(M, N, K)
            assert got["kind"] == 0 and tuple(got[f] for f in ("mt", "nt", "splitk", "waves", "depth", "xstage",
                                                               "wave_n")) == c
            acc = torch.empty((M, N), dtype=torch.int32, device=dev())
            gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, acc_out=acc)
            torch.cuda.synchronize()
            return to_host(acc)
        assert np.array_equal(_with_plan(plan, run), want), plan
