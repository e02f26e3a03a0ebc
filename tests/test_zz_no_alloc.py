"""gemm_w4a8_noalloc through the C ABI against gemm_w4a8 with a workspace.

The no-allocation entry point runs the same plans and kernels with the
library's fixed device scratch as the split-K / stream-K workspace.  Two (and
more) calls in a row share that scratch: a stream-K prefill call, then
smaller decode calls (N-split split-K, K-split split-K, unsplit), then the
large call again.  Each is compared with gemm_w4a8's INT32 accumulators and
fp16 outputs bit for bit, and with the oracle.  A shape whose plan needs more
than the scratch holds is rejected before any launch.
"""
import numpy as np
import pytest

import oracle as orc
from gpu_helpers import assert_y_close, dev, f16_bits, gpu_weights, say, to_dev, to_host
from w4a8_quantized_linear_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from w4a8_quantized_linear_amd import _lib
    _lib.load()
    yield


def test_noalloc_matches_gemm_w4a8_on_calls_in_a_row():
    import torch
    from w4a8_quantized_linear_amd import _lib, gemm_w4a8, gemm_w4a8_noalloc, quantize_act_per_token_i8
    # (M, K, N): stream-K TM=4 (33.6 MB of workspace), N-split split-K 2,
    # K-split split-K 4, unsplit, and the first shape again
    seq = [(768, 11008, 4096), (32, 4096, 11008), (16, 11008, 4096), (1, 4096, 4096), (768, 11008, 4096)]
    weights = {}
    for M, K, N in seq:
        need = _lib.gemm_w4a8_workspace_bytes(M, N, K)
        assert need <= _lib.NOALLOC_SCRATCH_BYTES
        say("no-alloc M=%d K=%d N=%d (workspace %d B, plan %s)" % (M, K, N, need, _lib.gemm_w4a8_plan(M, N, K)))
        if (K, N) not in weights:
            w = workloads.weights(1, K, N)
            weights[(K, N)] = (w, gpu_weights(w), orc.quantize_weights(w))
        w, wq, ref_w = weights[(K, N)]
        x = workloads.activations(1, M, K, N)
        qx, sa = quantize_act_per_token_i8(to_dev(x))
        acc_a = torch.full((M, N), 7, dtype=torch.int32, device=dev())
        acc_b = torch.full((M, N), 9, dtype=torch.int32, device=dev())
        y_a = torch.empty((M, N), dtype=torch.float16, device=dev())
        y_b = torch.empty((M, N), dtype=torch.float16, device=dev())
        gemm_w4a8_noalloc(qx, sa, wq["wpacked"], wq["s0"], N, y=y_a, acc_out=acc_a)
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=dev())
        gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, y=y_b, acc_out=acc_b, ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(acc_a), to_host(acc_b)), (M, K, N)
        assert np.array_equal(f16_bits(y_a), f16_bits(y_b)), (M, K, N)
        out = orc.linear(x, ref_w)
        assert np.array_equal(to_host(acc_a), out["acc"]), (M, K, N)
        assert_y_close(f16_bits(y_a), out["y"], "no-alloc M=%d" % M)


def test_noalloc_rejects_a_plan_larger_than_the_scratch():
    """The 70B down projection at 512 tokens plans TM = 8 with each of its 128
    tiles split into two K ranges (256 ranges): 67,174,400 bytes of
    workspace, more than the 64 MiB scratch.
    The call returns W4A8_E_SCRATCH and launches nothing (y keeps its
    contents); M = 0 stays a no-op."""
    import torch
    from w4a8_quantized_linear_amd import _lib
    M, K, N = 512, 28672, 8192
    need = _lib.gemm_w4a8_workspace_bytes(M, N, K)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    qx = torch.zeros((M, K), dtype=torch.int8, device=dev())
    sa = torch.zeros((M,), dtype=torch.float32, device=dev())
    wp = torch.zeros(_lib.w4a8_packed_weight_bytes(N, K), dtype=torch.uint8, device=dev())
    s0 = torch.zeros((N,), dtype=torch.int16, device=dev())
    y = torch.full((M, N), 3.0, dtype=torch.float16, device=dev())
    with pytest.raises(_lib.W4A8Error) as e:
        _lib.gemm_w4a8_noalloc(qx, sa, wp, s0, N, y=y)
    assert e.value.status == _lib.W4A8_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    _lib.gemm_w4a8_noalloc(qx[:0], sa[:0], wp, s0, N, y=y[:0])
