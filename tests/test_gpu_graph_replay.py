"""The hot path (act-quant + GEMM) captured in a HIP graph and replayed.

Split-K and stream-K plans keep arrival counters in the shared workspace and
rely on the last workgroup to reset them, so a replayed graph must leave the
workspace as an eager call does.  Each case captures the whole path once,
then replays it several times with other eager calls on the same workspace
and synchronisations in between, and checks every replay bit for bit against
the eager result of the same inputs.
"""
import os

import numpy as np
import pytest

from gpu_helpers import dev, f16_bits, say, to_host

pytestmark = pytest.mark.gpu

KEYS = ("W4A8_DECODE_PLAN", "W4A8_PREFILL_TM", "W4A8_PREFILL_P")

# (M, K, N, forced plan, plan fields that must hold)
CASES = [
    (8, 2048, 1024, {"W4A8_DECODE_PLAN": "1,2,4,4,2,0,0"}, {"kind": 0, "splitk": 4, "wave_n": 0}),
    (24, 2048, 2048, {"W4A8_DECODE_PLAN": "2,4,2,4,2,1,1"}, {"kind": 0, "splitk": 2, "wave_n": 1}),
    (257, 1152, 1040, {"W4A8_PREFILL_TM": "8", "W4A8_PREFILL_P": "64"}, {"kind": 1, "mt": 8, "splitk": 64}),
    (1100, 1024, 2048, {}, {"kind": 1, "splitk": 0}),
]


def _set_env(env):
    for k in KEYS:
        os.environ.pop(k, None)
    os.environ.update(env)


@pytest.mark.parametrize("M,K,N,env,want", CASES)
def test_graph_replays_match_eager(M, K, N, env, want):
    import torch

    from w4a8_quantized_linear_amd import (_lib, gemm_w4a8, gemm_w4a8_plan, quantize_act_per_token_i8,
                                           quantize_weights_w4g128, workloads)
    saved = {k: os.environ.get(k) for k in KEYS}
    try:
        _set_env(env)
        plan = gemm_w4a8_plan(M, N, K)
        say("graph replay M=%d K=%d N=%d env=%s plan=%s" % (M, K, N, env, plan))
        for k, v in want.items():
            assert plan[k] == v, (k, plan)
        d = dev()
        w = torch.from_numpy(workloads.weights(3, K, N)).to(d)
        wq = quantize_weights_w4g128(w, canonical=False)
        x = torch.from_numpy(workloads.activations(3, M, K, N)).to(d)
        ws = _lib.workspace(d, max(1, _lib.gemm_w4a8_workspace_bytes(M, N, K)))

        def path(qx, sa, y):
            quantize_act_per_token_i8(x, qx=qx, s_a=sa)
            gemm_w4a8(qx, sa, wq["wpacked"], wq["s0"], N, y=y, ws=ws)

        def buffers():
            return (torch.empty((M, K), dtype=torch.int8, device=d), torch.empty((M,), dtype=torch.float32, device=d),
                    torch.empty((M, N), dtype=torch.float16, device=d))

        ref = buffers()
        path(*ref)
        torch.cuda.synchronize()
        ref_q, ref_s, ref_y = to_host(ref[0]), to_host(ref[1]), f16_bits(ref[2])

        out = buffers()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                path(*out)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()

        # eager work on the same workspace between replays: another shape's
        # split plan of the same kind
        other = (max(1, M // 2), K, N)
        xo = torch.from_numpy(workloads.activations(3, other[0], K, N)).to(d)
        qo = torch.empty((other[0], K), dtype=torch.int8, device=d)
        so = torch.empty((other[0],), dtype=torch.float32, device=d)
        yo = torch.empty((other[0], N), dtype=torch.float16, device=d)
        for rep in range(4):
            for t in out:
                t.zero_()
            quantize_act_per_token_i8(xo, qx=qo, s_a=so)
            gemm_w4a8(qo, so, wq["wpacked"], wq["s0"], N, y=yo, ws=ws)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(to_host(out[0]), ref_q), rep
            assert np.array_equal(to_host(out[1]).view(np.uint32), ref_s.view(np.uint32)), rep
            assert np.array_equal(f16_bits(out[2]), ref_y), rep
        say("  %d replays bit-exact" % (rep + 1))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
