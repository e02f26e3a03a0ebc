"""Host-side checks of the sweep shape generators in tuning.py (no GPU):
they are deterministic per seed, stay inside the ranges their docstrings
state, and the mid-M shapes pass the decode route's tile condition, so that
gemm_w4a8 sends all but the very large weights among them to the decode
kernels (those sweeps time decode plans against the dispatcher's own pick)."""
import pytest

from w4a8_quantized_linear_amd import tuning


def test_wide_shapes_ranges_and_determinism():
    a = tuning.wide_shapes(150, 5)
    assert a == tuning.wide_shapes(150, 5) and a != tuning.wide_shapes(150, 6)
    for M, N, K in a:
        assert 129 <= M <= 256 and N >= 512 and N % 128 == 0 and M * N <= (1 << 20)
        assert 2048 <= K <= 28672 and K % 128 == 0
    b = tuning.wide_shapes(120, 17, (1 << 20, 1 << 21))
    assert all((1 << 20) < M * N <= (1 << 21) for M, N, K in b)


@pytest.mark.parametrize("seed", [11, 13])
def test_mid_shapes_take_the_decode_kernels(seed):
    from w4a8_quantized_linear_amd import _lib
    shapes = tuning.mid_shapes(60, seed)
    assert shapes == tuning.mid_shapes(60, seed)
    for M, N, K in shapes:
        assert 65 <= M <= 128 and 512 <= N <= 16384 and N % 128 == 0 and 2048 <= K <= 28672
        # the generator keeps shapes whose 64 x 256 many-token tiles fill under half of 256 CUs
        assert -(-M // 64) * -(-N // 256) * 2 < 256
    # all of them pass the tile condition; only very large weights go to the matrix-core kernel
    kinds = [_lib.gemm_w4a8_plan(M, N, K)["kind"] for M, N, K in shapes]
    assert all(k == 0 for k, (M, N, K) in zip(kinds, shapes) if N * K <= (3 << 25))
