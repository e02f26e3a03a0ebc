"""Shared helpers of the GPU parity tests (not collected as tests)."""
import sys

import numpy as np

import oracle as orc
from w4a8_quantized_linear_amd import workloads

ATOL = 1e-2
RTOL = 1e-3


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t):
    return t.detach().cpu().numpy()


def f16_bits(t):
    """fp16 / int16 tensor -> numpy uint16 bit patterns."""
    import torch
    return to_host(t.contiguous().view(torch.int16)).view(np.uint16)


def sample_rows(n, count, seed):
    """Sorted sample of `count` row indices that includes the first and last few rows."""
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    edge = min(16, count // 4)
    pick = set(range(edge)) | set(range(n - edge, n))
    rest = np.setdiff1d(np.arange(n), np.array(sorted(pick), dtype=np.int64))
    pick |= set(rng.choice(rest, count - len(pick), replace=False).tolist())
    return np.array(sorted(pick))


def assert_y_close(y_gpu_bits, y_ref_bits, where=""):
    y = y_gpu_bits.view(np.float16).astype(np.float64)
    r = y_ref_bits.view(np.float16).astype(np.float64)
    err = np.abs(y - r)
    bad = err > ATOL + RTOL * np.abs(r)
    assert not bad.any(), "%s: %d outputs outside tolerance, worst %g" % (where, bad.sum(), err.max())


def gpu_weights(w_np):
    import torch
    from w4a8_quantized_linear_amd import quantize_weights_w4g128
    w = to_dev(w_np)
    wq = quantize_weights_w4g128(w, canonical=True)
    torch.cuda.synchronize()
    del w
    return wq


def oracle_weights_rows(w_np, rows):
    return orc.quantize_weights(np.ascontiguousarray(w_np[rows]))


def case_inputs(family, M, K, N):
    return workloads.weights(family, K, N), workloads.activations(family, M, K, N)
