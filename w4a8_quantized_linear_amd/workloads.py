"""Seeded synthetic inputs for the W4A8 linear layer.

This module only draws random numbers; it holds none of the method's
arithmetic, and both the CPU oracle's callers and the GPU path's callers take
their inputs from it.

Recipe (one per workload family; every draw is seeded):
  * generator: numpy PCG64 seeded by SeedSequence([0x57A8, family, K, N, tensor_id(, M)])
    with tensor_id 0 = weights, 1 = activations (M appended), 2 = outlier channels,
    3 = the normalization's gamma and beta rows (family and N are 0 there);
  * weights: fp32, N(0, 0.02) -- or, for the heavy-tailed family, Student-t with
    nu = 4 scaled to the same std (divide by the population std sqrt(2));
  * activations: fp32 N(0, 1) with a fixed set of outlier channels (the same
    channels for every token) multiplied by a large factor, then rounded to fp16.
    Four channels x50 by default; 1% of channels x100 for the heavy-tailed family.
The outlier structure follows the pages' description of LLM activations: a
small fraction of feature channels, fixed across tokens, tens to hundreds of
times larger than the rest.
  * KV cache rows (decode attention over the 4-bit cache): keys and values
    N(0, 1) fp16, keys with 4 channels per head x10, fixed across tokens;
    queries N(0, 1); ragged context lengths uniform in [1, S];
  * normalization rows (the fused LayerNorm/RMSNorm producer): gamma =
    fp16(1 + 0.1 N(0, 1)), beta = fp16(0.05 N(0, 1)), stand-ins for trained
    affine parameters (no checkpoint is used).
"""
from __future__ import annotations

import dataclasses
from typing import List, Tuple

import numpy as np

SEED_ROOT = 0x57A8


@dataclasses.dataclass(frozen=True)
class Family:
    """One workload family (value distributions + shapes)."""
    index: int
    name: str
    ms: Tuple[int, ...]
    kns: Tuple[Tuple[int, int], ...]       # (K, N) pairs
    w_dist: str = "normal"                 # "normal" | "student_t4"
    n_outlier: int = 4                     # or -1 for 1% of K
    outlier_scale: float = 50.0


FAMILIES: List[Family] = [
    Family(0, "tiny: M=16, K=512, N=512", (16,), ((512, 512),)),
    Family(1, "7B decode: hidden 4096, MLP 11008", (1, 8, 32),
           ((4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096))),
    Family(2, "batched decode M=256, K=4096, N=11008, heavy-tailed weights", (256,),
           ((4096, 11008),), w_dist="student_t4", n_outlier=-1, outlier_scale=100.0),
    Family(3, "prefill M=4096", (4096,), ((4096, 11008), (11008, 4096))),
    Family(4, "70B layers: hidden 8192, MLP 28672", (1, 64, 512),
           ((8192, 10240), (8192, 57344), (28672, 8192))),
]

# The benchmark's workload: the 7B MLP projection K=4096 -> N=11008, swept over
# token counts from one decode token to a 4096-token prefill.
SWEEP_K, SWEEP_N = 4096, 11008
SWEEP_MS = (1, 8, 32, 256, 4096)


def _rng(family: int, K: int, N: int, tensor_id: int, *extra: int) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, family, K, N, tensor_id, *extra])
    return np.random.Generator(np.random.PCG64(ss))


def weights(family: int, K: int, N: int) -> np.ndarray:
    """fp32 weights [N, K] (independent of M)."""
    fam = FAMILIES[family]
    rng = _rng(family, K, N, 0)
    if fam.w_dist == "student_t4":
        w = rng.standard_t(4.0, size=(N, K)) * (0.02 / np.sqrt(2.0))
        return w.astype(np.float32)
    w = rng.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def outlier_channels(family: int, K: int, N: int) -> np.ndarray:
    fam = FAMILIES[family]
    n_out = fam.n_outlier if fam.n_outlier >= 0 else int(round(0.01 * K))
    n_out = min(n_out, K)
    rng = _rng(family, K, N, 2)
    return np.sort(rng.choice(K, n_out, replace=False))


def activations(family: int, M: int, K: int, N: int) -> np.ndarray:
    """fp16 activations [M, K] with fixed outlier channels."""
    fam = FAMILIES[family]
    rng = _rng(family, K, N, 1, M)
    x = rng.standard_normal((M, K), dtype=np.float32)
    cols = outlier_channels(family, K, N)
    x[:, cols] *= np.float32(fam.outlier_scale)
    return x.astype(np.float16)


def norm_affine(K: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 gamma [K] and beta [K] of the normalization in front of the quantizer."""
    rng = _rng(0, K, 0, 3)
    g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16)
    b = (0.05 * rng.standard_normal(K)).astype(np.float16)
    return g, b


# ---------------------------------------------------------------------------
# KV cache workloads (decode attention over the 4-bit cache).  The shapes are
# the lectures' reference 7B at a 4,096-token context (32 query heads of 128):
# multi-head (32 kv heads) and grouped-query with 8 kv heads.  Keys carry a
# few large channels, fixed per head across tokens (the QServe talk summary:
# the key cache has outlier channels, the value cache is closer to normal);
# values are N(0, 1).
# ---------------------------------------------------------------------------
KV_HEAD_DIM = 128
KV_CONFIGS = {
    "7b_mha": dict(B=64, Hq=32, Hkv=32, S=4096),
    "7b_gqa8": dict(B=256, Hq=32, Hkv=8, S=4096),
}
KV_OUTLIERS_PER_HEAD = 4
KV_OUTLIER_SCALE = 10.0


def _kv_rng(*ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_ROOT, 5, *ids])))


def kv_outlier_channels(seed: int, Hkv: int) -> np.ndarray:
    """[Hkv, KV_OUTLIERS_PER_HEAD] key channels that are large in every token."""
    rng = _kv_rng(seed, Hkv, 0)
    return np.stack([np.sort(rng.choice(KV_HEAD_DIM, KV_OUTLIERS_PER_HEAD, replace=False)) for _ in range(Hkv)])


def kv_rows(seed: int, B: int, T: int, Hkv: int, part: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 new keys and values [B, T, Hkv, 128] (part: an index for filling a cache piecewise)."""
    rng = _kv_rng(seed, B, T, Hkv, part + 1)
    k = rng.standard_normal((B, T, Hkv, KV_HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((B, T, Hkv, KV_HEAD_DIM), dtype=np.float32)
    cols = kv_outlier_channels(seed, Hkv)
    for g in range(Hkv):
        k[:, :, g, cols[g]] *= np.float32(KV_OUTLIER_SCALE)
    return k.astype(np.float16), v.astype(np.float16)


def kv_rows_torch(seed: int, B: int, T: int, Hkv: int, part: int, device):
    """The same distribution drawn on the GPU with torch's seeded generator (for filling
    caches too large to draw on the host); same outlier channels as kv_rows."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed((seed * 1000003 + part * 7919 + B * 131 + T * 17 + Hkv) & 0x7FFFFFFF)
    k = torch.randn((B, T, Hkv, KV_HEAD_DIM), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((B, T, Hkv, KV_HEAD_DIM), generator=gen, device=device, dtype=torch.float32)
    cols = torch.from_numpy(kv_outlier_channels(seed, Hkv)).to(device)
    scale = torch.ones((Hkv, KV_HEAD_DIM), device=device)
    scale.scatter_(1, cols, KV_OUTLIER_SCALE)
    k *= scale
    return k.half(), v.half()


def kv_query(seed: int, B: int, Hq: int) -> np.ndarray:
    """fp16 queries [B, Hq, 128], N(0, 1)."""
    return _kv_rng(seed, B, Hq, 0, 1).standard_normal((B, Hq, KV_HEAD_DIM), dtype=np.float32).astype(np.float16)


def kv_lens(seed: int, B: int, S: int) -> np.ndarray:
    """Ragged context lengths in [1, S] (uniform), the longest and shortest included."""
    rng = _kv_rng(seed, B, S, 0, 2)
    lens = rng.integers(1, S + 1, B).astype(np.int32)
    lens[0] = S
    if B > 1:
        lens[-1] = 1
    return lens


def all_cases():
    """Every (family, M, K, N) the families name."""
    for fam in FAMILIES:
        for (K, N) in fam.kns:
            for M in fam.ms:
                yield fam.index, M, K, N
