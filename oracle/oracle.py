"""ctypes wrappers around the C oracle (``w4a8_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Every function takes and
returns numpy arrays on the host; none touches a GPU.  Each wrapper names the
step of the method it computes; the citations of the pages are next to the C
implementation of that step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# A different build of the same source may be substituted (the mutation test
# of the pins loads deliberately broken copies this way).
_LIB_OVERRIDE = os.environ.get("W4A8_ORACLE_LIB")
_lock = threading.Lock()
_lib = None

GROUP = 128
PROTECT = 119


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB_PATH):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.orc_f16_to_f32.restype = ctypes.c_float
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_rne_div.argtypes = [I64, I64]
        lib.orc_rne_div.restype = I64
        lib.orc_quantize_act.argtypes = [P, I64, I64, I64, P, P]
        lib.orc_quantize_act.restype = None
        lib.orc_norm_quantize_act.argtypes = [P, I64, I64, I64, P, P, ctypes.c_float, ctypes.c_int,
                                              P, P, P, P, P]
        lib.orc_norm_quantize_act.restype = None
        lib.orc_weights_level1.argtypes = [P, I64, I64, P, P]
        lib.orc_weights_level1.restype = None
        lib.orc_weights_level2.argtypes = [P, I64, I64, P, P, P]
        lib.orc_weights_level2.restype = None
        lib.orc_pack_q4.argtypes = [P, I64, I64, P]
        lib.orc_pack_q4.restype = None
        lib.orc_dequant_i8.argtypes = [P, P, P, I64, I64, P]
        lib.orc_dequant_i8.restype = I64
        lib.orc_gemm_acc.argtypes = [P, P, I64, I64, I64, P]
        lib.orc_gemm_acc.restype = I64
        lib.orc_gemm_w4a16.argtypes = [P, I64, I64, P, P, I64, P, P]
        lib.orc_gemm_w4a16.restype = None
        lib.orc_quantize_kv4.argtypes = [P, I64, I64, P, P, P]
        lib.orc_quantize_kv4.restype = None
        lib.orc_kv4_attention.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, I64, P,
                                          ctypes.c_double, P, P, P, P]
        lib.orc_kv4_attention.restype = None
        lib.orc_epilogue.argtypes = [P, P, P, I64, I64, P]
        lib.orc_epilogue.restype = None
        lib.orc_linear.argtypes = [P, I64, I64, P, P, P, P, I64, P, P, P, P, P]
        lib.orc_linear.restype = ctypes.c_int
        lib.orc_num_threads.argtypes = []
        lib.orc_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _as(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# Scalar helpers
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: float) -> int:
    return int(_load().orc_f32_to_f16(float(x)))


def f16_bits_to_f32(h: int) -> float:
    return float(_load().orc_f16_to_f32(int(h) & 0xFFFF))


def f32_to_f16_bits_array(x: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = _as(x, np.float32).ravel()
    out = np.empty(flat.shape, np.uint16)
    for i, v in enumerate(flat):
        out[i] = lib.orc_f32_to_f16(float(v))
    return out.reshape(np.shape(x))


def rne_div(p: int, d: int) -> int:
    return int(_load().orc_rne_div(int(p), int(d)))


def num_threads() -> int:
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------
# The steps of the path
# --------------------------------------------------------------------------
def quantize_act(x_f16: np.ndarray):
    """Per-token absmax INT8 activations.  x: fp16 [M, K] -> (qx int8 [M,K], s_a fp32 [M])."""
    x = _as(x_f16, np.float16)
    M, K = x.shape
    qx = np.empty((M, K), np.int8)
    sa = np.empty((M,), np.float32)
    _load().orc_quantize_act(_p(x), M, K, K, _p(qx), _p(sa))
    return qx, sa


def norm_quantize_act(x_f16: np.ndarray, gamma_f16: np.ndarray, beta_f16=None,
                      eps: float = 1e-5, rms: bool = False):
    """LayerNorm (or RMSNorm) fused with the per-token INT8 quantizer.

    x: fp16 [M, K]; gamma, beta: fp16 [K] (beta may be None).  Returns a dict
    with qx int8 [M,K], s_a fp32 [M], h (the normalized fp16 row, as uint16
    bits [M,K]), mean and r (double [M]: the statistics before rounding to fp32).
    """
    x = _as(x_f16, np.float16)
    M, K = x.shape
    g = _as(gamma_f16, np.float16)
    b = None if beta_f16 is None else _as(beta_f16, np.float16)
    assert g.shape == (K,) and (b is None or b.shape == (K,))
    out = {"qx": np.empty((M, K), np.int8), "s_a": np.empty((M,), np.float32),
           "h": np.empty((M, K), np.uint16), "mean": np.empty((M,), np.float64),
           "r": np.empty((M,), np.float64)}
    _load().orc_norm_quantize_act(_p(x), M, K, K, _p(g), None if b is None else _p(b),
                                  float(np.float32(eps)), int(bool(rms)), _p(out["qx"]),
                                  _p(out["s_a"]), _p(out["h"]), _p(out["mean"]), _p(out["r"]))
    return out


def rstd_near_midpoint(r: np.ndarray, rel: float = 2.0 ** -36) -> np.ndarray:
    """Tokens whose double r lies within rel * r of a midpoint between two
    adjacent floats: another order of the sum of squares may round r to the
    other float there (see the C oracle's note).  False where r is infinite."""
    r = np.asarray(r, np.float64)
    out = np.zeros(r.shape, bool)
    fin = np.isfinite(r) & (r > 0)
    f = r[fin].astype(np.float32)
    lo = np.nextafter(f, np.float32(0)).astype(np.float64)
    hi = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    fd = f.astype(np.float64)
    d = np.minimum(np.abs(r[fin] - (fd + lo) / 2), np.abs(r[fin] - (fd + hi) / 2))
    out[fin] = d <= rel * r[fin]
    return out


def weights_level1(w: np.ndarray):
    """Per-channel INT8 in [-119, 119] with fp16 scale.  -> (q8 int8 [N,K], s0 fp16-bits uint16 [N])."""
    w = _as(w, np.float32)
    N, K = w.shape
    q8 = np.empty((N, K), np.int8)
    s0 = np.empty((N,), np.uint16)
    _load().orc_weights_level1(_p(w), N, K, _p(q8), _p(s0))
    return q8, s0


def weights_level2(q8: np.ndarray):
    """Per-group-128 UINT4 with integer scale and zero.  -> (q4 uint8 [N,K] one code per byte, s1 [N,G], z [N,G])."""
    q8 = _as(q8, np.int8)
    N, K = q8.shape
    assert K % GROUP == 0
    G = K // GROUP
    q4 = np.empty((N, K), np.uint8)
    s1 = np.empty((N, G), np.uint8)
    z = np.empty((N, G), np.uint8)
    _load().orc_weights_level2(_p(q8), N, K, _p(q4), _p(s1), _p(z))
    return q4, s1, z


def pack_q4(q4: np.ndarray) -> np.ndarray:
    """Canonical packing [N, K/2], even k in the low nibble."""
    q4 = _as(q4, np.uint8)
    N, K = q4.shape
    out = np.empty((N, K // 2), np.uint8)
    _load().orc_pack_q4(_p(q4), N, K, _p(out))
    return out


def dequant_i8(q4: np.ndarray, s1: np.ndarray, z: np.ndarray):
    """Subtract-after-multiply reconstruction r = q4*s1 - z*s1.  -> (r int8 [N,K], number of out-of-range values)."""
    q4 = _as(q4, np.uint8)
    s1 = _as(s1, np.uint8)
    z = _as(z, np.uint8)
    N, K = q4.shape
    r = np.empty((N, K), np.int8)
    bad = _load().orc_dequant_i8(_p(q4), _p(s1), _p(z), N, K, _p(r))
    return r, int(bad)


def gemm_acc(qx: np.ndarray, r: np.ndarray):
    """Exact INT32 accumulators acc[m,n] = sum_k qx[m,k] r[n,k] (int64 inside).  -> (acc int32 [M,N], overflow count)."""
    qx = _as(qx, np.int8)
    r = _as(r, np.int8)
    M, K = qx.shape
    N, K2 = r.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    bad = _load().orc_gemm_acc(_p(qx), _p(r), M, N, K, _p(acc))
    return acc, int(bad)


def epilogue(acc: np.ndarray, s_a: np.ndarray, s0: np.ndarray) -> np.ndarray:
    """fp16 output bits y = fp16((float(acc) * s_a[m]) * float(s0[n]))."""
    acc = _as(acc, np.int32)
    s_a = _as(s_a, np.float32)
    s0 = _as(s0, np.uint16)
    M, N = acc.shape
    y = np.empty((M, N), np.uint16)
    _load().orc_epilogue(_p(acc), _p(s_a), _p(s0), M, N, _p(y))
    return y


def gemm_w4a16(x_f16: np.ndarray, r: np.ndarray, s0: np.ndarray):
    """W4A16: ref[m,n] = sum_k x[m,k] r[n,k] s0[n] in double, and the sum of the |terms|.

    x: fp16 [M, K]; r: int8 [N, K] (from dequant_i8); s0: fp16 bits [N].  -> (ref, absref), double [M, N]."""
    x = _as(x_f16, np.float16)
    r = _as(r, np.int8)
    s0 = _as(s0, np.uint16)
    M, K = x.shape
    N = r.shape[0]
    assert r.shape == (N, K) and s0.shape == (N,)
    ref = np.empty((M, N), np.float64)
    absref = np.empty((M, N), np.float64)
    _load().orc_gemm_w4a16(_p(x), M, K, _p(r), _p(s0), N, _p(ref), _p(absref))
    return ref, absref


def quantize_kv4(x_f16: np.ndarray) -> dict:
    """4-bit KV cache rows: x fp16 [..., D] -> codes uint8 [..., D] (one per byte),
    s fp16 bits uint16 [...], z uint8 [...]; x ~ (codes - z) * s."""
    x = _as(x_f16, np.float16)
    D = x.shape[-1]
    lead = x.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    codes = np.empty(x.shape, np.uint8)
    s = np.empty(lead, np.uint16)
    z = np.empty(lead, np.uint8)
    _load().orc_quantize_kv4(_p(x.view(np.uint16)), rows, D, _p(codes), _p(s), _p(z))
    return {"codes": codes, "s": s, "z": z}


def kv4_dequant(kv: dict) -> np.ndarray:
    """(codes - z) * s in double."""
    s = np.array(kv["s"], np.uint16).view(np.float16).astype(np.float64)
    return (kv["codes"].astype(np.float64) - kv["z"][..., None].astype(np.float64)) * s[..., None]


def kv4_attention(q_f16: np.ndarray, k: dict, v: dict, lens: np.ndarray, sm_scale: float) -> dict:
    """Decode attention over the 4-bit cache.  q: fp16 [B, Hq, D]; k, v: quantize_kv4 outputs
    of shape [B, Hkv, S, D]; lens int32 [B].  -> dict of double arrays: out, absout [B, Hq, D],
    score, absscore [B, Hq, S]."""
    q = _as(q_f16, np.float16)
    B, Hq, D = q.shape
    _, Hkv, S, D2 = k["codes"].shape
    assert D2 == D and Hq % Hkv == 0 and v["codes"].shape == k["codes"].shape
    lens = _as(lens, np.int32)
    assert lens.shape == (B,) and np.all((lens >= 0) & (lens <= S))
    out = np.empty((B, Hq, D), np.float64)
    absout = np.empty((B, Hq, D), np.float64)
    score = np.empty((B, Hq, S), np.float64)
    absscore = np.empty((B, Hq, S), np.float64)
    kc, ks, kz = (_as(k["codes"], np.uint8), _as(k["s"], np.uint16), _as(k["z"], np.uint8))
    vc, vs, vz = (_as(v["codes"], np.uint8), _as(v["s"], np.uint16), _as(v["z"], np.uint8))
    _load().orc_kv4_attention(_p(q.view(np.uint16)), B, Hq, Hkv, D, _p(kc), _p(ks), _p(kz), _p(vc), _p(vs),
                              _p(vz), S, _p(lens), float(sm_scale), _p(out), _p(absout), _p(score),
                              _p(absscore))
    return {"out": out, "absout": absout, "score": score, "absscore": absscore}


def quantize_weights(w: np.ndarray) -> dict:
    """Both levels of the progressive weight quantization."""
    q8, s0 = weights_level1(w)
    q4, s1, z = weights_level2(q8)
    return {"q8": q8, "s0": s0, "q4": q4, "s1": s1, "z": z}


def linear(x_f16: np.ndarray, wq: dict) -> dict:
    """The serving-time path: activation quantization, dequant, contraction, epilogue."""
    qx, sa = quantize_act(x_f16)
    r, bad_r = dequant_i8(wq["q4"], wq["s1"], wq["z"])
    assert bad_r == 0
    acc, bad_a = gemm_acc(qx, r)
    assert bad_a == 0
    y = epilogue(acc, sa, wq["s0"])
    return {"qx": qx, "s_a": sa, "r": r, "acc": acc, "y": y}


def linear_timed_buffers(M: int, N: int, K: int):
    """Preallocated outputs for ``linear_into`` (used to time the oracle)."""
    return {"qx": np.empty((M, K), np.int8), "s_a": np.empty((M,), np.float32),
            "r": np.empty((N, K), np.int8), "acc": np.empty((M, N), np.int32),
            "y": np.empty((M, N), np.uint16)}


def linear_into(x_f16: np.ndarray, wq: dict, bufs: dict) -> int:
    """One whole serving-time call in C; returns the thread count it used."""
    x = _as(x_f16, np.float16)
    M, K = x.shape
    N = wq["q4"].shape[0]
    return int(_load().orc_linear(_p(x), M, K, _p(wq["q4"]), _p(wq["s1"]), _p(wq["z"]),
                                  _p(wq["s0"]), N, _p(bufs["qx"]), _p(bufs["s_a"]),
                                  _p(bufs["r"]), _p(bufs["acc"]), _p(bufs["y"])))


__all__ = [
    "GROUP", "PROTECT", "build", "f32_to_f16_bits", "f16_bits_to_f32", "f32_to_f16_bits_array",
    "rne_div", "num_threads", "quantize_act", "norm_quantize_act", "rstd_near_midpoint",
    "weights_level1", "weights_level2", "pack_q4",
    "dequant_i8", "gemm_acc", "gemm_w4a16", "epilogue", "quantize_weights", "linear",
    "quantize_kv4", "kv4_dequant", "kv4_attention",
    "linear_timed_buffers", "linear_into",
]
