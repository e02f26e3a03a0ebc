"""ctypes binding of libw4a8 (include/w4a8.h), with the same entry-point names.

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's kernels.  If
the library is not built the calls raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libw4a8.so")

W4A8_OK = 0
W4A8_E_NULL = -1
W4A8_E_SHAPE = -2
W4A8_E_ALIGN = -3
W4A8_E_WORKSPACE = -4
W4A8_E_HIP = -5
W4A8_E_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20     # W4A8_NOALLOC_SCRATCH_BYTES

# every symbol include/w4a8.h declares
EXPORTS = (
    "w4a8_status_string", "w4a8_version", "w4a8_packed_weight_bytes",
    "quantize_weights_w4g128", "w4a8_unpack_weights", "quantize_act_per_token_i8",
    "norm_quantize_act_i8", "gemm_w4a8_workspace_bytes", "gemm_w4a8", "gemm_w4a8_noalloc", "gemm_w4a16",
    "kv4_cache_bytes", "quantize_kv4", "kv4_unpack", "kv4_attention_workspace_bytes",
    "attention_kv4_decode", "gemm_w4a8_plan", "gemm_w4a8_plan_detail", "gemm_w4a8_decode_candidates",
    "gemm_w4a8_selector_score", "w4a8_hbm_read",
)

_lock = threading.Lock()
_lib = None


class W4A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))


def load() -> ctypes.CDLL:
    """Load libw4a8.so from the package directory (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise ImportError("libw4a8.so is not built (run `python -m w4a8_quantized_linear_amd.build`): %s"
                              % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        P, I64, SZ, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        lib.w4a8_status_string.argtypes = [I32]
        lib.w4a8_status_string.restype = ctypes.c_char_p
        lib.w4a8_version.argtypes = []
        lib.w4a8_version.restype = ctypes.c_char_p
        lib.w4a8_packed_weight_bytes.argtypes = [I64, I64]
        lib.w4a8_packed_weight_bytes.restype = SZ
        lib.quantize_weights_w4g128.argtypes = [P, I64, I64, P, P, P, P, P]
        lib.quantize_weights_w4g128.restype = I32
        lib.w4a8_unpack_weights.argtypes = [P, I64, I64, P, P, P, P]
        lib.w4a8_unpack_weights.restype = I32
        lib.quantize_act_per_token_i8.argtypes = [P, I64, I64, I64, P, P, P]
        lib.quantize_act_per_token_i8.restype = I32
        lib.norm_quantize_act_i8.argtypes = [P, I64, I64, I64, P, P, ctypes.c_float, I32, P, P, P]
        lib.norm_quantize_act_i8.restype = I32
        lib.gemm_w4a8_workspace_bytes.argtypes = [I64, I64, I64]
        lib.gemm_w4a8_workspace_bytes.restype = SZ
        lib.gemm_w4a8.argtypes = [P, P, P, P, I64, I64, I64, P, P, P, SZ, P]
        lib.gemm_w4a8.restype = I32
        lib.gemm_w4a8_noalloc.argtypes = [P, P, P, P, I64, I64, I64, P, P, P]
        lib.gemm_w4a8_noalloc.restype = I32
        lib.gemm_w4a16.argtypes = [P, I64, I64, I64, P, P, I64, P, P]
        lib.gemm_w4a16.restype = I32
        lib.gemm_w4a8_plan.argtypes = [I64, I64, I64, P]
        lib.gemm_w4a8_plan.restype = I32
        lib.w4a8_hbm_read.argtypes = [P, SZ, P, P]
        lib.w4a8_hbm_read.restype = I32
        lib.gemm_w4a8_plan_detail.argtypes = [I64, I64, I64, I32, P]
        lib.gemm_w4a8_plan_detail.restype = I32
        lib.gemm_w4a8_decode_candidates.argtypes = [I64, I64, I64, P, I32, P]
        lib.gemm_w4a8_decode_candidates.restype = I32
        lib.gemm_w4a8_selector_score.argtypes = [I64, I64, I64, P, I64]
        lib.gemm_w4a8_selector_score.restype = ctypes.c_float
        lib.kv4_cache_bytes.argtypes = [I64, I64, I64]
        lib.kv4_cache_bytes.restype = SZ
        lib.quantize_kv4.argtypes = [P, P, I64, I64, I64, P, P, P, I64, P]
        lib.quantize_kv4.restype = I32
        lib.kv4_unpack.argtypes = [P, I32, I64, I64, I64, P, P, P, P]
        lib.kv4_unpack.restype = I32
        lib.kv4_attention_workspace_bytes.argtypes = [I64, I64, I64]
        lib.kv4_attention_workspace_bytes.restype = SZ
        lib.attention_kv4_decode.argtypes = [P, I64, I64, I64, P, P, I64, P, ctypes.c_float, P, P, SZ, P]
        lib.attention_kv4_decode.restype = I32
        _lib = lib
        return lib


def status_string(st: int) -> str:
    return load().w4a8_status_string(int(st)).decode()


def version() -> str:
    return load().w4a8_version().decode()


def _check(st: int, where: str):
    if st != W4A8_OK:
        raise W4A8Error(st, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# --------------------------------------------------------------------------
# entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def w4a8_packed_weight_bytes(N: int, K: int) -> int:
    return int(load().w4a8_packed_weight_bytes(N, K))


def gemm_w4a8_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().gemm_w4a8_workspace_bytes(M, N, K))


def quantize_weights_w4g128(w, *, canonical: bool = True, stream=None):
    """fp32 weights [N, K] on the GPU -> dict(wpacked uint8, s0 int16 (fp16 bits)[, s1, z uint8 [N, K/128]])."""
    import torch
    assert w.dtype == torch.float32 and w.dim() == 2 and w.is_contiguous()
    N, K = w.shape
    nbytes = w4a8_packed_weight_bytes(N, K)
    if nbytes == 0:
        _check(W4A8_E_SHAPE, "quantize_weights_w4g128")
    dev = w.device
    out = {"N": N, "K": K,
           "wpacked": torch.empty(nbytes, dtype=torch.uint8, device=dev),
           "s0": torch.empty(N, dtype=torch.int16, device=dev)}
    if canonical:
        out["s1"] = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)
        out["z"] = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)
    st = load().quantize_weights_w4g128(_ptr(w), N, K, _ptr(out["wpacked"]), _ptr(out.get("s1")),
                                        _ptr(out.get("z")), _ptr(out["s0"]), _stream(stream))
    _check(st, "quantize_weights_w4g128")
    return out


def w4a8_unpack_weights(wpacked, N: int, K: int, *, stream=None):
    """Device weight stream -> (q4 canonical [N, K/2] uint8, s1 [N, K/128], z [N, K/128])."""
    import torch
    dev = wpacked.device
    q4 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    s1 = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)
    z = torch.empty((N, K // 128), dtype=torch.uint8, device=dev)
    st = load().w4a8_unpack_weights(_ptr(wpacked), N, K, _ptr(q4), _ptr(s1), _ptr(z), _stream(stream))
    _check(st, "w4a8_unpack_weights")
    return q4, s1, z


def quantize_act_per_token_i8(x, *, qx=None, s_a=None, stream=None):
    """fp16 activations [M, K] (row stride x.stride(0)) -> (qx int8 [M, K], s_a fp32 [M])."""
    import torch
    assert x.dtype == torch.float16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=x.device)
    st = load().quantize_act_per_token_i8(_ptr(x), M, K, x.stride(0), _ptr(qx), _ptr(s_a), _stream(stream))
    _check(st, "quantize_act_per_token_i8")
    return qx, s_a


def norm_quantize_act_i8(x, gamma, beta=None, *, eps: float = 1e-5, rms: bool = False, qx=None,
                         s_a=None, stream=None):
    """LayerNorm (rms=False) or RMSNorm (rms=True) of fp16 rows [M, K] with fp16 gamma [K]
    (and optional beta [K]), quantized per token -> (qx int8 [M, K], s_a fp32 [M])."""
    import torch
    assert x.dtype == torch.float16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    assert gamma.dtype == torch.float16 and gamma.shape == (K,) and gamma.is_contiguous()
    assert beta is None or (beta.dtype == torch.float16 and beta.shape == (K,) and beta.is_contiguous())
    if qx is None:
        qx = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if s_a is None:
        s_a = torch.empty((M,), dtype=torch.float32, device=x.device)
    st = load().norm_quantize_act_i8(_ptr(x), M, K, x.stride(0), _ptr(gamma), _ptr(beta), float(eps),
                                     int(bool(rms)), _ptr(qx), _ptr(s_a), _stream(stream))
    _check(st, "norm_quantize_act_i8")
    return qx, s_a


_ws_lock = threading.Lock()
_ws_cache = {}


def workspace(device, nbytes: int):
    """A zeroed split-K workspace of at least nbytes on `device`, cached per device.

    The kernels leave it zeroed after every call, so it is cleared only when
    first allocated (or grown).  Calls that share it must be stream-ordered."""
    import torch
    if nbytes == 0:
        return None
    key = torch.device(device)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=key)
            _ws_cache[key] = buf
        return buf


def gemm_w4a8(qx, s_a, wpacked, s0, N: int, *, y=None, acc_out=None, ws=None, use_workspace: bool = True,
              stream=None):
    """INT8 activations [M, K] x packed weights -> fp16 y [M, N] (and INT32 acc_out if given).

    ws: the split-K workspace (default: one cached per device); use_workspace=False passes NULL."""
    import torch
    M, K = qx.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=qx.device)
    need = gemm_w4a8_workspace_bytes(M, N, K)
    if not use_workspace:
        ws = None
    elif ws is None:
        ws = workspace(qx.device, need)
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().gemm_w4a8(_ptr(qx), _ptr(s_a), _ptr(wpacked), _ptr(s0), M, N, K, _ptr(y),
                          _ptr(acc_out), _ptr(ws), wsb, _stream(stream))
    _check(st, "gemm_w4a8")
    return y


def gemm_w4a8_noalloc(qx, s_a, wpacked, s0, N: int, *, y, acc_out=None, stream=None):
    """gemm_w4a8 with the library's fixed device scratch as its workspace: allocates nothing (y is
    required).  Calls that overlap on one GPU race."""
    M, K = qx.shape
    st = load().gemm_w4a8_noalloc(_ptr(qx), _ptr(s_a), _ptr(wpacked), _ptr(s0), M, N, K, _ptr(y),
                                  _ptr(acc_out), _stream(stream))
    _check(st, "gemm_w4a8_noalloc")
    return y


def gemm_w4a16(x, wpacked, s0, N: int, *, y=None, stream=None):
    """fp16 activations [M, K] (row stride x.stride(0)) x packed weights -> fp16 y [M, N]."""
    import torch
    assert x.dtype == torch.float16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    st = load().gemm_w4a16(_ptr(x), M, K, x.stride(0), _ptr(wpacked), _ptr(s0), N, _ptr(y), _stream(stream))
    _check(st, "gemm_w4a16")
    return y


PLAN_FIELDS = ("kind", "mt", "nt", "splitk", "waves", "depth", "xstage", "ws_bytes", "wave_n")
CANDIDATE_FIELDS = ("mt", "nt", "splitk", "waves", "depth", "xstage", "wave_n")


def gemm_w4a8_plan(M: int, N: int, K: int) -> dict:
    """The plan gemm_w4a8 launches for (M, N, K) (host-side query)."""
    desc = (ctypes.c_int64 * 9)()
    _check(load().gemm_w4a8_plan(M, N, K, desc), "gemm_w4a8_plan")
    return dict(zip(PLAN_FIELDS, list(desc)))


def w4a8_hbm_read(buf, sink, *, nbytes=None, stream=None):
    """Stream-read nbytes (default all) of the uint8 device tensor buf once (the streaming-read ceiling)."""
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    _check(load().w4a8_hbm_read(_ptr(buf), n, _ptr(sink), _stream(stream)), "w4a8_hbm_read")


def gemm_w4a8_plan_detail(M: int, N: int, K: int, with_workspace: bool = True) -> dict:
    """The plan gemm_w4a8 launches with a workspace (or with ws = NULL), and its LDS bytes per workgroup."""
    desc = (ctypes.c_int64 * 10)()
    _check(load().gemm_w4a8_plan_detail(M, N, K, int(bool(with_workspace)), desc), "gemm_w4a8_plan_detail")
    return dict(zip(PLAN_FIELDS + ("lds_bytes",), list(desc)))


def gemm_w4a8_decode_candidates(M: int, N: int, K: int) -> list:
    """Every decode-kernel plan that can run (M <= 1024), as tuples (mt, nt, splitk, waves, depth, xstage, wave_n)."""
    n = ctypes.c_int32(0)
    _check(load().gemm_w4a8_decode_candidates(M, N, K, None, 0, ctypes.byref(n)), "gemm_w4a8_decode_candidates")
    buf = (ctypes.c_int32 * (7 * max(1, n.value)))()
    _check(load().gemm_w4a8_decode_candidates(M, N, K, buf, n.value, ctypes.byref(n)), "gemm_w4a8_decode_candidates")
    return [tuple(buf[7 * i:7 * i + 7]) for i in range(n.value)]


def gemm_w4a8_selector_score(M: int, N: int, K: int, plan, cus: int = 256) -> float:
    """The compiled-in selector's predicted HBM fraction for one plan tuple (< 0: no model)."""
    arr = (ctypes.c_int32 * 7)(*[int(v) for v in (tuple(plan) + (0,))[:7]])
    return float(load().gemm_w4a8_selector_score(M, N, K, arr, cus))


def kv4_cache_bytes(B: int, Hkv: int, S: int) -> int:
    """Bytes of one 4-bit cache (keys or values) for B sequences, Hkv heads, S tokens (0: invalid)."""
    return int(load().kv4_cache_bytes(B, Hkv, S))


def kv4_cache_alloc(B: int, Hkv: int, S: int, device=None):
    """A (key, value) pair of uint8 device buffers of kv4_cache_bytes each."""
    import torch
    n = kv4_cache_bytes(B, Hkv, S)
    if n == 0:
        raise W4A8Error(W4A8_E_SHAPE, "kv4_cache_bytes")
    return (torch.empty(n, dtype=torch.uint8, device=device), torch.empty(n, dtype=torch.uint8, device=device))


def quantize_kv4(k, v, pos, k_cache, v_cache, S: int, *, stream=None):
    """New tokens k, v: fp16 [B, T, Hkv, 128]; pos: int32 [B] (first cache index per sequence)."""
    import torch
    assert k.dtype == torch.float16 and v.dtype == torch.float16 and k.shape == v.shape and k.dim() == 4
    assert k.is_contiguous() and v.is_contiguous() and pos.dtype == torch.int32
    B, T, Hkv, D = k.shape
    assert D == 128
    st = load().quantize_kv4(_ptr(k), _ptr(v), B, Hkv, T, _ptr(pos), _ptr(k_cache), _ptr(v_cache), S,
                             _stream(stream))
    _check(st, "quantize_kv4")


def kv4_unpack(cache, is_v: bool, B: int, Hkv: int, S: int, *, stream=None):
    """-> (codes uint8 [B, Hkv, S, 128], scales fp16-bits int16 [B, Hkv, S], zeros uint8 [B, Hkv, S])."""
    import torch
    dev = cache.device
    codes = torch.empty((B, Hkv, S, 128), dtype=torch.uint8, device=dev)
    sc = torch.empty((B, Hkv, S), dtype=torch.int16, device=dev)
    z = torch.empty((B, Hkv, S), dtype=torch.uint8, device=dev)
    st = load().kv4_unpack(_ptr(cache), int(bool(is_v)), B, Hkv, S, _ptr(codes), _ptr(sc), _ptr(z), _stream(stream))
    _check(st, "kv4_unpack")
    return codes, sc, z


def kv4_attention_workspace_bytes(B: int, Hq: int, S: int) -> int:
    return int(load().kv4_attention_workspace_bytes(B, Hq, S))


def attention_kv4_decode(q, k_cache, v_cache, S: int, Hkv: int, lens, sm_scale: float, *, out=None,
                         ws=None, stream=None):
    """q: fp16 [B, Hq, 128]; lens: int32 [B] -> fp16 [B, Hq, 128]."""
    import torch
    assert q.dtype == torch.float16 and q.dim() == 3 and q.is_contiguous() and lens.dtype == torch.int32
    B, Hq, D = q.shape
    assert D == 128
    if out is None:
        out = torch.empty_like(q)
    need = kv4_attention_workspace_bytes(B, Hq, S)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    st = load().attention_kv4_decode(_ptr(q), B, Hq, Hkv, _ptr(k_cache), _ptr(v_cache), S, _ptr(lens),
                                     float(sm_scale), _ptr(out), _ptr(ws), nbytes, _stream(stream))
    _check(st, "attention_kv4_decode")
    return out


def linear(x, wq: dict, *, acc_out=None, stream=None):
    """The serving-time call: quantize the fp16 activations, then the W4A8 GEMM."""
    qx, s_a = quantize_act_per_token_i8(x, stream=stream)
    return gemm_w4a8(qx, s_a, wq["wpacked"], wq["s0"], wq["N"], acc_out=acc_out, stream=stream)
