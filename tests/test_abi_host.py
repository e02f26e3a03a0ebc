"""Host-only checks of libw4a8: it loads, exports every entry point the header
declares, reports sizes, and rejects bad arguments before launching anything.

No test here makes a compute call: every call below fails host-side
validation.  They are skipped where a GPU is visible (the same checks run in
the CPU suite), so a regression in validation can never launch a kernel on
fake pointers.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")


@pytest.fixture(scope="module")
def lib():
    from w4a8_quantized_linear_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from w4a8_quantized_linear_amd import build
        build.build(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("quantize_weights_w4g128", "quantize_act_per_token_i8", "gemm_w4a8"):
        assert n in names
    from w4a8_quantized_linear_amd import _lib
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    from w4a8_quantized_linear_amd import _lib
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if " T " in l)
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings_and_version(lib):
    from w4a8_quantized_linear_amd import _lib
    for st in (0, -1, -2, -3, -4, -5, 7):
        assert len(_lib.status_string(st)) > 0
    assert re.match(r"^\d+\.\d+\.\d+$", _lib.version())


def test_size_queries(lib):
    from w4a8_quantized_linear_amd import _lib
    # codes + one parameter byte per (channel, group), groups padded to a multiple of 4
    assert _lib.w4a8_packed_weight_bytes(512, 512) == 512 * 256 + 512 * 4
    assert _lib.w4a8_packed_weight_bytes(4096, 11008) == 4096 * 5504 + 4096 * 88
    assert _lib.w4a8_packed_weight_bytes(16, 128) == 16 * 64 + 16 * 4
    for N, K in ((0, 128), (16, 0), (15, 128), (16, 100), (-16, 128)):
        assert _lib.w4a8_packed_weight_bytes(N, K) == 0
    assert _lib.gemm_w4a8_workspace_bytes(0, 512, 512) == 0
    assert _lib.gemm_w4a8_workspace_bytes(1, 15, 512) == 0
    # the fixed rules run these decode shapes unsplit; with the learned selector
    # the size query still agrees with the plan it picks
    import os
    from w4a8_quantized_linear_amd import gemm_w4a8_plan
    os.environ["W4A8_SELECTOR"] = "0"
    try:
        for (M, N, K) in ((1, 4096, 4096), (32, 22016, 4096)):
            assert _lib.gemm_w4a8_workspace_bytes(M, N, K) == 0
    finally:
        del os.environ["W4A8_SELECTOR"]
    for (M, N, K) in ((1, 4096, 4096), (32, 22016, 4096), (64, 22016, 4096)):
        assert _lib.gemm_w4a8_workspace_bytes(M, N, K) == gemm_w4a8_plan(M, N, K)["ws_bytes"]
    if not _gpu_visible():   # the planner assumes 256 CUs when no device is present
        # M=512, K=11008, N=4096: long K and 8 x 16 tiles of 64 x 256 fill half
        # the CUs -> 256 stream-K ranges: the fixed 64 KB of counters, then two
        # 64 x 256 INT32 partial slots per range
        assert _lib.gemm_w4a8_workspace_bytes(512, 4096, 11008) == 65536 + 2 * 256 * 64 * 256 * 4
        # K=4096 (32 groups): one workgroup per tile, no workspace
        assert _lib.gemm_w4a8_workspace_bytes(4096, 11008, 4096) == 0
        assert _lib.gemm_w4a8_workspace_bytes(256, 11008, 4096) == 0


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


needs_no_gpu = pytest.mark.skipif(_gpu_visible(), reason="validation checks use fake pointers; run on the CPU host only")

A = ctypes.c_void_p(0x10000)      # 16-byte aligned fake pointers (never dereferenced)
B = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x30008)    # misaligned
NUL = None
S = ctypes.c_void_p(0)


@needs_no_gpu
def test_quantize_weights_validation(lib):
    f = lib.quantize_weights_w4g128
    assert f(NUL, 16, 128, A, A, A, A, S) == -1
    assert f(A, 16, 128, NUL, A, A, A, S) == -1
    assert f(A, 16, 128, A, A, NUL, A, S) == -1           # s1 without z
    assert f(A, 16, 128, A, A, A, NUL, S) == -1
    assert f(A, 16, 100, A, NUL, NUL, A, S) == -2
    assert f(A, 20, 128, A, NUL, NUL, A, S) == -2
    assert f(A, 0, 128, A, NUL, NUL, A, S) == -2
    assert f(A, 16, -128, A, NUL, NUL, A, S) == -2
    assert f(MIS, 16, 128, A, NUL, NUL, A, S) == -3
    assert f(A, 16, 128, MIS, NUL, NUL, A, S) == -3


@needs_no_gpu
def test_unpack_validation(lib):
    f = lib.w4a8_unpack_weights
    assert f(NUL, 16, 128, A, A, A, S) == -1
    assert f(A, 16, 128, A, NUL, A, S) == -1
    assert f(A, 16, 127, A, A, A, S) == -2
    assert f(A, 16, 128, MIS, A, A, S) == -3


@needs_no_gpu
def test_act_quant_validation(lib):
    f = lib.quantize_act_per_token_i8
    assert f(A, 0, 128, 128, A, A, S) == 0                 # M == 0 is a no-op
    assert f(NUL, 0, 128, 128, NUL, NUL, S) == 0
    assert f(A, -1, 128, 128, A, A, S) == -2
    assert f(A, 4, 100, 100, A, A, S) == -2
    assert f(A, 4, 128, 64, A, A, S) == -2                 # ldx < K
    assert f(A, 4, 128, 130, A, A, S) == -2                # ldx not a multiple of 8
    assert f(NUL, 4, 128, 128, A, A, S) == -1
    assert f(A, 4, 128, 128, NUL, A, S) == -1
    assert f(A, 4, 128, 128, A, NUL, S) == -1
    assert f(MIS, 4, 128, 128, A, A, S) == -3
    assert f(A, 4, 128, 128, A, MIS, S) == -3


@needs_no_gpu
def test_norm_quant_validation(lib):
    f = lib.norm_quantize_act_i8

    def call(x=A, M=4, K=128, ldx=128, g=A, b=NUL, eps=1e-5, rms=0, qx=A, sa=B):
        return f(x, M, K, ldx, g, b, eps, rms, qx, sa, S)

    assert call(M=0) == 0 and call(M=0, x=NUL, g=NUL, qx=NUL, sa=NUL) == 0
    assert call(M=-1) == -2
    assert call(K=100, ldx=100) == -2
    assert call(ldx=64) == -2
    assert call(ldx=130) == -2
    assert call(K=(1 << 20) + 128, ldx=(1 << 20) + 128) == -2     # exact row sum would leave 64 bits
    assert call(eps=-1.0) == -2
    assert call(eps=float("nan")) == -2
    assert call(eps=float("inf")) == -2
    assert call(rms=2) == -2
    assert call(x=NUL) == -1
    assert call(g=NUL) == -1
    assert call(qx=NUL) == -1
    assert call(sa=NUL) == -1
    assert call(x=MIS) == -3
    assert call(g=MIS) == -3
    assert call(b=MIS) == -3
    assert call(sa=MIS) == -3


@needs_no_gpu
def test_w4a16_validation(lib):
    f = lib.gemm_w4a16

    def call(x=A, M=4, K=128, ldx=128, w=A, s0=A, N=16, y=B):
        return f(x, M, K, ldx, w, s0, N, y, S)

    assert call(M=0) == 0 and call(M=0, x=NUL, y=NUL) == 0
    assert call(M=-1) == -2
    assert call(K=100, ldx=100) == -2
    assert call(N=24) == -2
    assert call(ldx=64) == -2
    assert call(ldx=132) == -2
    assert call(x=NUL) == -1
    assert call(w=NUL) == -1
    assert call(s0=NUL) == -1
    assert call(y=NUL) == -1
    assert call(x=MIS) == -3
    assert call(w=MIS) == -3
    assert call(y=MIS) == -3


@needs_no_gpu
def test_kv4_validation(lib):
    assert lib.kv4_cache_bytes(2, 4, 64) == 2 * 4 * 64 * 68
    assert lib.kv4_cache_bytes(2, 4, 48) == 0 and lib.kv4_cache_bytes(0, 4, 64) == 0
    assert lib.kv4_attention_workspace_bytes(2, 8, 256) == 0            # one chunk: no partial sums
    assert lib.kv4_attention_workspace_bytes(2, 8, 512) == 2 * 8 * 2 * 130 * 4
    assert lib.kv4_attention_workspace_bytes(2, 8, 100) == 0

    def quant(k=A, v=A, Bn=2, H=4, T=1, pos=A, kc=B, vc=B, Sc=64):
        return lib.quantize_kv4(k, v, Bn, H, T, pos, kc, vc, Sc, S)

    assert quant(T=0) == 0 and quant(T=0, k=NUL) == 0
    assert quant(Sc=40) == -2 and quant(T=-1) == -2 and quant(H=0) == -2
    assert quant(k=NUL) == -1 and quant(pos=NUL) == -1 and quant(vc=NUL) == -1
    assert quant(k=MIS) == -3 and quant(kc=MIS) == -3

    def unpack(c=A, isv=0, Bn=2, H=4, Sc=64, codes=B, sc=B, z=B):
        return lib.kv4_unpack(c, isv, Bn, H, Sc, codes, sc, z, S)

    assert unpack(isv=2) == -2 and unpack(Sc=33) == -2
    assert unpack(c=NUL) == -1 and unpack(z=NUL) == -1
    assert unpack(c=MIS) == -3

    def attn(q=A, Bn=2, Hq=8, H=4, kc=A, vc=A, Sc=512, lens=A, sm=0.088, out=B, ws=B, wsb=1 << 20):
        return lib.attention_kv4_decode(q, Bn, Hq, H, kc, vc, Sc, lens, sm, out, ws, wsb, S)

    assert attn(Hq=6) == -2                    # Hq not a multiple of Hkv
    assert attn(Hq=4 * 17) == -2               # more than 16 query heads per kv head
    assert attn(Sc=500) == -2 and attn(sm=0.0) == -2 and attn(sm=float("nan")) == -2
    assert attn(q=NUL) == -1 and attn(lens=NUL) == -1 and attn(out=NUL) == -1
    assert attn(q=MIS) == -3 and attn(kc=MIS) == -3
    assert attn(ws=NUL, wsb=0) == -4           # two chunks need partial sums
    assert attn(wsb=100) == -4


@needs_no_gpu
def test_gemm_validation(lib, monkeypatch):
    f = lib.gemm_w4a8
    ok = dict(qx=A, sa=A, w=A, s0=A, M=1, N=16, K=128, y=B, acc=NUL, ws=NUL, wsb=0)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["qx"], a["sa"], a["w"], a["s0"], a["M"], a["N"], a["K"], a["y"], a["acc"],
                 a["ws"], a["wsb"], S)

    assert call(M=0, qx=NUL, y=NUL) == 0
    assert call(M=-1) == -2
    assert call(N=0) == -2
    assert call(N=24) == -2
    assert call(K=192) == -2
    assert call(K=1 << 23) == -2
    assert call(qx=NUL) == -1
    assert call(sa=NUL) == -1
    assert call(w=NUL) == -1
    assert call(s0=NUL) == -1
    assert call(y=NUL) == -1
    assert call(qx=MIS) == -3
    assert call(y=MIS) == -3
    assert call(acc=MIS) == -3
    # a split-K plan with too small a workspace (a NULL workspace is allowed:
    # the call then runs unsplit)
    from w4a8_quantized_linear_amd import _lib
    monkeypatch.setenv("W4A8_DECODE_PLAN", "1,1,4")
    need = _lib.gemm_w4a8_workspace_bytes(1, 4096, 4096)
    assert need > 0
    assert call(N=4096, K=4096, ws=A, wsb=need - 1) == -4
    # a stream-K prefill plan: the same rule
    monkeypatch.delenv("W4A8_DECODE_PLAN")
    monkeypatch.setenv("W4A8_PREFILL_P", "64")
    monkeypatch.setenv("W4A8_PREFILL_TM", "8")
    need = _lib.gemm_w4a8_workspace_bytes(4096, 4096, 4096)
    assert need > 64 * 2 * 128 * 256 * 4
    assert call(M=4096, N=4096, K=4096, ws=A, wsb=need - 1) == -4
    # TM = 16 tiles are never split (no stream-K there): no workspace
    monkeypatch.setenv("W4A8_PREFILL_TM", "16")
    assert _lib.gemm_w4a8_workspace_bytes(4096, 4096, 4096) == 0


def test_gemm_noalloc_validation(lib):
    f = lib.gemm_w4a8_noalloc
    ok = dict(qx=A, sa=A, w=A, s0=A, M=1, N=16, K=128, y=B, acc=NUL)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["qx"], a["sa"], a["w"], a["s0"], a["M"], a["N"], a["K"], a["y"], a["acc"], S)

    assert call(M=0, qx=NUL, y=NUL) == 0
    assert call(M=-1) == -2
    assert call(N=24) == -2
    assert call(K=1 << 23) == -2
    assert call(qx=NUL) == -1
    assert call(y=NUL) == -1
    assert call(y=MIS) == -3
    assert call(acc=MIS) == -3
    # a plan whose workspace exceeds the fixed scratch is rejected before launch
    from w4a8_quantized_linear_amd import _lib
    assert _lib.gemm_w4a8_workspace_bytes(512, 8192, 28672) > _lib.NOALLOC_SCRATCH_BYTES
    assert call(M=512, N=8192, K=28672) == -6
    assert "scratch" in _lib.status_string(-6)


CONFIG_KN = [(512, 512), (4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096), (4096, 11008),
             (8192, 10240), (8192, 57344), (28672, 8192)]


@pytest.mark.parametrize("K,N", CONFIG_KN)
def test_every_plan_fits_its_lds_with_and_without_workspace(lib, K, N):
    """For every config shape at 1..128 tokens (and a few more token counts
    up to 4096), the plan gemm_w4a8 launches with a workspace and the one it
    launches with ws == NULL both request LDS within the kernel's limit, and
    the NULL-workspace plan needs no workspace.  (An unsplit N-split plan at
    K = 28672 once asked for 137 KB, over the 128 KB decode limit.)"""
    from w4a8_quantized_linear_amd import _lib
    for M in list(range(1, 129)) + [136, 160, 200, 256, 257, 320, 384, 511, 512, 513, 768, 1024, 1025, 4096]:
        for with_ws in (True, False):
            d = _lib.gemm_w4a8_plan_detail(M, N, K, with_ws)
            limit = 160 * 1024 if d["kind"] == 1 else 128 * 1024
            assert 0 < d["lds_bytes"] <= limit, (M, with_ws, d)
            if not with_ws:
                assert d["ws_bytes"] == 0 and d["splitk"] in (0, 1), (M, d)
            else:
                assert d == dict(_lib.gemm_w4a8_plan(M, N, K), lds_bytes=d["lds_bytes"])


@pytest.mark.parametrize("M,K,N,kind", [
    (64, 4096, 11008, 0), (128, 11008, 4096, 0), (128, 4096, 22016, 1),
    (129, 11008, 4096, 0), (256, 11008, 4096, 0), (256, 4096, 2048, 0), (192, 13824, 5120, 0),
    (224, 13824, 5120, 1), (257, 11008, 4096, 1), (160, 28672, 8192, 1), (256, 4096, 11008, 1),
    (160, 8192, 6144, 0), (165, 16512, 5760, 1), (136, 9984, 7296, 1),
    (72, 8192, 10240, 0), (122, 19584, 8448, 1), (100, 27776, 8448, 1), (111, 12544, 9344, 1),
    (111, 6656, 14592, 0), (229, 2176, 5376, 0), (131, 2048, 12544, 0), (160, 4096, 12288, 1),
    (256, 4096, 8192, 0), (257, 2048, 4096, 0), (384, 8192, 2048, 0), (512, 4096, 1024, 0),
    (512, 4096, 4096, 0), (512, 11008, 4096, 1), (320, 4096, 4096, 0), (513, 4096, 1024, 0),
    (448, 28672, 2048, 0), (256, 28672, 2048, 0), (1024, 4096, 1024, 0), (1024, 28672, 1024, 0),
    (768, 8192, 2048, 1), (640, 4096, 2048, 0), (1025, 4096, 512, 1), (389, 27264, 2688, 1)])
def test_token_count_routes(lib, M, K, N, kind):
    """gemm_w4a8 takes the decode kernels up to 64 tokens; up to 128 while
    the 64 x 256 many-token tiles would fill under half of the CUs and the
    weights are not very large (N x K <= 3 x 2^25, or four-m-tile workgroups
    fit one round on the CUs); and up to 256 on layers with at most 2^20
    outputs (M x N) whose weights are small (N x K <= 2^26) or whose
    four-m-tile workgroups fit one round, or with at most 2^21 outputs and
    N x K <= 2^25 (up to 1024 tokens; past 256 tokens N x K <= 2^25, past
    512 N x K <= 2^23, unless four-m-tile workgroups fit one round).  The
    rest goes to the matrix-core kernel."""
    from w4a8_quantized_linear_amd import _lib
    p = _lib.gemm_w4a8_plan(M, N, K)
    assert p["kind"] == kind, (M, K, N, p)


@pytest.mark.parametrize("M,K,N,plan", [
    (129, 11008, 4096, (4, 4, 1, 4, 0, 0)), (256, 11008, 4096, (4, 4, 1, 4, 0, 0)),
    (256, 2048, 4096, (2, 4, 1, 4, 1, 1)), (192, 13824, 5120, (4, 4, 1, 4, 0, 0)),
    (200, 4096, 1024, (2, 2, 1, 4, 0, 0)), (160, 4096, 768, (1, 2, 1, 8, 1, 0)),
    (160, 12288, 768, (1, 2, 1, 8, 0, 0)), (200, 28672, 2048, (4, 4, 2, 4, 0, 0)),
    (160, 28672, 2048, (2, 4, 4, 4, 1, 1)), (160, 8192, 6144, (2, 4, 1, 4, 0, 0)),
    (232, 4096, 4096, (2, 4, 1, 4, 1, 1)), (252, 24192, 1152, (2, 4, 4, 4, 1, 1)),
    (100, 1152, 272, (1, 1, 1, 8, 0, 0)), (80, 4096, 1536, (1, 2, 1, 4, 0, 0)), (100, 8192, 768, (1, 2, 1, 4, 0, 0)),
    (128, 2048, 2048, (2, 2, 1, 8, 1, 0)), (96, 11008, 4096, (2, 4, 1, 4, 0, 0)), (96, 4096, 11008, (4, 4, 1, 4, 1, 1)),
    (72, 8192, 10240, (2, 4, 1, 4, 0, 0)), (112, 28672, 8192, (4, 4, 1, 4, 0, 0)),
    (128, 11008, 8448, (4, 8, 2, 4, 1, 1)), (448, 28672, 2048, (4, 4, 1, 4, 0, 0)),
    (1012, 18176, 512, (4, 4, 1, 4, 0, 0))])
def test_wide_decode_plan_rule(lib, M, K, N, plan):
    """Past 64 tokens the decode plan comes from fixed trees, one for 65..128
    tokens and one for 129..256 (the learned selector, trained on 1..64
    tokens, is not consulted): (m-tiles, n-tiles, split-K, waves, staged,
    waves splitting N) for shapes on each branch."""
    from w4a8_quantized_linear_amd import _lib
    p = _lib.gemm_w4a8_plan(M, N, K)
    assert p["kind"] == 0 and (p["mt"], p["nt"], p["splitk"], p["waves"], p["xstage"], p["wave_n"]) == plan, p


def test_decode_plan_override_forces_the_decode_kernels(lib, monkeypatch):
    """W4A8_DECODE_PLAN runs the named decode plan at any M <= 1024, also on
    shapes the dispatcher would send to the matrix-core kernel (tuning
    sweeps time decode plans there); past 1024 tokens it is ignored, and a
    plan no kernel variant implements still selects the decode kernels, with
    the dispatcher's own decode plan."""
    from w4a8_quantized_linear_amd import _lib
    assert _lib.gemm_w4a8_plan(165, 5760, 16512)["kind"] == 1
    monkeypatch.setenv("W4A8_DECODE_PLAN", "4,4,1,4,2,0,0")
    p = _lib.gemm_w4a8_plan(165, 5760, 16512)
    assert p["kind"] == 0 and (p["mt"], p["nt"], p["splitk"]) == (4, 4, 1), p
    assert _lib.gemm_w4a8_plan(4096, 11008, 4096)["kind"] == 1
    monkeypatch.setenv("W4A8_DECODE_PLAN", "3,4,1,4,2,0,0")
    assert _lib.gemm_w4a8_plan(165, 5760, 16512)["kind"] == 0


def test_gemm_k_limit(lib):
    from w4a8_quantized_linear_amd import _lib
    assert _lib.gemm_w4a8_workspace_bytes(1, 16, 1 << 23) == 0
    desc = (ctypes.c_int64 * 10)()
    assert lib.gemm_w4a8_plan_detail(1, 16, 1 << 23, 1, desc) == -2
    assert lib.gemm_w4a8_plan_detail(1, 16, 1 << 22, 2, desc) == -2
    # the longest K still plans a launchable kernel, with or without workspace
    for with_ws in (True, False):
        d = _lib.gemm_w4a8_plan_detail(1, 16, 1 << 22, with_ws)
        assert 0 < d["lds_bytes"] <= 160 * 1024


def test_binding_raises_without_library(monkeypatch, tmp_path):
    from w4a8_quantized_linear_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()
