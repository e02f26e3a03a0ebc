// api.hip -- the C ABI of libw4a8 (declared in include/w4a8.h): argument
// checks on the host, then launches on the caller's stream.  Every argument
// error is reported before anything is enqueued; nothing here allocates.
#include <cstdint>
#include <mutex>

#include "w4a8.h"
#include "w4a8_internal.h"

using namespace w4a8;

namespace {

constexpr int64_t kMaxM = (int64_t)65535 * 64;   // grid z limit of the GEMM (64 tokens per block)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The GEMM addresses the weight stream with 32-bit buffer offsets.
bool weight_shape_ok(int64_t N, int64_t K)
{
    return N > 0 && K > 0 && K % kGroup == 0 && N % kTileN == 0 && N <= ((int64_t)1 << 30) &&
           K <= ((int64_t)1 << 24) && code_bytes(N, K) + param_bytes(N, K) <= 0x7FFFFFFF;
}

// The GEMM also bounds K (kGemmMaxK) for its 32-bit activation offsets.
bool gemm_shape_ok(int64_t N, int64_t K) { return weight_shape_ok(N, K) && K <= kGemmMaxK; }

w4a8_status hip_status(hipError_t e) { return e == hipSuccess ? W4A8_OK : W4A8_E_HIP; }

}  // namespace

extern "C" {

const char *w4a8_status_string(w4a8_status st)
{
    switch (st) {
    case W4A8_OK: return "ok";
    case W4A8_E_NULL: return "a required pointer is NULL";
    case W4A8_E_SHAPE: return "invalid shape (need M >= 0, N > 0, K > 0, K % 128 == 0, N % 16 == 0, ldx >= K, ldx % 8 == 0)";
    case W4A8_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case W4A8_E_WORKSPACE: return "workspace missing or smaller than the *_workspace_bytes() size";
    case W4A8_E_HIP: return "HIP launch or runtime error";
    case W4A8_E_SCRATCH: return "the call needs more workspace than gemm_w4a8_noalloc's fixed scratch holds "
                                "(W4A8_NOALLOC_SCRATCH_BYTES); call gemm_w4a8 with a workspace";
    }
    return "unknown status";
}

const char *w4a8_version(void) { return "0.1.0"; }

size_t w4a8_packed_weight_bytes(int64_t N, int64_t K)
{
    if (!weight_shape_ok(N, K))
        return 0;
    return (size_t)(code_bytes(N, K) + param_bytes(N, K));
}

w4a8_status quantize_weights_w4g128(const float *w, int64_t N, int64_t K, void *wpacked,
                                    uint8_t *s1, uint8_t *z, uint16_t *s0_fp16,
                                    hipStream_t stream)
{
    if (!w || !wpacked || !s0_fp16 || ((s1 == nullptr) != (z == nullptr)))
        return W4A8_E_NULL;
    if (!weight_shape_ok(N, K))
        return W4A8_E_SHAPE;
    if (!aligned16(w) || !aligned16(wpacked) || !aligned16(s0_fp16) ||
        (s1 && (!aligned16(s1) || !aligned16(z))))
        return W4A8_E_ALIGN;
    return hip_status(launch_weight_quant(w, N, K, static_cast<uint8_t *>(wpacked), s1, z,
                                          s0_fp16, stream));
}

w4a8_status w4a8_unpack_weights(const void *wpacked, int64_t N, int64_t K, uint8_t *q4_canon,
                                uint8_t *s1, uint8_t *z, hipStream_t stream)
{
    if (!wpacked || !q4_canon || !s1 || !z)
        return W4A8_E_NULL;
    if (!weight_shape_ok(N, K))
        return W4A8_E_SHAPE;
    if (!aligned16(wpacked) || !aligned16(q4_canon) || !aligned16(s1) || !aligned16(z))
        return W4A8_E_ALIGN;
    return hip_status(launch_weight_unpack(static_cast<const uint8_t *>(wpacked), N, K, q4_canon,
                                           s1, z, stream));
}

w4a8_status quantize_act_per_token_i8(const uint16_t *x_fp16, int64_t M, int64_t K, int64_t ldx,
                                      int8_t *qx, float *s_a, hipStream_t stream)
{
    if (M < 0 || K <= 0 || K % kGroup != 0 || ldx < K || ldx % 8 != 0 || M > ((int64_t)1 << 31) - 1)
        return W4A8_E_SHAPE;
    if (M == 0)
        return W4A8_OK;
    if (!x_fp16 || !qx || !s_a)
        return W4A8_E_NULL;
    if (!aligned16(x_fp16) || !aligned16(qx) || !aligned16(s_a))
        return W4A8_E_ALIGN;
    return hip_status(launch_act_quant(x_fp16, M, K, ldx, qx, s_a, stream));
}

w4a8_status norm_quantize_act_i8(const uint16_t *x_fp16, int64_t M, int64_t K, int64_t ldx,
                                 const uint16_t *gamma_fp16, const uint16_t *beta_fp16, float eps,
                                 int rms, int8_t *qx, float *s_a, hipStream_t stream)
{
    if (M < 0 || K <= 0 || K % kGroup != 0 || K > ((int64_t)1 << 20) || ldx < K || ldx % 8 != 0 ||
        M > ((int64_t)1 << 31) - 1 || !(eps >= 0.0f && eps <= 3.4e38f) || (rms != 0 && rms != 1))
        return W4A8_E_SHAPE;
    if (M == 0)
        return W4A8_OK;
    if (!x_fp16 || !gamma_fp16 || !qx || !s_a)
        return W4A8_E_NULL;
    if (!aligned16(x_fp16) || !aligned16(gamma_fp16) || (beta_fp16 && !aligned16(beta_fp16)) ||
        !aligned16(qx) || !aligned16(s_a))
        return W4A8_E_ALIGN;
    return hip_status(launch_norm_quant(x_fp16, M, K, ldx, gamma_fp16, beta_fp16, eps, rms, qx, s_a,
                                        stream));
}

w4a8_status gemm_w4a16(const uint16_t *x_fp16, int64_t M, int64_t K, int64_t ldx,
                       const void *wpacked, const uint16_t *s0_fp16, int64_t N, uint16_t *y_fp16,
                       hipStream_t stream)
{
    if (M < 0 || M > ((int64_t)1 << 31) - 1 || !weight_shape_ok(N, K) || ldx < K || ldx % 8 != 0)
        return W4A8_E_SHAPE;
    if (M == 0)
        return W4A8_OK;
    if (!x_fp16 || !wpacked || !s0_fp16 || !y_fp16)
        return W4A8_E_NULL;
    if (!aligned16(x_fp16) || !aligned16(wpacked) || !aligned16(s0_fp16) || !aligned16(y_fp16))
        return W4A8_E_ALIGN;
    return hip_status(launch_gemm_w4a16(x_fp16, M, K, ldx, static_cast<const uint8_t *>(wpacked),
                                        s0_fp16, N, y_fp16, stream));
}

// KV cache shapes: head_dim 128; S a multiple of 32; B * Hkv and B * Hq
// within the grid's x range; the 8-token blocks of one call within y.
static bool kv_shape_ok(int64_t B, int64_t Hkv, int64_t S)
{
    return B > 0 && Hkv > 0 && S > 0 && S % 32 == 0 && B * Hkv <= ((int64_t)1 << 31) - 1 &&
           S <= ((int64_t)1 << 24) && kv4_buffer_bytes(B, Hkv, S) <= ((int64_t)1 << 46);
}

size_t kv4_cache_bytes(int64_t B, int64_t Hkv, int64_t S)
{
    return kv_shape_ok(B, Hkv, S) ? (size_t)kv4_buffer_bytes(B, Hkv, S) : 0;
}

w4a8_status quantize_kv4(const uint16_t *k_fp16, const uint16_t *v_fp16, int64_t B, int64_t Hkv, int64_t T,
                         const int32_t *pos, void *k_cache, void *v_cache, int64_t S, hipStream_t stream)
{
    if (!kv_shape_ok(B, Hkv, S) || T < 0 || T > ((int64_t)1 << 19))
        return W4A8_E_SHAPE;
    if (T == 0)
        return W4A8_OK;
    if (!k_fp16 || !v_fp16 || !pos || !k_cache || !v_cache)
        return W4A8_E_NULL;
    if (!aligned16(k_fp16) || !aligned16(v_fp16) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(pos) & 3u))
        return W4A8_E_ALIGN;
    return hip_status(launch_kv4_quant(k_fp16, v_fp16, B, Hkv, T, pos, static_cast<uint8_t *>(k_cache),
                                       static_cast<uint8_t *>(v_cache), S, stream));
}

w4a8_status kv4_unpack(const void *cache, int is_v, int64_t B, int64_t Hkv, int64_t S, uint8_t *codes,
                       uint16_t *scales_fp16, uint8_t *zeros, hipStream_t stream)
{
    if (!kv_shape_ok(B, Hkv, S) || (is_v != 0 && is_v != 1) || B * Hkv * S > ((int64_t)1 << 32))
        return W4A8_E_SHAPE;
    if (!cache || !codes || !scales_fp16 || !zeros)
        return W4A8_E_NULL;
    if (!aligned16(cache) || !aligned16(codes) || (reinterpret_cast<uintptr_t>(scales_fp16) & 1u))
        return W4A8_E_ALIGN;
    return hip_status(launch_kv4_unpack(static_cast<const uint8_t *>(cache), is_v, B, Hkv, S, codes,
                                        scales_fp16, zeros, stream));
}

size_t kv4_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t S)
{
    if (B <= 0 || Hq <= 0 || S <= 0 || S % 32 != 0 || S > ((int64_t)1 << 24))
        return 0;
    const int64_t ns = kv4_splits(S);
    return ns <= 1 ? 0 : (size_t)(B * Hq * ns * (kKvHeadDim + 2) * 4);
}

w4a8_status attention_kv4_decode(const uint16_t *q_fp16, int64_t B, int64_t Hq, int64_t Hkv, const void *k_cache,
                                 const void *v_cache, int64_t S, const int32_t *lens, float sm_scale,
                                 uint16_t *out_fp16, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!kv_shape_ok(B, Hkv, S) || Hq <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16 ||
        B * Hq > ((int64_t)1 << 31) - 1 || kv4_splits(S) > 65535)
        return W4A8_E_SHAPE;
    if (!(sm_scale > 0.0f) || sm_scale > 1e30f)
        return W4A8_E_SHAPE;
    if (!q_fp16 || !k_cache || !v_cache || !lens || !out_fp16)
        return W4A8_E_NULL;
    if (!aligned16(q_fp16) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out_fp16) ||
        (reinterpret_cast<uintptr_t>(lens) & 3u) || (ws && !aligned16(ws)))
        return W4A8_E_ALIGN;
    const size_t need = kv4_attention_workspace_bytes(B, Hq, S);
    if (need > 0 && (ws == nullptr || ws_bytes < need))
        return W4A8_E_WORKSPACE;
    return hip_status(launch_kv4_attention(q_fp16, B, Hq, Hkv, static_cast<const uint8_t *>(k_cache),
                                           static_cast<const uint8_t *>(v_cache), S, lens, sm_scale, out_fp16,
                                           ws, stream));
}

w4a8_status gemm_w4a8_plan_detail(int64_t M, int64_t N, int64_t K, int with_workspace, int64_t *desc)
{
    if (!desc)
        return W4A8_E_NULL;
    if (M <= 0 || M > kMaxM || !gemm_shape_ok(N, K) || (with_workspace != 0 && with_workspace != 1))
        return W4A8_E_SHAPE;
    GemmPlan p = plan_gemm(M, N, K);
    if (!with_workspace && p.ws_bytes > 0)
        p = plan_without_workspace(p, M, N, K);
    const int64_t d[10] = {p.kind, p.mt, p.nt, p.splitk, p.waves, p.depth, p.xstage ? 1 : 0, (int64_t)p.ws_bytes,
                           p.wave_n, (int64_t)plan_lds_bytes(p, M, N, K)};
    for (int i = 0; i < 10; i++)
        desc[i] = d[i];
    return W4A8_OK;
}

w4a8_status gemm_w4a8_plan(int64_t M, int64_t N, int64_t K, int64_t *desc)
{
    if (!desc)
        return W4A8_E_NULL;
    int64_t d[10];
    const w4a8_status st = gemm_w4a8_plan_detail(M, N, K, 1, d);
    if (st != W4A8_OK)
        return st;
    for (int i = 0; i < 9; i++)
        desc[i] = d[i];
    return W4A8_OK;
}

w4a8_status gemm_w4a8_decode_candidates(int64_t M, int64_t N, int64_t K, int32_t *plans, int32_t max_plans,
                                        int32_t *count)
{
    if (!count || (max_plans > 0 && !plans))
        return W4A8_E_NULL;
    if (M <= 0 || M > kDecodeMaxM || max_plans < 0 || !gemm_shape_ok(N, K))
        return W4A8_E_SHAPE;
    GemmPlan cand[256];
    const int n = decode_candidates(M, N, K, cand, 256);
    *count = n;
    for (int i = 0; i < n && i < max_plans && i < 256; i++) {
        const int32_t row[7] = {cand[i].mt, cand[i].nt, cand[i].splitk, cand[i].waves, cand[i].depth,
                                cand[i].xstage ? 1 : 0, cand[i].wave_n};
        for (int j = 0; j < 7; j++)
            plans[7 * i + j] = row[j];
    }
    return W4A8_OK;
}

float gemm_w4a8_selector_score(int64_t M, int64_t N, int64_t K, const int32_t *plan, int64_t cus)
{
    if (!plan || M <= 0 || M > kDecodeMaxM || !gemm_shape_ok(N, K) || cus <= 0)
        return -1.0f;
    GemmPlan p{};
    p.mt = plan[0];
    p.nt = plan[1];
    p.splitk = plan[2];
    p.waves = plan[3];
    p.depth = plan[4];
    p.xstage = plan[5] != 0;
    p.wave_n = plan[6];
    if (p.mt <= 0 || p.nt <= 0 || p.splitk <= 0 || p.waves <= 0 || p.depth <= 0 || p.wave_n < 0 || p.wave_n > 1)
        return -1.0f;
    p.m_blocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.n_blocks = (N / kTileN + p.nt - 1) / p.nt;
    float x[kSelFeatures];
    selector_features(p, M, N, K, cus, x);
    return selector_predict(x);
}

size_t gemm_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || M > kMaxM || !gemm_shape_ok(N, K))
        return 0;
    return plan_gemm(M, N, K).ws_bytes;
}

}  // extern "C"

namespace {

// Argument checks shared by gemm_w4a8 and gemm_w4a8_noalloc, in the order
// the header documents (shape, then M == 0 as a no-op, then pointers).
// Returns W4A8_OK with *noop set for M == 0.
w4a8_status gemm_args(const int8_t *qx, const float *s_a, const void *wpacked, const uint16_t *s0_fp16,
                      int64_t M, int64_t N, int64_t K, const uint16_t *y_fp16, const int32_t *acc_out,
                      const void *ws, bool *noop)
{
    *noop = false;
    if (M < 0 || M > kMaxM || !gemm_shape_ok(N, K))
        return W4A8_E_SHAPE;
    if (M == 0) {
        *noop = true;
        return W4A8_OK;
    }
    if (!qx || !s_a || !wpacked || !s0_fp16 || !y_fp16)
        return W4A8_E_NULL;
    if (!aligned16(qx) || !aligned16(s_a) || !aligned16(wpacked) || !aligned16(s0_fp16) ||
        !aligned16(y_fp16) || (acc_out && !aligned16(acc_out)) || (ws && !aligned16(ws)))
        return W4A8_E_ALIGN;
    return W4A8_OK;
}

// ---- the workspace of gemm_w4a8_noalloc -------------------------------------
// A fixed array in device memory, one copy per device the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not a device address: its address on the current device comes
// from hipGetSymbolAddress, once per device, and only that pointer is passed
// to kernels.  The array's arrival counters (the first kWsCounters dwords)
// must be zero before the first GEMM that splits K; every GEMM leaves them
// zero again, and the partial slots after them are scratch.
static_assert(W4A8_NOALLOC_SCRATCH_BYTES % 256 == 0 && W4A8_NOALLOC_SCRATCH_BYTES > kWsPartOffset,
              "scratch holds the counters and partial slots");

}  // namespace

static __device__ __align__(256) uint8_t scratch[W4A8_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void clear_counters_kernel(uint32_t *cnt, int n)
{
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n)
        cnt[i] = 0u;
}

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`.  The first call on a device
// looks it up (hipGetSymbolAddress, return code checked) and clears the
// counters with a fill kernel on `st` (a kernel, so that a caller capturing
// `st` into a graph records no memset).
hipError_t noalloc_scratch(void **ptr, hipStream_t st)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0)
            return hipErrorInvalidSymbol;
        hipLaunchKernelGGL(clear_counters_kernel, dim3((unsigned)(kWsCounters / 256)), dim3(256), 0, st,
                           static_cast<uint32_t *>(p), (int)kWsCounters);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

w4a8_status gemm_w4a8_noalloc(const int8_t *qx, const float *s_a, const void *wpacked, const uint16_t *s0_fp16,
                              int64_t M, int64_t N, int64_t K, uint16_t *y_fp16, int32_t *acc_out,
                              hipStream_t stream)
{
    bool noop = false;
    const w4a8_status st = gemm_args(qx, s_a, wpacked, s0_fp16, M, N, K, y_fp16, acc_out, nullptr, &noop);
    if (st != W4A8_OK || noop)
        return st;
    const GemmPlan p = plan_gemm(M, N, K);
    if (p.ws_bytes > (size_t)W4A8_NOALLOC_SCRATCH_BYTES)
        return W4A8_E_SCRATCH;
    void *ws = nullptr;
    if (p.ws_bytes > 0 && noalloc_scratch(&ws, stream) != hipSuccess)
        return W4A8_E_HIP;
    return hip_status(launch_gemm(p, qx, s_a, static_cast<const uint8_t *>(wpacked), s0_fp16, M, N, K, y_fp16,
                                  acc_out, ws, stream));
}

w4a8_status gemm_w4a8(const int8_t *qx, const float *s_a, const void *wpacked,
                      const uint16_t *s0_fp16, int64_t M, int64_t N, int64_t K, uint16_t *y_fp16,
                      int32_t *acc_out, void *ws, size_t ws_bytes, hipStream_t stream)
{
    bool noop = false;
    const w4a8_status st = gemm_args(qx, s_a, wpacked, s0_fp16, M, N, K, y_fp16, acc_out, ws, &noop);
    if (st != W4A8_OK || noop)
        return st;
    GemmPlan p = plan_gemm(M, N, K);
    if (p.ws_bytes > 0 && ws == nullptr)
        p = plan_without_workspace(p, M, N, K);
    if (p.ws_bytes > 0 && ws_bytes < p.ws_bytes)
        return W4A8_E_WORKSPACE;
    return hip_status(launch_gemm(p, qx, s_a, static_cast<const uint8_t *>(wpacked), s0_fp16, M,
                                  N, K, y_fp16, acc_out, ws, stream));
}

}  // extern "C"
