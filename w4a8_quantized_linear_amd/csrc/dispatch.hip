// dispatch.hip -- shape-keyed choice of GEMM kernel, tile and split-K.
//
// The QFactory reading notes (6.1-6.2) make tile shapes compile-time template
// parameters and pick an instantiation per shape; here the pick is a small
// deterministic rule of (M, N, K), so the workspace size a caller queries and
// the plan gemm_w4a8 launches always agree.  W4A8_DECODE_PLAN="mt,nt,splitk"
// overrides the decode choice (for tuning sweeps).
#include <cstdlib>
#include <cstdio>

#include "w4a8_internal.h"

namespace w4a8 {

size_t decode_lds_bytes(int64_t M, int64_t K, int mt, int nt, int splitk);
hipError_t launch_gemm_decode(const GemmPlan &p, const int8_t *qx, const float *s_a,
                              const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                              int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *ws,
                              hipStream_t st);

namespace {

constexpr int64_t kTargetBlocks = 1024;    // four 4-wave workgroups per CU

size_t ws_size(int64_t M, int64_t N, int splitk, int64_t tiles)
{
    if (splitk <= 1)
        return 0;
    return ((size_t)M * N * 4 + 255) / 256 * 256 + (size_t)tiles * 4;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K)
{
    GemmPlan p{};
    p.kind = 0;
    const int64_t ntiles = N / kTileN;
    const int64_t G = num_groups(K);
    p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
    p.m_blocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.nt = ntiles >= 512 ? 4 : (ntiles >= 128 ? 2 : 1);
    p.n_blocks = (ntiles + p.nt - 1) / p.nt;
    int64_t blocks = p.n_blocks * p.m_blocks;
    int64_t sk = (kTargetBlocks + blocks - 1) / blocks;
    int64_t sk_max = G / 8 > 0 ? G / 8 : 1;          // at least one pair of groups per wave
    if (sk > sk_max)
        sk = sk_max;
    if (sk < 1)
        sk = 1;
    p.splitk = (int)sk;

    if (const char *env = std::getenv("W4A8_DECODE_PLAN")) {
        int mt = 0, nt = 0, s = 0;
        if (std::sscanf(env, "%d,%d,%d", &mt, &nt, &s) == 3 && (mt == 1 || mt == 2 || mt == 4) &&
            (nt == 1 || nt == 2 || nt == 4) && s >= 1 && s <= G) {
            p.mt = mt;
            p.nt = nt;
            p.splitk = s;
            p.m_blocks = (M + 16 * mt - 1) / (16 * mt);
            p.n_blocks = (ntiles + nt - 1) / nt;
        }
    }
    p.ws_bytes = ws_size(M, N, p.splitk, p.m_blocks * p.n_blocks);
    return p;
}

hipError_t launch_gemm(const GemmPlan &p, const int8_t *qx, const float *s_a,
                       const uint8_t *stream_bytes, const uint16_t *s0, int64_t M, int64_t N,
                       int64_t K, uint16_t *y, int32_t *acc_out, void *ws, hipStream_t st)
{
    if (std::getenv("W4A8_LOG"))
        std::fprintf(stderr, "w4a8: gemm M=%lld N=%lld K=%lld kind=%d mt=%d nt=%d splitk=%d grid=%lldx%dx%lld\n",
                     (long long)M, (long long)N, (long long)K, p.kind, p.mt, p.nt, p.splitk,
                     (long long)p.n_blocks, p.splitk, (long long)p.m_blocks);
    return launch_gemm_decode(p, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
}

}  // namespace w4a8
