// Host-only driver of the C ABI for the sanitizer build (test infrastructure).
// Exercises every entry point's argument checks and the host-side planning
// (plans with and without workspace, decode candidates, selector scores) over
// the configuration shapes and edge shapes.  No call launches a kernel: the
// pointers are fake and every compute call fails validation first.  Exit
// status 0 when every expectation holds; the sanitizers abort on any error.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "w4a8.h"

static int failures = 0;
#define EXPECT(cond)                                                          \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
            failures++;                                                       \
        }                                                                     \
    } while (0)

int main()
{
    void *A = reinterpret_cast<void *>(0x10000), *B = reinterpret_cast<void *>(0x20000);
    void *MIS = reinterpret_cast<void *>(0x30008);
    hipStream_t S = nullptr;
    for (int st = -7; st <= 1; st++)
        EXPECT(w4a8_status_string((w4a8_status)st) != nullptr);
    EXPECT(w4a8_version() != nullptr);

    const int64_t kn[][2] = {{512, 512},   {4096, 12288}, {4096, 4096},  {4096, 22016}, {11008, 4096},
                             {4096, 11008}, {8192, 10240}, {8192, 57344}, {28672, 8192}, {128, 16},
                             {384, 48},     {1 << 22, 16}};
    const int64_t ms[] = {1, 2, 5, 8, 16, 17, 24, 32, 33, 48, 64, 65, 96, 256, 512, 768, 4096, 70000};
    std::vector<int32_t> cand(7 * 256);
    for (const auto &p : kn) {
        const int64_t K = p[0], N = p[1];
        EXPECT(w4a8_packed_weight_bytes(N, K) > 0);
        for (int64_t M : ms) {
            int64_t d1[10], d0[10], d9[9];
            EXPECT(gemm_w4a8_plan_detail(M, N, K, 1, d1) == W4A8_OK);
            EXPECT(gemm_w4a8_plan_detail(M, N, K, 0, d0) == W4A8_OK);
            EXPECT(gemm_w4a8_plan(M, N, K, d9) == W4A8_OK);
            EXPECT(d0[7] == 0 && d1[9] > 0 && d0[9] > 0 && d1[9] <= 160 * 1024 && d0[9] <= 160 * 1024);
            EXPECT((size_t)d1[7] == gemm_w4a8_workspace_bytes(M, N, K));
            if (M <= 64) {
                int32_t count = 0;
                EXPECT(gemm_w4a8_decode_candidates(M, N, K, cand.data(), 256, &count) == W4A8_OK);
                // with very long K no decode plan fits its LDS; the plan is then the many-token kernel
                EXPECT(count >= 0 && count <= 256 && (count > 0 || d1[0] == 1));
                for (int i = 0; i < count && i < 256; i++) {
                    const float u = gemm_w4a8_selector_score(M, N, K, &cand[7 * i], 256);
                    EXPECT(u >= 0.0f && u <= 1.0f);
                }
            }
            // compute calls that fail validation before any launch
            EXPECT(gemm_w4a8((const int8_t *)A, (const float *)A, A, (const uint16_t *)A, M, N, K, nullptr, nullptr,
                             nullptr, 0, S) == W4A8_E_NULL);
            EXPECT(gemm_w4a8_noalloc((const int8_t *)MIS, (const float *)A, A, (const uint16_t *)A, M, N, K,
                                     (uint16_t *)B, nullptr, S) == W4A8_E_ALIGN);
            if (d1[7] > 0)
                EXPECT(gemm_w4a8((const int8_t *)A, (const float *)A, A, (const uint16_t *)A, M, N, K, (uint16_t *)B,
                                 nullptr, B, (size_t)d1[7] - 1, S) == W4A8_E_WORKSPACE);
        }
    }
    // shapes the ABI rejects
    int64_t d[10];
    EXPECT(gemm_w4a8_plan_detail(1, 16, (int64_t)1 << 23, 1, d) == W4A8_E_SHAPE);
    EXPECT(gemm_w4a8_plan_detail(0, 16, 128, 1, d) == W4A8_E_SHAPE);
    EXPECT(gemm_w4a8_plan_detail(1, 24, 128, 1, d) == W4A8_E_SHAPE);
    EXPECT(gemm_w4a8_plan_detail(1, 16, 128, 1, nullptr) == W4A8_E_NULL);
    EXPECT(gemm_w4a8_workspace_bytes(1, 16, 192) == 0);
    EXPECT(w4a8_packed_weight_bytes(16, 100) == 0);
    EXPECT(quantize_act_per_token_i8((const uint16_t *)A, 4, 128, 64, (int8_t *)B, (float *)B, S) == W4A8_E_SHAPE);
    EXPECT(quantize_act_per_token_i8(nullptr, 4, 128, 128, (int8_t *)B, (float *)B, S) == W4A8_E_NULL);
    EXPECT(norm_quantize_act_i8((const uint16_t *)A, 4, 128, 128, (const uint16_t *)A, nullptr, -1.0f, 0, (int8_t *)B,
                                (float *)B, S) == W4A8_E_SHAPE);
    EXPECT(gemm_w4a16((const uint16_t *)MIS, 4, 128, 128, A, (const uint16_t *)A, 16, (uint16_t *)B, S) ==
           W4A8_E_ALIGN);
    EXPECT(quantize_weights_w4g128(nullptr, 16, 128, A, nullptr, nullptr, (uint16_t *)A, S) == W4A8_E_NULL);
    EXPECT(w4a8_unpack_weights(A, 16, 100, (uint8_t *)B, (uint8_t *)B, (uint8_t *)B, S) == W4A8_E_SHAPE);
    EXPECT(kv4_cache_bytes(2, 8, 4096) > 0 && kv4_cache_bytes(2, 8, 100) == 0);
    EXPECT(kv4_attention_workspace_bytes(2, 32, 4096) > 0);
    EXPECT(quantize_kv4((const uint16_t *)A, (const uint16_t *)A, 2, 8, 1, nullptr, B, B, 4096, S) == W4A8_E_NULL);
    EXPECT(attention_kv4_decode((const uint16_t *)A, 2, 32, 8, A, A, 4096, (const int32_t *)A, 0.1f, (uint16_t *)B,
                                nullptr, 0, S) == W4A8_E_WORKSPACE);
    EXPECT(w4a8_hbm_read(A, 100, (uint32_t *)B, S) == W4A8_E_SHAPE);
    EXPECT(w4a8_hbm_read(MIS, 1024, (uint32_t *)B, S) == W4A8_E_ALIGN);
    std::printf("abi driver: %d failures\n", failures);
    return failures == 0 ? 0 : 1;
}
