// w4a8_internal.h -- layout constants and launcher declarations shared by the
// HIP translation units of libw4a8 (private to the library).
//
// Device weight stream (written by quantize_weights_w4g128, read by the GEMM):
//
//   [ codes: N*K/2 bytes ][ group parameters: N * G4 bytes ]
//
// Codes.  The weight matrix is cut into tiles of 16 output channels x 128 k
// (one quantization group), 1024 bytes each, stored n-tile major:
//   tile (nt, g) at byte (nt * G + g) * 1024.
// Inside a tile, lane l of a 64-wide wave owns bytes [16 l, 16 l + 16): the 32
// codes of channel n = 16 nt + (l & 15) that the two 16x16x64 INT8 MFMA
// fragments of that lane need, for k-block kb = l >> 4.  Byte b of dword d
// holds, in its low nibble, the code of k = 128 g + 16 kb + 4 d + b (first
// 64-k half of the group) and, in its high nibble, the code of
// k = 128 g + 64 + 16 kb + 4 d + b (second half).  So one 16-byte load per
// lane is one MFMA B-fragment pair, `x & 0x0F0F0F0F` is the first fragment's
// dword and `(x >> 4) & 0x0F0F0F0F` the second's.  This is the
// compute-aware reordering of the QServe talk summary ("Challenges and
// Design Details of QServe GEMM Kernel") redone for the gfx950 MFMA operand
// shape: the weights sit in HBM in exactly the order each lane consumes them.
//
// Group parameters.  One byte per (n, g): (s1 - 1) | (z << 4).  G is padded
// to G4 = round_up(G, 4) and the bytes of four consecutive groups of one
// channel form one dword:
//   byte ((nt * (G4/4) + g/4) * 16 + (n & 15)) * 4 + (g & 3).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>

namespace w4a8 {

constexpr int kGroup = 128;
constexpr int kTileN = 16;
constexpr int kTileBytes = 1024;

__host__ __device__ inline int64_t num_groups(int64_t K) { return K / kGroup; }
__host__ __device__ inline int64_t groups_padded(int64_t K) { return (K / kGroup + 3) / 4 * 4; }
__host__ __device__ inline int64_t code_bytes(int64_t N, int64_t K) { return N * K / 2; }
__host__ __device__ inline int64_t param_bytes(int64_t N, int64_t K) { return N * groups_padded(K); }
__host__ __device__ inline int64_t param_index(int64_t n, int64_t g, int64_t G4)
{
    return ((n / 16 * (G4 / 4) + g / 4) * 16 + (n & 15)) * 4 + (g & 3);
}

// ---- launchers (defined in the kernel translation units) ----------------
hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                            int8_t *qx, float *s_a, hipStream_t st);
hipError_t launch_norm_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                             const uint16_t *gamma, const uint16_t *beta, float eps, int rms,
                             int8_t *qx, float *s_a, hipStream_t st);

hipError_t launch_gemm_w4a16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                             const uint8_t *stream_bytes, const uint16_t *s0, int64_t N, uint16_t *y,
                             hipStream_t st);

hipError_t launch_weight_quant(const float *w, int64_t N, int64_t K, uint8_t *stream_bytes,
                               uint8_t *s1, uint8_t *z, uint16_t *s0, hipStream_t st);

hipError_t launch_weight_unpack(const uint8_t *stream_bytes, int64_t N, int64_t K,
                                uint8_t *q4_canon, uint8_t *s1, uint8_t *z, hipStream_t st);

// 4-bit KV cache (kv4_attention.hip).  One buffer for K and one for V, each
// [ codes: B*Hkv*S rows x 64 bytes ][ params: B*Hkv*S dwords ], row
// (b, g, t) = (b * Hkv + g) * S + t, S the capacity in tokens (a multiple of
// 32).  The code layouts are described in kv4_attention.hip.
constexpr int kKvHeadDim = 128;
constexpr int kKvRowBytes = 64;
#ifndef KV4_CHUNK
#define KV4_CHUNK 256
#endif
constexpr int kKvChunk = KV4_CHUNK;    // tokens per attention workgroup
__host__ __device__ inline int64_t kv4_code_bytes(int64_t B, int64_t Hkv, int64_t S) { return B * Hkv * S * kKvRowBytes; }
__host__ __device__ inline int64_t kv4_buffer_bytes(int64_t B, int64_t Hkv, int64_t S) { return B * Hkv * S * (kKvRowBytes + 4); }
__host__ __device__ inline int64_t kv4_splits(int64_t S) { return (S + kKvChunk - 1) / kKvChunk; }
// Chunks per attention workgroup: enough workgroups for the chip (about
// kKvTargetWgs) with as few split runs per sequence as that allows, at most
// 16 chunks per run.
#ifndef KV4_TARGET_WGS
#define KV4_TARGET_WGS 4096
#endif
constexpr int64_t kKvTargetWgs = KV4_TARGET_WGS;
inline int kv4_chunks_per_run(int64_t pairs, int64_t S)
{
    const int64_t nch = kv4_splits(S);
    int64_t cps = nch * pairs / kKvTargetWgs;
    return (int)std::max<int64_t>(1, std::min<int64_t>(cps, 16));
}

hipError_t launch_kv4_quant(const uint16_t *k, const uint16_t *v, int64_t B, int64_t Hkv, int64_t T,
                            const int32_t *pos, uint8_t *k_cache, uint8_t *v_cache, int64_t S, hipStream_t st);
hipError_t launch_kv4_unpack(const uint8_t *cache, int is_v, int64_t B, int64_t Hkv, int64_t S, uint8_t *codes,
                             uint16_t *s, uint8_t *z, hipStream_t st);
hipError_t launch_kv4_attention(const uint16_t *q, int64_t B, int64_t Hq, int64_t Hkv, const uint8_t *k_cache,
                                const uint8_t *v_cache, int64_t S, const int32_t *lens, float sm_scale,
                                uint16_t *out, void *ws, hipStream_t st);

// GEMM workspace (split-K of decode shapes, stream-K of prefill shapes).  One
// fixed layout for every call, so that calls of different shapes may share a
// buffer: kWsCounters arrival counters at the front (the only part that must
// be zero between calls; every call leaves them zero), then partial-sum
// slots from kWsPartOffset on, which are scratch (written before they are
// read, never assumed zero).  Plans with more output tiles than counters run
// unsplit.
constexpr int64_t kWsCounters = 16384;
constexpr int64_t kWsPartOffset = kWsCounters * 4;

// GEMM plan: which kernel, its tile shape and the split-K factor.
struct GemmPlan {
    int kind;        // 0 = decode (weights streamed, split-K), 1 = prefill (matrix-core tiles)
    int mt;          // 16-row m-tiles per workgroup (decode); TM, 16-row tiles per wave (prefill)
    int nt;          // 16-column n-tiles per workgroup (decode)
    int splitk;      // decode: K slices across workgroups; prefill: stream-K ranges (0: one
                     // workgroup per tile)
    int waves;       // waves per workgroup, splitting the slice (decode)
    int depth;       // pairs of groups in flight per wave (decode)
    bool xstage;     // activation rows staged in LDS (decode, few tokens)
    int wave_n;      // decode kernel: 0 waves split K (gemm_decode.hip); 1 waves split the
                     // n-tiles, activations in LDS windows (gemm_decode_ns.hip)
    int64_t m_blocks;
    int64_t n_blocks;
    size_t ws_bytes; // workspace needed (0 if none)
};

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K);

// Decode plans that can run (M, N, K): every instantiated decode variant with
// every split-K count in {1, 2, 4, 8} the K groups allow, whose LDS fits in
// kDecodeLdsMax.  Writes at most max plans, returns how many there are.
int decode_candidates(int64_t M, int64_t N, int64_t K, GemmPlan *out, int max);
bool decode_ns_variant_exists(int mt, int ntw, int depth);
size_t decode_ns_lds_bytes(const GemmPlan &p, int64_t K);
hipError_t launch_gemm_decode_ns(const GemmPlan &p, const int8_t *qx, const float *s_a, const uint8_t *stream_bytes,
                                 const uint16_t *s0, int64_t M, int64_t N, int64_t K, uint16_t *y, int32_t *acc_out,
                                 void *ws, hipStream_t st);
// Largest dynamic LDS a decode plan may take.  A workgroup can hold 160 KB,
// but a launch asking for all of it is refused, and plans that large leave
// one workgroup per compute unit anyway.
constexpr size_t kDecodeLdsMax = 128 * 1024;
// the decode kernels take up to this many tokens (plan_gemm decides from 65 on)
constexpr int64_t kDecodeMaxM = 1024;

// Learned plan selector (selector.hip): the QFactory reading notes (6.2) rank
// kernel configurations by a small MLP's predicted memory-bandwidth
// utilization, from the matrix shape and the tiling parameters.
constexpr int kSelFeatures = 13;
constexpr float kSelMargin = 0.0f;
void selector_features(const GemmPlan &p, int64_t M, int64_t N, int64_t K, int64_t cus, float *x);
float selector_predict(const float *x);      // predicted fraction of HBM peak; < 0: no model
bool selector_enabled();
bool selector_knows_wave_n(int wave_n);   // the model was trained on plans of this kernel

// compute units of the current device (256 when it cannot be queried)
int64_t num_cus();

// The same computation without a workspace (no split-K, no stream-K): the
// plan itself with its K unsplit when that still fits its LDS, else the
// best-scored unsplit decode candidate, else the many-token kernel.
GemmPlan plan_without_workspace(GemmPlan p, int64_t M, int64_t N, int64_t K);

// Dynamic LDS bytes per workgroup that launching the plan requests.
size_t plan_lds_bytes(const GemmPlan &p, int64_t M, int64_t N, int64_t K);

// Raise a kernel's dynamic-LDS limit on the current device to `bytes`, once
// per (kernel, device); safe to call from several host threads.
hipError_t raise_lds_limit(const void *kernel, int bytes);

// Largest K the GEMM accepts: the many-token kernel addresses a block of
// activation rows with 32-bit offsets, and needs at least two blocks of its
// largest tile (512 rows) within them.
constexpr int64_t kGemmMaxK = (int64_t)1 << 22;

hipError_t launch_gemm(const GemmPlan &p, const int8_t *qx, const float *s_a,
                       const uint8_t *stream_bytes, const uint16_t *s0, int64_t M, int64_t N,
                       int64_t K, uint16_t *y, int32_t *acc_out, void *ws, hipStream_t st);

}  // namespace w4a8
