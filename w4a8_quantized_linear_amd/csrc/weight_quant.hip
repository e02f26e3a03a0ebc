// weight_quant.hip -- offline progressive (two-level) weight quantization and
// packing into the device weight stream, plus its inverse for inspection.
//
// QServe talk summary, "Progressive Group Quantization for W4A8 GEMM", and
// Lecture 15 notes, 15.6: level 1 quantizes each output channel to INT8 with
// an fp16 scale inside the protective range [-119, 119]; level 2 quantizes
// each group of 128 INT8 values of a channel to UINT4 with an integer scale
// and a zero point.  The protective range is what makes the later INT4 ->
// INT8 rebuild q4*s1 - z*s1 fit INT8 (QServe talk summary, "Challenges and
// Design Details of QServe GEMM Kernel").
//
//   level 1 (per channel n):  s0 = fp16_rne(absmax / 119)  (fp32 division)
//                             q8 = clamp(rint(w / float(s0)), -119, 119)
//   level 2 (per group):      lo = min(0, min q8), hi = max(0, max q8)
//                             s1 = max(1, ceil((hi - lo) / 15))
//                             z  = rne(-lo / s1)
//                             q4 = clamp(rne(q8 / s1) + z, 0, 15)
//
// One 256-thread workgroup per 16-channel n-tile.  Phase 1 reduces the 16
// channel absmaxes (16 lanes per channel).  Phase 2 walks the groups four at
// a time: each thread quantizes 8 consecutive k of one channel in each of the
// four groups, the 16 lanes of a channel reduce the group range with
// cross-lane moves, the codes land in an LDS staging tile, and each wave then
// assembles one 1024-byte device tile (see w4a8_internal.h for the order)
// and writes it with one 16-byte store per lane.
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kProtect = 119;

// Integer division rounded to nearest, ties to even, for |p| <= 255, 1 <= d <= 16.
__device__ inline int div_rne(int p, int d)
{
    int q = p >= 0 ? p / d : -((d - 1 - p) / d);   // floor(p / d)
    int r = p - q * d;                              // 0 <= r < d
    int twice = 2 * r;
    q += (twice > d) ? 1 : ((twice == d) ? (q & 1) : 0);
    return q;
}

__device__ inline float group16_max(float v)
{
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline int group16_min_i(int v)
{
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
        v = min(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ inline int group16_max_i(int v)
{
#pragma unroll
    for (int off = 8; off > 0; off >>= 1)
        v = max(v, __shfl_xor(v, off, 64));
    return v;
}

__global__ __launch_bounds__(kThreads) void weight_quant_kernel(
    const float *__restrict__ w, int64_t K, uint8_t *__restrict__ codes,
    uint8_t *__restrict__ params, uint8_t *__restrict__ s1_out, uint8_t *__restrict__ z_out,
    uint16_t *__restrict__ s0_out)
{
    __shared__ float s0f[kTileN];
    __shared__ uint8_t q4s[4][kTileN][kGroup];   // four groups of staged codes

    const int64_t nt = blockIdx.x;
    const int tid = threadIdx.x;
    const int r = tid >> 4;          // channel within the tile
    const int j = tid & 15;          // 8-wide k slot within a group
    const int64_t n = nt * kTileN + r;
    const int64_t G = num_groups(K);
    const int64_t G4 = groups_padded(K);
    const float *wrow = w + n * K;

    // ---- level 1: channel absmax -> s0 ------------------------------------
    float a = 0.0f;
    for (int64_t k = 8 * j; k < K; k += 128) {
        float4 v0 = *reinterpret_cast<const float4 *>(wrow + k);
        float4 v1 = *reinterpret_cast<const float4 *>(wrow + k + 4);
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v0.x), fabsf(v0.y)), fmaxf(fabsf(v0.z), fabsf(v0.w))));
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v1.x), fabsf(v1.y)), fmaxf(fabsf(v1.z), fabsf(v1.w))));
    }
    a = group16_max(a);
    if (j == 0) {
        _Float16 h = (_Float16)(a / (float)kProtect);
        s0f[r] = (float)h;
        s0_out[n] = __builtin_bit_cast(uint16_t, h);
    }
    __syncthreads();
    const float s0 = s0f[r];

    // ---- level 2, four groups per pass ------------------------------------
    for (int64_t gb = 0; gb < G4; gb += 4) {
        uint32_t pbytes = 0;
#pragma unroll
        for (int gg = 0; gg < 4; gg++) {
            const int64_t g = gb + gg;
            if (g < G) {
                const float *src = wrow + g * kGroup + 8 * j;
                float4 v0 = *reinterpret_cast<const float4 *>(src);
                float4 v1 = *reinterpret_cast<const float4 *>(src + 4);
                const float vals[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                int q8[8];
                int lo = 0, hi = 0;
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    float q = 0.0f;
                    if (s0 != 0.0f)
                        q = fminf(fmaxf(__builtin_rintf(vals[i] / s0), -(float)kProtect),
                                  (float)kProtect);
                    q8[i] = (int)q;
                    lo = min(lo, q8[i]);
                    hi = max(hi, q8[i]);
                }
                lo = group16_min_i(lo);
                hi = group16_max_i(hi);
                const int D = hi - lo;
                const int s1 = max(1, (D + 14) / 15);
                const int z = div_rne(-lo, s1);
#pragma unroll
                for (int i = 0; i < 8; i++)
                    q4s[gg][r][8 * j + i] = (uint8_t)min(15, max(0, div_rne(q8[i], s1) + z));
                pbytes |= (uint32_t)((s1 - 1) | (z << 4)) << (8 * gg);
                if (j == 0 && s1_out != nullptr) {
                    s1_out[n * G + g] = (uint8_t)s1;
                    z_out[n * G + g] = (uint8_t)z;
                }
            }
        }
        // one dword of parameters per channel per four groups (padding groups are 0)
        if (j == 0)
            *reinterpret_cast<uint32_t *>(params + param_index(n, gb, G4)) = pbytes;
        __syncthreads();

        // wave w assembles the device tile of group gb + w
        const int wv = tid >> 6;
        const int l = tid & 63;
        const int64_t g = gb + wv;
        if (g < G) {
            const int cn = l & 15;
            const int kb = l >> 4;
            uint32_t out[4];
#pragma unroll
            for (int d = 0; d < 4; d++) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; b++) {
                    uint32_t lo4 = q4s[wv][cn][16 * kb + 4 * d + b];
                    uint32_t hi4 = q4s[wv][cn][64 + 16 * kb + 4 * d + b];
                    v |= (lo4 | (hi4 << 4)) << (8 * b);
                }
                out[d] = v;
            }
            uint4 *dst = reinterpret_cast<uint4 *>(codes + (nt * G + g) * kTileBytes) + l;
            *dst = make_uint4(out[0], out[1], out[2], out[3]);
        }
        __syncthreads();
    }
}

// Inverse of the packing: one 64-lane slot per (n-tile, group) tile.
__global__ __launch_bounds__(kThreads) void weight_unpack_kernel(
    const uint8_t *__restrict__ codes, const uint8_t *__restrict__ params, int64_t N, int64_t K,
    uint8_t *__restrict__ q4c, uint8_t *__restrict__ s1_out, uint8_t *__restrict__ z_out)
{
    const int64_t G = num_groups(K);
    const int64_t G4 = groups_padded(K);
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= (N / kTileN) * G)
        return;
    const int l = threadIdx.x & 63;
    const int64_t nt = tile / G;
    const int64_t g = tile % G;
    const int64_t n = nt * kTileN + (l & 15);
    const int kb = l >> 4;
    const uint4 v = reinterpret_cast<const uint4 *>(codes + tile * kTileBytes)[l];
    const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
    // canonical byte (n, k/2): even k in the low nibble
#pragma unroll
    for (int d = 0; d < 4; d++) {
#pragma unroll
        for (int b = 0; b < 4; b += 2) {
            uint32_t e0 = (dw[d] >> (8 * b)) & 0xFF;
            uint32_t e1 = (dw[d] >> (8 * b + 8)) & 0xFF;
            uint32_t cl = (e0 & 0xF) | ((e1 & 0xF) << 4);
            uint32_t ch = (e0 >> 4) | (e1 & 0xF0);
            int idx = 2 * d + b / 2;          // 0..7 within the 8 canonical bytes
            lo[idx / 4] |= cl << (8 * (idx & 3));
            hi[idx / 4] |= ch << (8 * (idx & 3));
        }
    }
    uint8_t *row = q4c + n * (K / 2);
    *reinterpret_cast<uint2 *>(row + (g * kGroup + 16 * kb) / 2) = make_uint2(lo[0], lo[1]);
    *reinterpret_cast<uint2 *>(row + (g * kGroup + 64 + 16 * kb) / 2) = make_uint2(hi[0], hi[1]);
    if (kb == 0) {
        uint32_t p = params[param_index(n, g, G4)];
        s1_out[n * G + g] = (uint8_t)((p & 15) + 1);
        z_out[n * G + g] = (uint8_t)(p >> 4);
    }
}

}  // namespace

hipError_t launch_weight_quant(const float *w, int64_t N, int64_t K, uint8_t *stream_bytes,
                               uint8_t *s1, uint8_t *z, uint16_t *s0, hipStream_t st)
{
    uint8_t *codes = stream_bytes;
    uint8_t *params = stream_bytes + code_bytes(N, K);
    hipLaunchKernelGGL(weight_quant_kernel, dim3((unsigned)(N / kTileN)), dim3(kThreads), 0, st,
                       w, K, codes, params, s1, z, s0);
    return hipGetLastError();
}

hipError_t launch_weight_unpack(const uint8_t *stream_bytes, int64_t N, int64_t K,
                                uint8_t *q4_canon, uint8_t *s1, uint8_t *z, hipStream_t st)
{
    const int64_t tiles = (N / kTileN) * num_groups(K);
    hipLaunchKernelGGL(weight_unpack_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(kThreads), 0,
                       st, stream_bytes, stream_bytes + code_bytes(N, K), N, K, q4_canon, s1, z);
    return hipGetLastError();
}

}  // namespace w4a8
