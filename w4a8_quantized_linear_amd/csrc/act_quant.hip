// act_quant.hip -- per-token INT8 activation quantization for gfx950.
//
// QServe talk summary, "Precision Data Flow and Activation Quantization
// Fusion": every linear layer consumes 8-bit activations.  Per token m:
//   s_a[m]  = max_k |x[m,k]| / 127            (IEEE fp32 division)
//   qx[m,k] = clamp(rint(x[m,k] / s_a[m]), -127, 127)   (0 when s_a == 0)
//
// One 256-thread workgroup per token.  The row is read once from HBM with
// 16-byte loads and held in registers (up to 32768 elements per row; longer
// rows re-read their tail), reduced to the absmax in-wave with cross-lane
// moves and across the four waves through LDS, then quantized from the
// registers and written with 8-byte stores.  Memory bound: 3 bytes per
// element (+4 per token).
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kRegChunks = 16;   // 16-byte chunks (8 halves) kept per thread

__device__ inline float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

__device__ inline float chunk_absmax(const uint4 &c, float a)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        a = fmaxf(a, fabsf(h2f(w[i] & 0xFFFFu)));
        a = fmaxf(a, fabsf(h2f(w[i] >> 16)));
    }
    return a;
}

__device__ inline int quant1(float x, float s, bool zero)
{
    if (zero)
        return 0;
    float q = __builtin_rintf(x / s);
    q = fminf(fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

__device__ inline uint2 chunk_quant(const uint4 &c, float s, bool zero)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t out[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t lo = (uint32_t)(quant1(h2f(w[i] & 0xFFFFu), s, zero)) & 0xFFu;
        uint32_t hi = (uint32_t)(quant1(h2f(w[i] >> 16), s, zero)) & 0xFFu;
        out[i / 2] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    return make_uint2(out[0], out[1]);
}

__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                             int64_t K, int64_t ldx,
                                                             int8_t *__restrict__ qx,
                                                             float *__restrict__ s_a)
{
    __shared__ float red[kThreads / 64];
    const int64_t m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint4 *row = reinterpret_cast<const uint4 *>(x + m * ldx);
    const int64_t nchunks = K / 8;

    uint4 buf[kRegChunks];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < kRegChunks; i++) {
        int64_t c = tid + (int64_t)i * kThreads;
        if (c < nchunks) {
            buf[i] = row[c];
            a = chunk_absmax(buf[i], a);
        }
    }
    for (int64_t c = tid + (int64_t)kRegChunks * kThreads; c < nchunks; c += kThreads)
        a = chunk_absmax(row[c], a);

    // in-wave reduction, then across the waves
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        a = fmaxf(a, __shfl_xor(a, off, 64));
    if ((tid & 63) == 0)
        red[tid >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    const float s = a / 127.0f;
    const bool zero = (a == 0.0f);
    if (tid == 0)
        s_a[m] = s;

    uint2 *out = reinterpret_cast<uint2 *>(qx + m * K);
#pragma unroll
    for (int i = 0; i < kRegChunks; i++) {
        int64_t c = tid + (int64_t)i * kThreads;
        if (c < nchunks)
            out[c] = chunk_quant(buf[i], s, zero);
    }
    for (int64_t c = tid + (int64_t)kRegChunks * kThreads; c < nchunks; c += kThreads)
        out[c] = chunk_quant(row[c], s, zero);
}

}  // namespace

hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qx,
                            float *s_a, hipStream_t st)
{
    if (M == 0)
        return hipSuccess;
    hipLaunchKernelGGL(act_quant_kernel, dim3((unsigned)M), dim3(kThreads), 0, st, x, K, ldx, qx,
                       s_a);
    return hipGetLastError();
}

}  // namespace w4a8
