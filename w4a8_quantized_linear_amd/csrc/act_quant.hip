// act_quant.hip -- per-token INT8 activation quantization for gfx950.
//
// QServe talk summary, "Precision Data Flow and Activation Quantization
// Fusion": every linear layer consumes 8-bit activations.  Per token m:
//   s_a[m]  = max_k |x[m,k]| / 127            (IEEE fp32 division)
//   qx[m,k] = clamp(rint(x[m,k] / s_a[m]), -127, 127)   (0 when s_a == 0)
//
// Layout: W waves per token (W = 4 while few tokens leave waves idle, else
// W = 1), four waves per workgroup.  Each lane keeps R 16-byte chunks of its
// row in registers, so a row of up to 512 R W elements is read from HBM once
// (longer rows re-read their tail from cache); loads are all issued before
// the first use.  The absmax is reduced as 15-bit fp16 magnitudes with
// packed integer max (for finite halves, magnitude bits order like values),
// across lanes with cross-lane moves and across the W waves through LDS.
//
// Division: x / s_a needs one correctly rounded fp32 quotient per element
// (the scale is a/127 by IEEE division, so 1/s_a is not exact).  Every
// element takes t = x * fl(1/s_a), which is within 3 units in the last place
// of the quotient (|t - x/s| <= |x/s| (3u + u^2), u = 2^-24, |x/s| <= 127 +
// 2^-16), i.e. within 2.3e-5 of it.  rint(t) and rint(fl(x/s)) can only
// differ when a half-integer lies between them, so a chunk whose t are all
// farther than 2^-14 from a half-integer is quantized from t; otherwise the
// whole chunk is recomputed with the IEEE division (a chunk takes that path
// with probability ~1e-3 on smooth data, every time on exact ties).
// Memory bound: 3 bytes per element (+4 per token).
//
// The same kernel also runs the normalization that the QServe talk summary
// fuses with this quantizer (same section: the quantization is folded into
// the preceding layer, e.g. LayerNorm, whose output is written as 8 bits).
// Per token, with the row held in registers:
//   LayerNorm: mean = (exact integer sum of the row in units of 2^-24) * 2^-24
//              / K in double; RMSNorm: mean = 0;
//   var  = sum_k (double(x) - mean)^2 / K in double (the lanes' partial sums
//          are added in a tree, so var may differ from a sequential sum in
//          its last bits);
//   rstd = float(1 / sqrt(var + eps)) (0 when var + eps == 0), mean32 =
//          float(mean);
//   h    = fp16(((float(x) - mean32) * rstd) * float(gamma) + float(beta))
// in place of x, then the quantizer above on h.  Extra arithmetic, same
// bytes: 3 per element (+ the gamma and beta rows, read from cache).
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 1 << 22;  // workgroups per launch (slots loop over the rest)
constexpr float kNearTie = 1.0f / 16384; // 2^-14 > the 2.3e-5 bound above

// the normalization in front of the quantizer (unused when it is off)
struct NormArgs {
    const uint16_t *gamma;   // [K] fp16
    const uint16_t *beta;    // [K] fp16, or null
    float eps;
    int rms;                 // 1: RMSNorm (no centering)
};

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

__device__ inline float h2f(uint32_t bits16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// running max of the two 15-bit magnitudes held in each half of a dword
__device__ inline uint32_t chunk_absmax(const uint4 &c, uint32_t a)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    us2 m = __builtin_bit_cast(us2, a);
#pragma unroll
    for (int i = 0; i < 4; i++)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(us2, w[i] & 0x7FFF7FFFu));
    return __builtin_bit_cast(uint32_t, m);
}

// low bytes of four dwords -> one dword
__device__ inline uint32_t pack4(uint32_t q0, uint32_t q1, uint32_t q2, uint32_t q3)
{
    const uint32_t lo = __builtin_amdgcn_perm(q1, q0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(q3, q2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Exact row sums: every finite fp16 value is a multiple of 2^-24 below 2^16,
// so a sum of at most 2^13 of them is a multiple of 2^-24 below 2^29 -- at
// most 53 significant bits, exact in double.  A lane adds at most K / 64 <=
// 128 values (one wave per token, K <= 8192) or K / 256 <= 4096 (four waves
// per token, K <= 2^20), so its double sum is exact; the lanes' sums then go
// through int64 (units of 2^-24), whose tree sum is exact in any order.
// (two accumulators per lane: shorter dependency chains)
__device__ inline void chunk_sum(const uint4 &c, double (&acc)[2])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        acc[0] = acc[0] + (double)h2f(w[i] & 0xFFFFu);
        acc[1] = acc[1] + (double)h2f(w[i] >> 16);
    }
}

// sums of (double(x) - mean)^2 over 8 halves, each product and sum rounded
// (two accumulators per lane)
__device__ inline void chunk_sqdev(const uint4 &c, double mean, double (&acc)[2])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const double d0 = (double)h2f(w[i] & 0xFFFFu) - mean;
        const double d1 = (double)h2f(w[i] >> 16) - mean;
        acc[0] = acc[0] + d0 * d0;
        acc[1] = acc[1] + d1 * d1;
    }
}

// h = fp16(((float(x) - mean32) * rstd) * float(gamma) [+ float(beta)]) on 8
// halves.  Each step is one rounding of an exact result, written as an fma
// so that the half operand converts inside it (v_fma_mix): x * 1 - mean32,
// t * gamma - 0 (the -0 addend keeps the sign of a zero product), beta * 1 +
// t.  `one` and `nzero` are 1 and -0, hidden from the optimizer so that it
// keeps the fmas instead of folding them to a separate convert and add.
__device__ inline uint4 chunk_norm(const uint4 &c, const uint4 &g, const uint4 &b, bool has_beta,
                                   float mean32, float rstd, float one, float nzero)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w}, gw[4] = {g.x, g.y, g.z, g.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        float t[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            t[j] = __builtin_fmaf(h2f((w[i] >> (16 * j)) & 0xFFFFu), one, -mean32);
            t[j] = t[j] * rstd;
            t[j] = __builtin_fmaf(t[j], h2f((gw[i] >> (16 * j)) & 0xFFFFu), nzero);
            if (has_beta)
                t[j] = __builtin_fmaf(h2f((bw[i] >> (16 * j)) & 0xFFFFu), one, t[j]);
        }
        typedef _Float16 h2v __attribute__((ext_vector_type(2)));
        const h2v hv = {(_Float16)t[0], (_Float16)t[1]};
        o[i] = __builtin_bit_cast(uint32_t, hv);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Round-to-nearest-even to an integer by adding 1.5 * 2^23: for |v| < 2^22
// the sum's ulp is 1, so the sum is rint(v) + 1.5 * 2^23 exactly and its low
// byte is rint(v) as a two's-complement int8.
constexpr float kRoundC = 12582912.0f;

// quantize 8 halves; inv = fl(1/s) (0 for an all-zero row, whose s is 0).
// No clamp: |x| <= a and s = fl(a/127) >= (a/127)(1 - 2^-24) bound both
// quotients by 127 + 2^-16, so their rint is within [-127, 127].
__device__ inline uint2 chunk_quant(const uint4 &c, float s, float inv)
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    float x[8], r[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = h2f(w[i] & 0xFFFFu);
        x[2 * i + 1] = h2f(w[i] >> 16);
    }
    // the largest distance of t to its nearest integer (t - rint(t) is exact)
    float dmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        // x * inv as one mixed-precision fma straight from the half (the +0
        // addend changes no rounding and keeps the fma from folding to a mul)
        const float t = __builtin_fmaf(x[i], inv, 0.0f);
        r[i] = t + kRoundC;
        dmax = fmaxf(dmax, fabsf(t - (r[i] - kRoundC)));
    }
    if (__builtin_expect(dmax >= 0.5f - kNearTie, 0)) {
#pragma unroll
        for (int i = 0; i < 8; i++)
            r[i] = x[i] / s + kRoundC;
    }
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
        b[i] = __builtin_bit_cast(uint32_t, r[i]);
    return make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
}

// W waves per token, R register chunks per lane.  Token slots (a wave, or a
// workgroup when W = 4) walk the tokens with a stride of the slot count;
// the next token's row is loaded before the current one is quantized, so
// loads, arithmetic and stores of successive tokens overlap.  Every load is
// unconditional, so the waits for one row never include the next row's
// loads: a lane index past the row is clamped to its last chunk (a repeated
// chunk leaves the absmax unchanged; only its store is skipped), and the
// prefetch after a slot's last token re-reads that token's row from cache.
// Exact: the row is exactly R chunks per lane (no clamping, no tail).
// NORM: normalize the row first (see the top of the file).
template <int W, int R, bool Exact, bool NORM>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(const uint16_t *__restrict__ x,
                                                             int64_t M, int64_t K, int64_t ldx,
                                                             int8_t *__restrict__ qx,
                                                             float *__restrict__ s_a, NormArgs na)
{
    constexpr int L = 64 * W;               // lanes per token
    constexpr int kTok = kThreads / L;      // token slots per workgroup
    const int lane = threadIdx.x % L;
    const int64_t slots = (int64_t)gridDim.x * kTok;
    int64_t m = (int64_t)blockIdx.x * kTok + threadIdx.x / L;
    if (m >= M)
        return;                              // whole slots only (W = 1)
    const int64_t nchunks = K / 8;
    __shared__ uint32_t red[kThreads / 64];
    __shared__ int64_t red64[kThreads / 64];

    auto chunk = [&](int i) -> int64_t {
        const int64_t c = lane + (int64_t)L * i;
        return Exact ? c : std::min<int64_t>(c, nchunks - 1);
    };
    auto load = [&](uint4(&b)[R], int64_t t) {
        const uint4 *row = reinterpret_cast<const uint4 *>(x + t * ldx);
#pragma unroll
        for (int i = 0; i < R; i++)
            b[i] = row[chunk(i)];
        __builtin_amdgcn_sched_barrier(0);   // issue the row's loads before what follows
    };
    // sum over the row's lanes (and the token's W waves) of a 64-bit value
    auto row_sum = [&](auto v) {
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            v += __shfl_xor(v, off, 64);
        if (W > 1) {
            if ((threadIdx.x & 63) == 0)
                red64[threadIdx.x >> 6] = __builtin_bit_cast(int64_t, v);
            __syncthreads();
            decltype(v) total = 0;
#pragma unroll
            for (int u = 0; u < W; u++)   // the same order in every lane
                total += __builtin_bit_cast(decltype(v), red64[(threadIdx.x / L) * W + u]);
            __syncthreads();                 // red64 is rewritten next
            v = total;
        }
        return v;
    };
    const uint4 *gam = reinterpret_cast<const uint4 *>(na.gamma);
    const uint4 *bet = reinterpret_cast<const uint4 *>(na.beta);
    const bool has_beta = NORM && na.beta != nullptr;
    float mean32 = 0.0f, rstd = 0.0f;
    float one = 1.0f, nzero = -0.0f;
    asm volatile("" : "+v"(one), "+v"(nzero));
    // chunk c of the normalized row, from the raw chunk v (gamma and beta
    // are read from cache: every token reads the same rows)
    auto xform = [&](const uint4 &v, int64_t c) -> uint4 {
        if (!NORM)
            return v;
        return chunk_norm(v, gam[c], has_beta ? bet[c] : make_uint4(0, 0, 0, 0), has_beta, mean32, rstd,
                          one, nzero);
    };

    auto opaque = [](uint4(&b)[R]) {
#pragma unroll
        for (int i = 0; i < R; i++)
            asm volatile("" : "+v"(b[i].x), "+v"(b[i].y), "+v"(b[i].z), "+v"(b[i].w));
    };
    auto quantize = [&](uint4(&b)[R], int64_t t) {
        const uint4 *row = reinterpret_cast<const uint4 *>(x + t * ldx);
        if (NORM) {
            // statistics over the row (chunks past it, clamped copies, are skipped)
            double mean = 0.0;
            if (!na.rms) {
                double sl[2] = {0.0, 0.0};
#pragma unroll
                for (int i = 0; i < R; i++)
                    if (Exact || lane + (int64_t)L * i < nchunks)
                        chunk_sum(b[i], sl);
                if (!Exact)
                    for (int64_t c = lane + (int64_t)L * R; c < nchunks; c += L)
                        chunk_sum(row[c], sl);
                // each partial sum is exact; as integers in units of 2^-24 so is their total
                const int64_t S = row_sum((int64_t)__builtin_ldexp(sl[0], 24) + (int64_t)__builtin_ldexp(sl[1], 24));
                mean = __builtin_ldexp((double)S, -24) / (double)K;
            }
            // (the row is made opaque before each pass, so that the compiler
            // converts it again instead of keeping every converted double live
            // from one pass to the next)
            opaque(b);
            double sq[2] = {0.0, 0.0};
#pragma unroll
            for (int i = 0; i < R; i++)
                if (Exact || lane + (int64_t)L * i < nchunks)
                    chunk_sqdev(b[i], mean, sq);
            if (!Exact)
                for (int64_t c = lane + (int64_t)L * R; c < nchunks; c += L)
                    chunk_sqdev(row[c], mean, sq);
            const double ss = row_sum(sq[0] + sq[1]);
            const double ve = ss / (double)K + (double)na.eps;
            rstd = ve == 0.0 ? 0.0f : (float)(1.0 / __builtin_sqrt(ve));
            mean32 = (float)mean;
            opaque(b);
#pragma unroll
            for (int i = 0; i < R; i++)
                b[i] = xform(b[i], chunk(i));
        }
        uint32_t am = 0;
#pragma unroll
        for (int i = 0; i < R; i++)
            am = chunk_absmax(b[i], am);
        if (!Exact)
            for (int64_t c = lane + (int64_t)L * R; c < nchunks; c += L)
                am = chunk_absmax(xform(row[c], c), am);
        am = max(am & 0xFFFFu, am >> 16);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            am = max(am, (uint32_t)__shfl_xor((int)am, off, 64));
        if (W > 1) {
            if ((threadIdx.x & 63) == 0)
                red[threadIdx.x >> 6] = am;
            __syncthreads();
#pragma unroll
            for (int v = 0; v < W; v++)
                am = max(am, red[(threadIdx.x / L) * W + v]);
            __syncthreads();                 // red is rewritten for the next token
        }
        const float a = h2f(am);
        const float s = a / 127.0f;
        const float inv = a == 0.0f ? 0.0f : 1.0f / s;
        if (lane == 0)
            s_a[t] = s;
        uint2 *out = reinterpret_cast<uint2 *>(qx + t * K);
#pragma unroll
        for (int i = 0; i < R; i++) {
            const int64_t c = lane + (int64_t)L * i;
            const uint2 v = chunk_quant(b[i], s, inv);
            if (Exact || c < nchunks)
                out[c] = v;
        }
        if (!Exact)
            for (int64_t c = lane + (int64_t)L * R; c < nchunks; c += L)
                out[c] = chunk_quant(xform(row[c], c), s, inv);
    };

    uint4 A[R], B[R];
    load(A, m);
    while (true) {
        const int64_t m1 = m + slots;
        load(B, m1 < M ? m1 : m);
        quantize(A, m);
        if (m1 >= M)
            break;
        const int64_t m2 = m1 + slots;
        load(A, m2 < M ? m2 : m1);
        quantize(B, m1);
        if (m2 >= M)
            break;
        m = m2;
    }
}

template <int W, int R>
hipError_t launch_wr(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qx,
                     float *s_a, int64_t slots, const NormArgs *na, hipStream_t st)
{
    const int64_t tok = kThreads / (64 * W);
    const int64_t blocks = std::min<int64_t>((slots + tok - 1) / tok, kMaxBlocks);
    const bool exact = K / 8 == (int64_t)64 * W * R;
    const NormArgs a = na ? *na : NormArgs{nullptr, nullptr, 0.0f, 0};
    auto *k = na ? (exact ? act_quant_kernel<W, R, true, true> : act_quant_kernel<W, R, false, true>)
                 : (exact ? act_quant_kernel<W, R, true, false> : act_quant_kernel<W, R, false, false>);
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, st, x, M, K, ldx, qx, s_a, a);
    return hipGetLastError();
}

// register chunks per lane for a row of K halves over W waves (24 at most;
// longer rows read the rest in a second pass from cache)
int regs_for(int64_t K, int W)
{
    const int64_t per_lane = (K / 8 + 64 * W - 1) / (64 * W);
    for (int r : {2, 4, 8, 12, 16})
        if (per_lane <= r)
            return r;
    return 24;
}

template <int W>
hipError_t launch_w(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qx, float *s_a,
                    int64_t slots, const NormArgs *na, hipStream_t st)
{
    switch (regs_for(K, W)) {
    case 2: return launch_wr<W, 2>(x, M, K, ldx, qx, s_a, slots, na, st);
    case 4: return launch_wr<W, 4>(x, M, K, ldx, qx, s_a, slots, na, st);
    case 8: return launch_wr<W, 8>(x, M, K, ldx, qx, s_a, slots, na, st);
    case 12: return launch_wr<W, 12>(x, M, K, ldx, qx, s_a, slots, na, st);
    case 16: return launch_wr<W, 16>(x, M, K, ldx, qx, s_a, slots, na, st);
    default: return launch_wr<W, 24>(x, M, K, ldx, qx, s_a, slots, na, st);
    }
}

hipError_t launch(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qx, float *s_a,
                  const NormArgs *na, hipStream_t st)
{
    if (M == 0)
        return hipSuccess;
    // The plain quantizer: four waves per token, every token its own slot up
    // to 16 slots per compute unit, beyond that each slot walks its tokens with
    // the row prefetch (timed on MI355X: at 4096 tokens four waves per token
    // beat one wave by 10% at K = 4096 and 23% at K = 11008, and were never
    // slower up to 16384 tokens or K = 28672).  The fused normalization keeps
    // one wave per token from 1024 tokens on, unless its rows are too long for
    // one wave's registers; from four tokens per slot on, each slot walks its
    // tokens (two slots per SIMD, one if the two row buffers take more than
    // half its registers).  W4A8_ACT_SLOTS=n overrides the slot count,
    // W4A8_ACT_WAVES=1|4 the waves per token.
    int64_t slots = 0;
    if (const char *env = std::getenv("W4A8_ACT_SLOTS"))
        slots = std::atoll(env);
    const int64_t cus = num_cus();
    // (the normalizing variant holds at most 16 chunks per lane in registers:
    // with 24 its two row buffers no longer fit and go to scratch)
    const bool wide = (K / 8 + 63) / 64 > (na ? 16 : 24);
    int waves = M < 1024 || wide || !na ? 4 : 1;
    if (const char *env = std::getenv("W4A8_ACT_WAVES"))   // 1 or 4 (sweeps; 1 only where it fits)
        waves = std::atoi(env) == 4 || wide ? 4 : (std::atoi(env) == 1 ? 1 : waves);
    if (waves == 4) {
        if (slots <= 0)
            slots = !na ? std::min<int64_t>(M, 16 * cus) : (M >= 4 * cus ? 2 * cus : M);
        return launch_w<4>(x, M, K, ldx, qx, s_a, std::min(slots, M), na, st);
    }
    if (slots <= 0) {
        const int64_t per_simd = regs_for(K, 1) <= 16 ? 2 : 1;
        slots = M >= 4 * per_simd * 4 * cus ? per_simd * 4 * cus : M;
    }
    return launch_w<1>(x, M, K, ldx, qx, s_a, std::min(slots, M), na, st);
}

}  // namespace

hipError_t launch_act_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, int8_t *qx,
                            float *s_a, hipStream_t st)
{
    return launch(x, M, K, ldx, qx, s_a, nullptr, st);
}

hipError_t launch_norm_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                             const uint16_t *gamma, const uint16_t *beta, float eps, int rms,
                             int8_t *qx, float *s_a, hipStream_t st)
{
    const NormArgs na{gamma, beta, eps, rms};
    return launch(x, M, K, ldx, qx, s_a, &na, st);
}

}  // namespace w4a8
