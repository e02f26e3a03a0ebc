// kv4_attention.hip -- the 4-bit KV cache and decode attention over it, gfx950.
//
// The QServe talk summary stores keys and values in 4 bits ("Smooth Attention
// for K4V4 KV Cache Compression") and speeds up the attention kernel over
// that cache with a cheap INT4 -> FP16 conversion, simple control flow and
// prefetched zero points and scales ("Attention Computation Acceleration");
// those factors are per cached token ("Long Context Challenges": they grow
// with the sequence).  Lecture 15 notes (15.6) add that the kernel reads the
// int4 cache directly and never writes it back at higher precision.  Each
// (token, head) row of 128 values is stored as UINT4 codes with an fp16 scale
// and an integer zero point, x ~ (code - zero) * scale (QFactory notes, 2.1).
//
// Three kernels:
//  * kv4_quant_kernel: quantizes new tokens' K and V rows and writes them into
//    the cache at per-sequence positions (rounding rules as the weights'
//    level 2: the range includes 0, scale = fp16(range / 15), zero and codes
//    by fp32 IEEE division and rint, clamped to [0, 15]);
//  * kv4_attn_kernel: one workgroup per (sequence, kv head, chunk of 256
//    tokens), for all the query heads of that kv head (grouped-query
//    attention: up to 16 query heads share one kv head);
//  * kv4_combine_kernel: merges the chunks' partial softmax sums.
//
// Attention arithmetic.  Scores are s_t * sum_d q_d (code_td - zero_t): the
// fp16 operand (code - zero) is exact, every q * (code - zero) is exact in
// fp32, the sums run on v_mfma_f32_16x16x32_f16 and the token's scale (with
// sm_scale * log2 e) multiplies the sum.  p_t = exp2(score - chunk max).  The
// value side folds the token's scale into the probability operand,
// P'_t = fp16(p_t s_t 2^E), times the exact (code - zero) operand; 2^E is a
// power of two per chunk that puts max_t s_t 2^E just under 2^14, so P' keeps
// full fp16 precision, and it is divided out exactly afterwards.
//
// INT4 -> FP16 conversion: ((u >> 4m) & 0x000F000F) | 0x64006400 is a pair of
// fp16 values 1024 + code, and one v_pk_add_f16 of -(1024 + zero) makes the
// exact pair (code - zero): three VALU instructions per two values (two for
// m = 0), the zero point applied for free.
//
// Cache layout (one buffer each for K and V, see w4a8_internal.h): codes of
// all rows, then one dword of parameters per row (fp16 scale | zero << 16).
//  * K codes, token-major, 64 bytes per (token, head): dword 4 kb + i holds
//    channels 32 i + 8 kb + j (j < 8), channel j in nibble (j >> 1) + 4 (j & 1).
//    Lane l of the QK product loads the 16 bytes of k-block kb = l >> 4 of
//    token l & 15: the B operands of the four MFMAs (32 channels each).
//  * V codes, blocks of 8 tokens x 128 channels (512 bytes): the dword at
//    position 32 (ct >> 1) + 2 (c & 15) + (ct & 1), ct = c >> 4, holds the 8
//    tokens of channel c, token j in nibble (j >> 1) + 4 (j & 1).  In the PV
//    product wave w owns channel tiles 2w and 2w + 1, and lane l loads the two
//    dwords of channel l & 15 of block kb: 8 bytes, 128 contiguous bytes per
//    16 lanes.
#include <algorithm>
#include <cmath>

#include "kernel_common.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kD = kKvHeadDim;
constexpr int kC = kKvChunk;            // tokens per attention workgroup
constexpr int kKT = kC / 16 / 4;        // 16-token K tiles per wave
constexpr int kVT = kC / 32;            // 32-token V tiles per chunk
constexpr int kSC = kC + 4;             // fp32 score row stride (spreads the rows over the banks)
constexpr int kPC = kC + 8;             // fp16 P' row stride

__device__ __host__ inline int nib(int j) { return (j >> 1) + 4 * (j & 1); }

__device__ inline float half_lo(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xFFFFu)); }

// Constants of the INT4 -> FP16 conversion, held in registers so that each
// masked OR is one v_and_or_b32 (a VOP3 instruction takes no literal on this
// chip and reads at most one scalar register): masks in SGPRs, biases in VGPRs.
struct Deq {
    uint32_t m0, m1;          // 0x000F000F, 0x00F000F0
    uint32_t b0, b1;          // 0x64006400 (1024 + c), 0x54005400 (64 + c)
};

__device__ inline Deq deq_consts()
{
    Deq d;
    d.m0 = 0x000F000Fu;
    d.m1 = 0x00F000F0u;
    d.b0 = 0x64006400u;
    d.b1 = 0x54005400u;
    asm volatile("" : "+s"(d.m0), "+s"(d.m1));
    asm volatile("" : "+v"(d.b0), "+v"(d.b1));
    return d;
}

// The four fp16 pairs (code - zero) of one code dword u, in operand order:
// pair d takes nibbles d and d + 4.  Nibbles at bits 0-3 (and 16-19) under
// the exponent of 1024 read 1024 + c; nibbles at bits 4-7 under the exponent
// of 64 read 64 + c (the mantissa step there is 1/16); the upper byte of each
// half is shifted down once.  z10 = -(1024 + zero), z6 = -(64 + zero) per half.
__device__ inline v4i deq8(uint32_t u, const Deq &k, uint32_t z10a, uint32_t z6a, uint32_t z10b, uint32_t z6b)
{
    const uint32_t u8 = u >> 8;
    const uint32_t p0 = (u & k.m0) | k.b0, p1 = (u & k.m1) | k.b1;
    const uint32_t p2 = (u8 & k.m0) | k.b0, p3 = (u8 & k.m1) | k.b1;
    auto add = [](uint32_t x, uint32_t z) {
        return (int)__builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, x) + __builtin_bit_cast(h2, z));
    };
    return v4i{add(p0, z10a), add(p1, z6a), add(p2, z10b), add(p3, z6b)};
}

// -(1024 + z) and -(64 + z) as fp16 bits
__device__ inline uint32_t zneg10(uint32_t z) { return 0xE400u | z; }
__device__ inline uint32_t zneg6(uint32_t z) { return 0xD400u | (z << 4); }

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fminf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// quantize + append
// ---------------------------------------------------------------------------
struct QuantArgs {
    const uint16_t *k, *v;     // [B][T][Hkv][128] fp16
    const int32_t *pos;        // [B] first cache index written per sequence
    uint8_t *kc, *vc;          // caches
    int64_t B, Hkv, T, S;
};

// One wave quantizes one (token, head) row; lane l holds channels 2l, 2l + 1.
__device__ inline void quant_row(const uint16_t *src, int l, uint8_t *codes_lds, uint32_t *param)
{
    const uint32_t pr = reinterpret_cast<const uint32_t *>(src)[l];
    const float x0 = half_lo(pr), x1 = half_lo(pr >> 16);
    const float lo = wave_min(fminf(fminf(x0, x1), 0.0f));
    const float hi = wave_max(fmaxf(fmaxf(x0, x1), 0.0f));
    const _Float16 sh = (_Float16)((hi - lo) / 15.0f);
    const float sf = (float)sh;
    uint32_t z = 0, c0 = 0, c1 = 0, sbits = __builtin_bit_cast(uint16_t, sh);
    if (sf == 0.0f) {
        sbits = 0;
    } else {
        const float zf = fminf(fmaxf(__builtin_rintf(-lo / sf), 0.0f), 15.0f);
        z = (uint32_t)zf;
        c0 = (uint32_t)fminf(fmaxf(__builtin_rintf(x0 / sf) + zf, 0.0f), 15.0f);
        c1 = (uint32_t)fminf(fmaxf(__builtin_rintf(x1 / sf) + zf, 0.0f), 15.0f);
    }
    codes_lds[2 * l] = (uint8_t)c0;
    codes_lds[2 * l + 1] = (uint8_t)c1;
    if (l == 0)
        *param = sbits | (z << 16);
}

__global__ __launch_bounds__(256) void kv4_quant_kernel(QuantArgs a)
{
    __shared__ uint8_t qk[8][kD], qv[8][kD];
    const int64_t bg = blockIdx.x;
    const int64_t b = bg / a.Hkv;
    const int64_t p0 = a.pos[b];
    const int64_t blk = p0 / 8 + blockIdx.y;                  // 8-token block of the cache
    const int64_t t_lo = std::max<int64_t>(p0, blk * 8);
    const int64_t t_hi = std::min<int64_t>(std::min<int64_t>(p0 + a.T, blk * 8 + 8), a.S);
    if (p0 < 0 || t_lo >= t_hi)
        return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    uint32_t *kpar = reinterpret_cast<uint32_t *>(a.kc + kv4_code_bytes(a.B, a.Hkv, a.S)) + bg * a.S;
    uint32_t *vpar = reinterpret_cast<uint32_t *>(a.vc + kv4_code_bytes(a.B, a.Hkv, a.S)) + bg * a.S;
    const int64_t g = bg % a.Hkv;
#pragma unroll
    for (int jj = 0; jj < 2; jj++) {
        const int j = 2 * w + jj;
        const int64_t t = blk * 8 + j;
        if (t < t_lo || t >= t_hi)
            continue;
        const int64_t src = ((b * a.T + (t - p0)) * a.Hkv + g) * kD;
        quant_row(a.k + src, l, qk[j], kpar + t);
        quant_row(a.v + src, l, qv[j], vpar + t);
    }
    __syncthreads();
    if (tid < 128) {
        // K: dword d of token j's row
        const int j = tid >> 4, d = tid & 15;
        const int64_t t = blk * 8 + j;
        if (t >= t_lo && t < t_hi) {
            const int kb = d >> 2, i = d & 3;
            uint32_t u = 0;
#pragma unroll
            for (int jj = 0; jj < 8; jj++)
                u |= (uint32_t)qk[j][32 * i + 8 * kb + jj] << (4 * nib(jj));
            reinterpret_cast<uint32_t *>(a.kc + (bg * a.S + t) * kKvRowBytes)[d] = u;
        }
    } else {
        // V: the dword of one channel over the block's 8 tokens (read-modify-
        // write when the call covers only part of the block)
        const int P = tid - 128;
        const int ct = 2 * (P >> 5) + (P & 1), c = 16 * ct + ((P >> 1) & 15);
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.vc + (bg * a.S + blk * 8) * kKvRowBytes) + P;
        uint32_t u = (t_lo == blk * 8 && t_hi == blk * 8 + 8) ? 0u : *dst;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int64_t t = blk * 8 + j;
            if (t >= t_lo && t < t_hi) {
                u &= ~(15u << (4 * nib(j)));
                u |= (uint32_t)qv[j][c] << (4 * nib(j));
            }
        }
        *dst = u;
    }
}

// ---------------------------------------------------------------------------
// unpack (test inverse of the layout)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void kv4_unpack_kernel(const uint8_t *cache, int is_v, int64_t rows,
                                                         int64_t B, int64_t Hkv, int64_t S, uint8_t *codes,
                                                         uint16_t *s, uint8_t *z)
{
    const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    const int c = threadIdx.x & 127;
    if (row >= rows)
        return;
    uint32_t u;
    int sh;
    if (!is_v) {
        const int i = c >> 5, kb = (c >> 3) & 3, j = c & 7;
        u = reinterpret_cast<const uint32_t *>(cache + row * kKvRowBytes)[4 * kb + i];
        sh = 4 * nib(j);
    } else {
        const int ct = c >> 4;
        const int P = 32 * (ct >> 1) + 2 * (c & 15) + (ct & 1);
        const int64_t blk0 = row / 8 * 8;
        u = reinterpret_cast<const uint32_t *>(cache + blk0 * kKvRowBytes)[P];
        sh = 4 * nib((int)(row & 7));
    }
    codes[row * kD + c] = (uint8_t)((u >> sh) & 15u);
    if (c == 0) {
        const uint32_t p = reinterpret_cast<const uint32_t *>(cache + kv4_code_bytes(B, Hkv, S))[row];
        s[row] = (uint16_t)(p & 0xFFFFu);
        z[row] = (uint8_t)((p >> 16) & 15u);
    }
}

// ---------------------------------------------------------------------------
// decode attention
// ---------------------------------------------------------------------------
struct AttnArgs {
    const uint16_t *q;         // [B][Hq][128] fp16
    const uint8_t *kc, *vc;
    const int32_t *lens;       // [B]
    int64_t B, Hq, Hkv, S;
    int G;
    int nsplit;                // workspace slots per (sequence, query head)
    int cps;                   // 256-token chunks per workgroup
    float kscale;              // sm_scale * log2(e)
    uint16_t *out;             // [B][Hq][128] fp16
    float *ws_o;               // [B][Hq][nsplit][128]
    float *ws_ml;              // [B][Hq][nsplit][2]
};

__device__ inline int seq_len(const AttnArgs &a, int64_t b)
{
    const int L = a.lens[b];
    return L < 0 ? 0 : (int)std::min<int64_t>(L, a.S);
}

// buffer resources over the chunk's rows, addressed with 32-bit offsets from a
// scalar base (no per-load 64-bit address arithmetic)
using dev::kBufFlags;
using dev::rsrc;

#ifndef KV4_ATTN_WAVES
#define KV4_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = KV4_ATTN_WAVES;  // waves per SIMD the register budget is cut for

// GP: the number of query heads per kv head rounded up to a power of two;
// the softmax gives each of those rows 256 / GP threads.  A workgroup takes
// a run of cps chunks of one (sequence, kv head) and carries the softmax
// across them (running maximum and sum per query head, the output
// accumulators rescaled when the maximum grows); the runs of one sequence
// meet in kv4_combine_kernel.
template <int GP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kAttnWaves, 8))) void kv4_attn_kernel(AttnArgs a)
{
    constexpr int P = 256 / GP;             // threads per softmax row
    constexpr int PW = P > 64 ? P / 64 : 1; // waves per row
    __shared__ float sc[GP][kSC];
    __shared__ __attribute__((aligned(16))) _Float16 pp[GP][kPC];
    __shared__ uint32_t vpar[kC];
    __shared__ __attribute__((aligned(16))) uint32_t zc10[kC / 2], zc6[kC / 2];
    __shared__ float red[4], redm[4], redl[4];
    __shared__ float mrow[GP], lrow[GP], arow[GP];
    __shared__ __attribute__((aligned(16))) uint16_t qs[GP][kD];

    const int64_t bg = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = bg / a.Hkv, g = bg % a.Hkv;
    const int L = seq_len(a, b);
    const int nch = (L + kC - 1) / kC;
    const int cb = split * a.cps, ce = std::min(cb + a.cps, nch);
    if (cb >= ce)
        return;
    const int tid = threadIdx.x, l = tid & 63, lr = l & 15, kb = l >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = a.G;
    const int64_t codes_total = kv4_code_bytes(a.B, a.Hkv, a.S);

    // the group's query rows, 16 bytes per thread, staged in LDS once the
    // first chunk's loads are in flight; rows past G re-read head 0 of the
    // group: their results are never stored
    v4i qv = v4i{0, 0, 0, 0};
    if (tid < GP * kD / 8) {
        const int hr = tid / (kD / 8);
        qv = *reinterpret_cast<const v4i *>(a.q + (b * a.Hq + g * G + (hr < G ? hr : 0)) * kD + 8 * (tid % (kD / 8)));
    }
    const Deq dq = deq_consts();
    const int qr = lr < GP ? lr : 0;
    const int row = tid / P, part = tid % P;          // softmax role
    float m_run = -INFINITY, l_run = 0.0f;            // per row (l: this thread's share)
    f4 o2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};

    for (int c = cb; c < ce; c++) {
        const int c0 = c * kC;
        const int n = std::min(kC, L - c0);
        const int n32 = (n + 31) & ~31;
        const int64_t row0 = bg * a.S + c0;
        const __amdgpu_buffer_rsrc_t rk = rsrc(a.kc + row0 * kKvRowBytes, n32 * kKvRowBytes);
        const __amdgpu_buffer_rsrc_t rkp = rsrc(a.kc + codes_total + row0 * 4, n32 * 4);
        const __amdgpu_buffer_rsrc_t rv = rsrc(a.vc + row0 * kKvRowBytes, n32 * kKvRowBytes);
        const __amdgpu_buffer_rsrc_t rvp = rsrc(a.vc + codes_total + row0 * 4, n32 * 4);

        // every load of the chunk up front: V parameters, this wave's K tiles,
        // the V codes of this wave's channel slice.  Loads and tile loops are
        // unconditional (tiles past the end re-read the chunk's first tile and
        // are masked), so no load is sunk into a branch and every wait is a
        // counted vmcnt.
        const uint32_t vp_reg = __builtin_amdgcn_raw_buffer_load_b32(rvp, 4 * (tid < n32 ? tid : 0), 0, 0);
        const int nk = (n + 15) >> 4;
        v4i kq[kKT];
        uint32_t kp[kKT];
#pragma unroll
        for (int j = 0; j < kKT; j++) {
            const int tt = (w + 4 * j) < nk ? w + 4 * j : 0;            // wave-uniform
            kq[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, lr * kKvRowBytes + 16 * kb, 16 * tt * kKvRowBytes, 0);
            kp[j] = __builtin_amdgcn_raw_buffer_load_b32(rkp, 4 * lr, 64 * tt, 0);
        }
        v2i vq[kVT];
#pragma unroll
        for (int j = 0; j < kVT; j++) {
            const int js = 32 * j < n ? j : 0;
            vq[j] = __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(rv, kb * 512 + 4 * (32 * w + 2 * lr),
                                                                                 js * 2048, 0));
        }
        if (c == cb) {
            if (tid < GP * kD / 8)
                *reinterpret_cast<v4i *>(&qs[tid / (kD / 8)][8 * (tid % (kD / 8))]) = qv;
            __syncthreads();
        }

        // scores (log2 units) of this wave's tiles; rows past GP are not stored
#pragma unroll
        for (int j = 0; j < kKT; j++) {
            const int t0 = 16 * (w + 4 * j);
            const uint32_t par = kp[j];
            const uint32_t zk = (par >> 16) & 15u;
            const uint32_t z10 = zneg10(zk) * 0x10001u, z6 = zneg6(zk) * 0x10001u;
            f4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const v4i bw = deq8((uint32_t)kq[j][i], dq, z10, z6, z10, z6);
                const v4i qa = *reinterpret_cast<const v4i *>(&qs[qr][32 * i + 8 * kb]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, qa), __builtin_bit_cast(h8, bw),
                                                             acc, 0, 0, 0);
            }
            const float f = half_lo(par) * a.kscale;
#pragma unroll
            for (int r = 0; r < 4; r++)
                if (4 * kb + r < GP)
                    sc[4 * kb + r][t0 + lr] = acc[r] * f;
        }
        vpar[tid] = vp_reg;
        {
            const float mx = wave_max(tid < n ? half_lo(vp_reg) : 0.0f);
            if (l == 0)
                red[w] = mx;
        }
        __syncthreads();

        // softmax step: P threads per row, GP tokens per thread (t = part + P i)
        const float smax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        int e = 0;
        (void)frexpf(smax, &e);
        const float sfac = smax > 0.0f ? ldexpf(1.0f, 14 - e) : 1.0f;    // 2^E: max scale * 2^E < 2^14
        float sv[GP];                                  // this thread's scores, read once
#pragma unroll
        for (int i = 0; i < GP; i++)
            sv[i] = sc[row][part + P * i];
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < GP; i++)
            if (part + P * i < n)
                m = fmaxf(m, sv[i]);
#pragma unroll
        for (int o = (P < 64 ? P : 64) / 2; o > 0; o >>= 1)
            m = fmaxf(m, __shfl_xor(m, o));
        if constexpr (PW > 1) {
            if (l == 0)
                redm[w] = m;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < PW; i++)
                m = fmaxf(m, redm[row * PW + i]);
        }
        const float m_new = fmaxf(m_run, m);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first chunk
        m_run = m_new;
        float lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < GP; i++) {
            const int t = part + P * i;
            float pv = 0.0f;
            if (t < n) {
                const float p = __builtin_amdgcn_exp2f(sv[i] - m_new);
                lsum += p;
                pv = p * (half_lo(vpar[t]) * sfac);
            }
            pp[row][t] = (_Float16)pv;                 // every token of the chunk: the PV loop reads them all
        }
        l_run = l_run * alpha + lsum;
        if (part == 0)
            arow[row] = alpha;
        if (tid < kC / 2) {
            uint32_t z0 = 0, z1 = 0;                    // tokens past the end: any finite operand
            if (tid < n32 / 2) {
                z0 = (vpar[2 * tid] >> 16) & 15u;
                z1 = (vpar[2 * tid + 1] >> 16) & 15u;
            }
            zc10[tid] = zneg10(z0) | (zneg10(z1) << 16);
            zc6[tid] = zneg6(z0) | (zneg6(z1) << 16);
        }
        __syncthreads();

        // PV: this wave's two 16-channel tiles over the chunk.  Operand rows of
        // heads past G (and past GP, which re-read row 0) only feed output rows
        // that are not stored: row i of the product depends on row i of P'.
        const int prow = lr < GP ? lr : 0;
        f4 t2[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int j = 0; j < kVT; j++) {
            const v4i pa = *reinterpret_cast<const v4i *>(&pp[prow][32 * j + 8 * kb]);
            const v4i z10 = *reinterpret_cast<const v4i *>(&zc10[16 * j + 4 * kb]);
            const v4i z6 = *reinterpret_cast<const v4i *>(&zc6[16 * j + 4 * kb]);
#pragma unroll
            for (int c2 = 0; c2 < 2; c2++) {
                // operand pair d holds tokens 2d, 2d + 1 of the lane's 8-token block
                const v4i bw = deq8((uint32_t)vq[j][c2], dq, (uint32_t)z10[0], (uint32_t)z6[1], (uint32_t)z10[2],
                                    (uint32_t)z6[3]);
                t2[c2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, pa),
                                                                __builtin_bit_cast(h8, bw), t2[c2], 0, 0, 0);
            }
        }
        const float unscale = 1.0f / sfac;             // exact: a power of two
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const float al = arow[4 * kb + r < GP ? 4 * kb + r : 0];
#pragma unroll
            for (int c2 = 0; c2 < 2; c2++)
                o2[c2][r] = o2[c2][r] * al + t2[c2][r] * unscale;
        }
    }

    // the rows' sums, then the outputs: final when this run covers the whole
    // sequence, else a partial (max, sum, unnormalized output) for the combine
#pragma unroll
    for (int o = (P < 64 ? P : 64) / 2; o > 0; o >>= 1)
        l_run += __shfl_xor(l_run, o);
    if constexpr (PW > 1) {
        if (l == 0)
            redl[w] = l_run;
        __syncthreads();
        if (part == 0) {
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < PW; i++)
                t += redl[row * PW + i];
            lrow[row] = t;
            mrow[row] = m_run;
        }
    } else {
        if (part == 0) {
            lrow[row] = l_run;
            mrow[row] = m_run;
        }
    }
    __syncthreads();
    const bool single = cb == 0 && ce == nch;
#pragma unroll
    for (int r = 0; r < 4; r++) {
        const int hh = 4 * kb + r;
        if (hh >= G || hh >= GP)
            continue;
        const int64_t bh = b * a.Hq + g * G + hh;
        const float inv_l = single ? __builtin_amdgcn_rcpf(lrow[hh]) : 1.0f;
#pragma unroll
        for (int c2 = 0; c2 < 2; c2++) {
            const int ch = 16 * (2 * w + c2) + lr;
            if (single)
                a.out[bh * kD + ch] = __builtin_bit_cast(uint16_t, (_Float16)(o2[c2][r] * inv_l));
            else
                a.ws_o[(bh * a.nsplit + split) * kD + ch] = o2[c2][r];
        }
    }
    if (!single && tid < G) {
        const int64_t bh = b * a.Hq + g * G + tid;
        a.ws_ml[(bh * a.nsplit + split) * 2] = mrow[tid];
        a.ws_ml[(bh * a.nsplit + split) * 2 + 1] = lrow[tid];
    }
}

// Sequences split over several workgroups: merge their (max, sum, partial
// output); empty sequences get zeros.  One wave per (sequence, query head):
// lane i reads split i's max and sum, the weights 2^(m_i - M) are shared
// across the wave, and each lane then adds two channels over the splits.
__global__ __launch_bounds__(64) void kv4_combine_kernel(AttnArgs a)
{
    __shared__ float wgt[64];
    const int64_t bh = blockIdx.x;
    const int64_t b = bh / a.Hq;
    const int L = seq_len(a, b);
    const int l = threadIdx.x;
    uint32_t *o = reinterpret_cast<uint32_t *>(a.out + bh * kD);
    if (L == 0) {
        o[l] = 0;
        return;
    }
    const int nch = (L + kC - 1) / kC;
    const int ns = (nch + a.cps - 1) / a.cps;
    if (ns == 1)
        return;
    const float *ml = a.ws_ml + bh * a.nsplit * 2;
    const float *po = a.ws_o + bh * a.nsplit * kD + 2 * l;
    float M = -INFINITY;
    for (int i = l; i < ns; i += 64)
        M = fmaxf(M, ml[2 * i]);
    M = wave_max(M);
    float den = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int i0 = 0; i0 < ns; i0 += 64) {
        const int i = i0 + l;
        float wi = 0.0f;
        if (i < ns) {
            wi = __builtin_amdgcn_exp2f(ml[2 * i] - M);
            den += ml[2 * i + 1] * wi;
        }
        wgt[l] = wi;
        __syncthreads();
        const int cnt = std::min(64, ns - i0);
        int k = 0;
        for (; k + 4 <= cnt; k += 4) {
            float2 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++)
                v[u] = *reinterpret_cast<const float2 *>(po + (int64_t)(i0 + k + u) * kD);
#pragma unroll
            for (int u = 0; u < 4; u++) {
                o0 += v[u].x * wgt[k + u];
                o1 += v[u].y * wgt[k + u];
            }
        }
        for (; k < cnt; k++) {
            const float2 v = *reinterpret_cast<const float2 *>(po + (int64_t)(i0 + k) * kD);
            o0 += v.x * wgt[k];
            o1 += v.y * wgt[k];
        }
        __syncthreads();
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        den += __shfl_xor(den, off);
    const float inv = 1.0f / den;
    const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)(o0 * inv));
    const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)(o1 * inv));
    o[l] = lo | (hi << 16);
}

}  // namespace

hipError_t launch_kv4_quant(const uint16_t *k, const uint16_t *v, int64_t B, int64_t Hkv, int64_t T,
                            const int32_t *pos, uint8_t *k_cache, uint8_t *v_cache, int64_t S, hipStream_t st)
{
    QuantArgs a{k, v, pos, k_cache, v_cache, B, Hkv, T, S};
    const int64_t nblk = (T + 7) / 8 + 1;                 // blocks a run of T tokens can touch
    hipLaunchKernelGGL(kv4_quant_kernel, dim3((unsigned)(B * Hkv), (unsigned)nblk), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_kv4_unpack(const uint8_t *cache, int is_v, int64_t B, int64_t Hkv, int64_t S, uint8_t *codes,
                             uint16_t *s, uint8_t *z, hipStream_t st)
{
    const int64_t rows = B * Hkv * S;
    hipLaunchKernelGGL(kv4_unpack_kernel, dim3((unsigned)((rows + 1) / 2)), dim3(256), 0, st, cache, is_v, rows,
                       B, Hkv, S, codes, s, z);
    return hipGetLastError();
}

hipError_t launch_kv4_attention(const uint16_t *q, int64_t B, int64_t Hq, int64_t Hkv, const uint8_t *k_cache,
                                const uint8_t *v_cache, int64_t S, const int32_t *lens, float sm_scale,
                                uint16_t *out, void *ws, hipStream_t st)
{
    AttnArgs a;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.lens = lens;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.S = S;
    a.G = (int)(Hq / Hkv);
    a.nsplit = (int)kv4_splits(S);
    a.cps = kv4_chunks_per_run(B * Hkv, S);
    a.kscale = sm_scale * 1.4426950408889634f;
    a.out = out;
    a.ws_o = static_cast<float *>(ws);
    a.ws_ml = a.ws_o ? a.ws_o + B * Hq * a.nsplit * kD : nullptr;
    const dim3 grid((unsigned)(B * Hkv), (unsigned)((a.nsplit + a.cps - 1) / a.cps));
    switch (a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : a.G <= 8 ? 8 : 16) {
    case 1: hipLaunchKernelGGL(kv4_attn_kernel<1>, grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL(kv4_attn_kernel<2>, grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL(kv4_attn_kernel<4>, grid, dim3(256), 0, st, a); break;
    case 8: hipLaunchKernelGGL(kv4_attn_kernel<8>, grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL(kv4_attn_kernel<16>, grid, dim3(256), 0, st, a); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(kv4_combine_kernel, dim3((unsigned)(B * Hq)), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace w4a8
