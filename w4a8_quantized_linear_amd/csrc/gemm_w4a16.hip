// gemm_w4a16.hip -- W4A16 GEMM on the W4A8 weight stream, gfx950.
//
// The activations stay fp16 (no per-token quantization) and the weights are
// dequantized to fp16 inside the main loop: the QFactory reading notes (2.1)
// give the dequantization w = (w_quant - zero) * scale, and Lecture 15 notes
// (15.5) describe this int4 -> fp16 path as the one whose per-weight
// instruction count decides decode time.  On the two-level weights of this
// library the dequantized weight is r s0 with r = q4 s1 - z s1 (an integer in
// [-127, 127]), so
//   y[m,n] = fp16( s0[n] * sum_k x[m,k] r[n,k] )
// with r exact in fp16, every product x r exact in fp32, the sums in fp32 on
// the matrix cores (v_mfma_f32_16x16x32_f16) and s0 in the epilogue.
//
// Rebuild per 4 weights (one dword of codes): mask, v_pk_mad_u16 to the
// biased bytes r + 128 (exactly as the W4A8 path, without its final xor),
// then two v_perm_b32 that place each byte under the fp16 exponent of 1024
// (0x64XX = 1024 + r + 128) and two v_pk_add_f16 of -1152: 1.75 VALU
// instructions per weight with the shift, against 0.875 for int4 -> int8.
//
// Operand order.  A lane's 16-byte weight load holds, for its channel, the
// codes of k = 16 kb + [0, 16) (low nibbles) and 64 + 16 kb + [0, 16) (high
// nibbles), kb = lane / 16.  Each group is four MFMAs of 32 k; MFMA q takes
// from every lane the 8 consecutive k = 8 (q & 1) + 64 (q >> 1) + 16 kb + j,
// j < 8, for both operands (the activation operand of a lane is one 16-byte
// load of those 8 halves), so the weights are used in their stored order and
// the contraction still covers each k once.
//
// Work decomposition (decode shapes: the weight stream is read once per 16
// MT tokens).  A workgroup of four waves owns NT tiles of 16 channels and MT
// tiles of 16 tokens (each rebuilt weight operand feeds MT MFMAs); the waves
// split the K groups into four runs and stream their
// weight tiles, parameter dwords and activation operands DEPTH groups ahead
// (unconditional loads, so the compiler's vmcnt waits are exact).  The four
// partial sums meet in LDS and are added in wave order (deterministic).
// For a few tokens (XS) the workgroup first copies its tokens' fp16 rows
// into LDS (direct-to-LDS loads, 16-byte row pad) and the waves read their
// activation operands there: the weight tile is then the only vector-memory
// load of a group, where four 16-byte activation loads per group would keep
// the texture units busier than the weight stream does.
#include <algorithm>
#include <cstdlib>

#include "kernel_common.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

using dev::kBufFlags;
using dev::rsrc;
constexpr int kWaves = 4;
constexpr int kDepth = 4;                // groups of loads in flight per wave
static_assert(kDepth == 4, "ring slot d holds the groups d mod 4 of a run: one parameter dword per slot-0 group");

// four biased bytes u = r + 128 (k order) -> two fp16 pairs r
__device__ inline void to_half(uint32_t u, uint32_t &lo, uint32_t &hi)
{
    const h2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    lo = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + off);
    hi = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + off);
}

struct W16Args {
    const uint16_t *x;        // [M, ldx] fp16
    const uint8_t *codes;
    const uint8_t *params;
    const uint16_t *s0;       // [N] fp16
    int64_t M, N, K, ldx;
    uint16_t *y;              // [M, N] fp16
    int cx;                   // activation operands loaded row-contiguous, lanes exchanged
};

template <int NT, int MT>
struct Slot {
    v4i w[NT];                // codes of the NT tiles, one group
    uint32_t p[NT];           // parameter dword (four groups) of the lane's channel
    v4i x[MT][4];             // activation operands of the group's four MFMAs, per token tile
};

template <int NT, int MT, bool XS>
__global__ __launch_bounds__(64 * kWaves) void gemm_w4a16_kernel(W16Args a)
{
    static_assert(!XS || MT == 1, "staged rows serve one token tile");
    __shared__ f4 red[kWaves][MT][NT][64];
    extern __shared__ __align__(16) uint8_t xsm[];   // XS: fp16 rows [mrows][2 K + 16]
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int l = threadIdx.x & 63, lr = l & 15, kb = l >> 4;
    const int nt0 = blockIdx.x * NT;                  // first 16-channel tile
    const int ntiles = (int)(a.N / kTileN);
    const int64_t m0 = (int64_t)blockIdx.y * 16 * MT;
    const int G = (int)(a.K / kGroup), G4 = (int)groups_padded(a.K);
    // the waves split K in runs of whole parameter dwords (4 groups), so that
    // one dword load per 4 groups serves a run (a wave's first group is 4-aligned)
    const int nq = G4 / 4;
    const int g0 = 4 * (nq * wv / kWaves), g1 = min(4 * (nq * (wv + 1) / kWaves), G);

    // tiles past N re-read the last tile (their outputs are not stored);
    // tokens past M re-read the last token's row
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, (a.M - 1) * a.ldx * 2 + a.K * 2);
    int tile[NT];
#pragma unroll
    for (int t = 0; t < NT; t++)
        tile[t] = min(nt0 + t, ntiles - 1);
    // an operand's 16 bytes for lane (lr, kb): token row lr, k-block kb.  With
    // cx the lanes load the block row by row instead (lane 4 r + q: row r,
    // k-block q, so four neighbouring lanes read one row's 128-byte line)
    // and ds_bpermute gives lane (lr, kb) the piece lane 4 lr + kb loaded
    int xoff[MT];                                        // bytes: token row, k-block
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int64_t row = min<int64_t>(m0 + 16 * mt + (a.cx ? l >> 2 : lr), a.M - 1);
        xoff[mt] = (int)(row * a.ldx * 2) + 32 * (a.cx ? l & 3 : kb);
    }
    const int xsrc = 4 * (4 * lr + kb);
    const int glast = max(g1 - 1, g0);
    const int len = g1 - g0;

    // XS: the block's token rows go straight into LDS (buffer form of the
    // direct-to-LDS load, counted below), issued before the weight prologue
    const int mrows = (int)min<int64_t>(16, a.M - m0);
    const int xstride = 2 * (int)a.K + 16;
    if constexpr (XS) {
        const int nch = (mrows * xstride + 1023) / 1024;
        for (int ch = wv; ch < nch; ch += kWaves) {
            const int o = ch * 1024 + 16 * l;
            const int r = o / xstride;
            const int col = o - r * xstride;
            const bool ok = r < mrows && col < 2 * (int)a.K;
            dev::lds_copy16(rx, xsm + ch * 1024, ok ? (int)((m0 + r) * a.ldx * 2) + col : 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    const int8_t *xrow = reinterpret_cast<const int8_t *>(xsm) + min(lr, mrows - 1) * xstride + 32 * kb;

    // ring slot d holds groups g0 + d (mod 4): slot 0 also loads the parameter
    // dword of its quad of groups (d is a constant in the unrolled loops)
    auto load = [&](Slot<NT, MT> &s, int i, int d) {
        const int g = min(g0 + i, glast);
#pragma unroll
        for (int t = 0; t < NT; t++) {
            s.w[t] = __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * l, ((int64_t)tile[t] * G + g) * kTileBytes, 2);
            if (d == 0)
                s.p[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, (int)(param_index(tile[t] * 16 + lr, g, G4) & ~3),
                                                              0, 0);
        }
        if constexpr (!XS) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    s.x[mt][q] = __builtin_amdgcn_raw_buffer_load_b128(
                        rx, xoff[mt], g * 256 + 2 * (8 * (q & 1) + 64 * (q >> 1)), 0);
        }
    };

    f4 acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int t = 0; t < NT; t++)
            acc[mt][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    Slot<NT, MT> ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; d++)
        load(ring[d], d, d);
    if constexpr (XS) {
        // loads retire in order: once only the weight prologue is
        // outstanding, this thread's row copies have landed
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kDepth + 1) * NT) : "memory");
        dev::lds_barrier();
    }

    uint32_t pq[NT];                    // parameter dwords of the current quad of groups
    auto step = [&](Slot<NT, MT> &s, int i, int d) {
        const int g = g0 + i;
        if (d == 0) {
#pragma unroll
            for (int t = 0; t < NT; t++)
                pq[t] = s.p[t];
        }
        if constexpr (XS) {
#pragma unroll
            for (int q = 0; q < 4; q++)
                s.x[0][q] = *reinterpret_cast<const v4i *>(xrow + g * 256 + 2 * (8 * (q & 1) + 64 * (q >> 1)));
        } else if (a.cx) {
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int q = 0; q < 4; q++)
#pragma unroll
                    for (int d = 0; d < 4; d++)
                        s.x[mt][q][d] = __builtin_amdgcn_ds_bpermute(xsrc, s.x[mt][q][d]);
        }
#pragma unroll
        for (int t = 0; t < NT; t++) {
            const uint32_t pb = (pq[t] >> (8 * d)) & 0xFFu;
            const uint32_t s1 = (pb & 15u) + 1u;
            const uint32_t c16 = ((128u - (pb >> 4) * s1) * 257u) & 0xFFFFu;
            const us2 S = {(unsigned short)s1, (unsigned short)s1};
            const us2 C = {(unsigned short)c16, (unsigned short)c16};
            uint32_t b[2][4][2];   // [k-half][dword][pair]: fp16 pairs of the rebuilt weights
#pragma unroll
            for (int d = 0; d < 4; d++) {
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const uint32_t nib = ((uint32_t)s.w[t][d] >> (4 * h)) & 0x0F0F0F0Fu;
                    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_bit_cast(us2, nib) * S + C);
                    to_half(u, b[h][d][0], b[h][d][1]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int h = q >> 1, d0 = 2 * (q & 1);
                const v4i bw = {(int)b[h][d0][0], (int)b[h][d0][1], (int)b[h][d0 + 1][0], (int)b[h][d0 + 1][1]};
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
                    acc[mt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        __builtin_bit_cast(h8, s.x[mt][q]), __builtin_bit_cast(h8, bw), acc[mt][t], 0, 0, 0);
            }
        }
        load(s, i + kDepth, d);
    };

    int i = 0;
    for (; i + kDepth <= len; i += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; d++)
            step(ring[d], i + d, d);
    }
#pragma unroll
    for (int d = 0; d < kDepth - 1; d++)
        if (i + d < len)
            step(ring[d], i + d, d);

    // the waves' partial sums, added in wave order; lane l holds tokens
    // 16 mt + 4 (l / 16) + r, channel l % 16 of each tile
#pragma unroll
    for (int mt = 0; mt < MT; mt++)
#pragma unroll
        for (int t = 0; t < NT; t++)
            red[wv][mt][t][l] = acc[mt][t];
    __syncthreads();
    if (wv == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
#pragma unroll
            for (int t = 0; t < NT; t++) {
                f4 v = red[0][mt][t][l];
#pragma unroll
                for (int w = 1; w < kWaves; w++)
                    v += red[w][mt][t][l];
                if (nt0 + t >= ntiles)
                    continue;
                const int64_t n = (int64_t)(nt0 + t) * 16 + lr;
                const float sc = (float)__builtin_bit_cast(_Float16, a.s0[n]);
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int64_t m = m0 + 16 * mt + 4 * kb + r;
                    if (m < a.M)
                        a.y[m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)(v[r] * sc));
                }
            }
        }
    }
}

// LDS of the staged token rows (0 when they do not fit the 64 KB that keeps
// several workgroups per compute unit)
inline size_t w16_xs_bytes(int64_t M, int64_t K)
{
    const int64_t b = (std::min<int64_t>(16, M) * (2 * K + 16) + 1023) / 1024 * 1024;
    return b <= 64 * 1024 ? (size_t)b : 0;
}

template <int NT, int MT, bool XS>
hipError_t launch_nt(const W16Args &a, hipStream_t st)
{
    const int64_t nblk = (a.N / kTileN + NT - 1) / NT;
    const int64_t mblk = (a.M + 16 * MT - 1) / (16 * MT);
    const size_t lds = XS ? w16_xs_bytes(a.M, a.K) : 0;
    if constexpr (XS) {
        // staged rows plus the reduction array pass the 64 KB default
        const hipError_t e =
            raise_lds_limit(reinterpret_cast<const void *>(&gemm_w4a16_kernel<NT, MT, XS>), 80 * 1024);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((gemm_w4a16_kernel<NT, MT, XS>), dim3((unsigned)nblk, (unsigned)mblk), dim3(64 * kWaves), lds,
                       st, a);
    return hipGetLastError();
}

}  // namespace

// Tiles per workgroup.  Every workgroup reads the activation operands of its
// 16 tokens from L2 once, so NT tiles share that read: with more than 8
// distinct tokens it costs as much as the weight tiles and four tiles per
// workgroup pay off when the launch still has at least 160 workgroups
// (measured: with 128, N = 8192 at 9..16 tokens, two tiles are 22-35% faster
// at every K; with 160 and more, four are 7-26% faster); otherwise two tiles
// when that still leaves 256 workgroups per 16 tokens (or there are several
// token blocks), else one.  W4A8_W16_NT=1|2|4 overrides (sweeps).
static int pick_nt(int64_t M, int64_t N)
{
    const int64_t tiles = N / kTileN;
    if (M > 8 && tiles >= 512 && (tiles / 4) * ((M + 15) / 16) >= 160)
        return 4;
    if (tiles >= 512 || M > 16)
        return 2;
    return 1;
}

// Token tiles per workgroup (MT) at 17..64 tokens: with two, each weight
// tile is read and rebuilt once per 32 tokens instead of 16, at the cost of
// more registers (one wave per SIMD at four channel tiles) and, for 17..32
// tokens, half the workgroups.  Graph-timed on MI355X (K = 4096 unless
// noted; NT x MT, us):
//   N = 22016 (1376 tiles): M = 17 2x2 21.4 against 24.7 for the rule above,
//     M = 32 2x2 25.3 / 26.2, M = 48 4x2 39.6 / 39.7, M = 64 4x2 42.0 / 48.9;
//   N = 11008 and 12288 (688, 768 tiles): M = 17 and 32 4x2 13.6-15.0 against
//     16.4-18.7; at 48 and 64 tokens 4x1 stays (within 2-6% of the best);
//   N = 4096 (256 tiles; K = 4096 and 11008): at 17 and 32 tokens 2x1 stays
//     (two token tiles halve the workgroups and run 10-40% slower); M = 48
//     and 64 2x2 10.0-10.2 against 11.2-11.5 (K = 11008: 19.2-19.6 / 23.1-23.4).
// Each token's sum is the same MFMA sequence either way: the results are
// bit-identical.  W4A8_W16_MT=1|2 overrides (sweeps).
static void pick_tokens(int64_t M, int64_t N, int &nt, int &mt)
{
    const int64_t tiles = N / kTileN;
    if (M <= 16 || M > 64)
        return;
    if (tiles >= 1024) {
        mt = 2;
        nt = M <= 32 ? 2 : 4;
    } else if (tiles >= 512) {
        if (M <= 32) {
            mt = 2;
            nt = 4;
        }
    } else if (M > 32) {
        mt = 2;
        nt = 2;
    }
}

hipError_t launch_gemm_w4a16(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                             const uint8_t *stream_bytes, const uint16_t *s0, int64_t N, uint16_t *y,
                             hipStream_t st)
{
    // the activations are addressed with 32-bit buffer offsets: launches of
    // at most rows_max tokens
    const int64_t rows_max = std::max<int64_t>(16, (0x7FFFFFFF - 2 * K) / (2 * ldx) / 16 * 16);
    for (int64_t r0 = 0; r0 < M; r0 += rows_max) {
        W16Args a;
        a.x = x + r0 * ldx;
        a.codes = stream_bytes;
        a.params = stream_bytes + code_bytes(N, K);
        a.s0 = s0;
        a.M = std::min(rows_max, M - r0);
        a.N = N;
        a.K = K;
        a.ldx = ldx;
        a.y = y + r0 * N;
        // staged rows for up to 4 tokens on wide layers (>= 512 tiles) when
        // they fit, one tile per workgroup.  Measured on MI355X, M = 1: K =
        // 4096, N = 11008 8.0 us against 9.9 for the best register form; K =
        // 8192, N = 28672 24.1 against 28.9.  With 256 tiles the register
        // form is 2-10% faster (fewer workgroups hide less of the staging).
        // At 6 and 8 tokens (rows staged in up to 72 KB, a build that allowed
        // it) staging was 4-30% slower on the 7B layers (K = 4096, N = 11008,
        // M = 8: 11.0-12.6 us against 10.6).
        // W4A8_W16_XS=0|1 and W4A8_W16_NT=1|2|4 override, for sweeps
        bool xs = a.M <= 4 && N / kTileN >= 512 && w16_xs_bytes(a.M, K) > 0;
        if (const char *env = std::getenv("W4A8_W16_XS"))
            xs = std::atoi(env) != 0 && w16_xs_bytes(a.M, K) > 0;
        int nt = xs ? 1 : pick_nt(a.M, N);
        // row-contiguous activation loads from 8 tokens on (measured on
        // MI355X, K = 4096, N = 11008: M = 32 17.5 us against 20.6; M = 8 11.0
        // against 11.1; below 8 tokens up to 9% slower); W4A8_W16_CX=0|1
        // overrides, for sweeps
        a.cx = a.M >= 8;
        if (const char *env = std::getenv("W4A8_W16_CX"))
            a.cx = std::atoi(env) != 0;
        if (const char *env = std::getenv("W4A8_W16_NT"))
            nt = std::atoi(env) == 4 ? 4 : (std::atoi(env) == 2 ? 2 : (std::atoi(env) == 1 ? 1 : nt));
        int mt = 1;
        if (!xs)
            pick_tokens(a.M, N, nt, mt);
        if (const char *env = std::getenv("W4A8_W16_MT"))
            mt = std::atoi(env) == 2 ? 2 : 1;
        if (xs)
            mt = 1;
        hipError_t e;
        if (xs)
            e = nt == 4 ? launch_nt<4, 1, true>(a, st)
                        : (nt == 2 ? launch_nt<2, 1, true>(a, st) : launch_nt<1, 1, true>(a, st));
        else if (mt == 2)
            e = nt == 4 ? launch_nt<4, 2, false>(a, st)
                        : (nt == 2 ? launch_nt<2, 2, false>(a, st) : launch_nt<1, 2, false>(a, st));
        else
            e = nt == 4 ? launch_nt<4, 1, false>(a, st)
                        : (nt == 2 ? launch_nt<2, 1, false>(a, st) : launch_nt<1, 1, false>(a, st));
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace w4a8
