// gemm_decode.hip -- W4A8 GEMM for few tokens (decode shapes), gfx950.
//
// QServe talk summary, "Quantized Matrix Multiplication (GEMM) Kernel on
// GPUs" and "Challenges and Design Details of QServe GEMM Kernel"; Lecture
// 15 notes, 15.5-15.6.  The main loop streams the UINT4 weights once from HBM,
// rebuilds INT8 weights in registers as q4*s1 - z*s1 (subtraction after
// multiplication), feeds the INT8 matrix cores, and leaves both scales to the
// epilogue:
//   acc[m,n] = sum_k qx[m,k] * (q4[n,k] s1 - z s1)        (exact INT32)
//   y[m,n]   = fp16((float(acc) * s_a[m]) * float(s0[n]))
//
// Work decomposition.  A 256-thread workgroup (4 waves) owns NT n-tiles of 16
// channels, up to MT m-tiles of 16 tokens, and one K slice (split-K).  The
// four waves split the slice into runs of group pairs.  Each wave streams its
// weight tiles from HBM straight into registers with 16-byte non-temporal
// loads, together with the matching activation fragments (tiny, L2-resident)
// and the group-parameter dword, two groups per buffer, double buffered.
// Every load is unconditional (addresses clamped at the edges) so the compiler
// emits exact vmcnt waits and keeps both buffers in flight.  Each 16-byte lane
// load is the fragment pair of two v_mfma_i32_16x16x64_i8 (the device layout
// puts the codes in that order), so there is no shuffling: mask/shift, one
// packed 16-bit multiply-add and one xor per 4 weights, then the MFMA with the
// weights as the A operand (rows = channels) and the tokens as the B operand.
// The four waves' partial accumulators are summed through LDS; with split-K
// the workgroups of one tile add their partials into an INT32 workspace with
// atomics (exact, so any arrival order gives the same bits) and the last to
// arrive applies the epilogue and clears its part of the workspace.
//
// The packed rebuild.  For a dword holding four codes b in [0, 15], one per
// byte, v_pk_mad_u16(x, s1, C) with C = 257 (128 - z s1) mod 2^16 computes in
// each byte b s1 - z s1 + 128, which the protective range keeps in [1, 255],
// so no carry or borrow crosses a byte; xor 0x80808080 then turns each byte
// into the signed INT8 value b s1 - z s1.  Subtracting the zero first would
// put negative values into the packed lanes and borrow across bytes, which is
// the overflow hazard the QServe talk summary attributes to subtraction
// before multiplication.
#include <algorithm>
#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ inline uint32_t rebuild4(uint32_t nib, us2 S, us2 C)
{
    us2 v = __builtin_bit_cast(us2, nib);
    v = v * S + C;
    return __builtin_bit_cast(uint32_t, v) ^ 0x80808080u;
}

__device__ inline v4i load_nt16(const uint8_t *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

struct DecodeArgs {
    const int8_t *qx;
    const float *s_a;
    const uint8_t *codes;
    const uint8_t *params;
    const uint16_t *s0;
    int64_t M, N, K;
    int splitk;
    uint16_t *y;
    int32_t *acc_out;
    int32_t *ws_acc;     // [M, N] int32 (split-K only)
    uint32_t *ws_cnt;    // one counter per (m-block, n-block)
};

// One double-buffer slot: the loads of one pair of groups (2 x 128 k).
template <int MT, int NT>
struct Chunk {
    v4i w[NT][2];       // weight fragments: 16 B per lane per (n-tile, group)
    uint32_t p[NT];     // group-parameter dword (four groups of this lane's channel)
    v4i x[MT][2][2];    // activation fragments: (m-tile, group, 64-k half)
};

template <int MT, int NT>
__global__ __launch_bounds__(kThreads) void gemm_decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    const int l = tid & 63;
    const int c = l & 15;          // weight row (channel) fed / token column read by this lane
    const int kb = l >> 4;         // 16-byte k-block within a 64-k MFMA step

    const int64_t G = num_groups(a.K);
    const int64_t G4 = groups_padded(a.K);
    const int64_t P = (G + 1) / 2;                 // pairs of groups
    const int64_t ntiles_total = a.N / kTileN;
    const int64_t nt0 = (int64_t)blockIdx.x * NT;
    const int s = blockIdx.y;
    const int64_t m0 = (int64_t)blockIdx.z * (16 * MT);
    const int mrows = (int)min<int64_t>(16 * MT, a.M - m0);   // real token rows in this block

    // this workgroup's K slice and this wave's part of it, in pairs of groups
    const int64_t ps0 = P * s / a.splitk;
    const int64_t ps1 = P * (s + 1) / a.splitk;
    const int64_t pw0 = ps0 + (ps1 - ps0) * wv / kWaves;
    const int64_t pw1 = ps0 + (ps1 - ps0) * (wv + 1) / kWaves;

    // per-lane base pointers (tiles past N are clamped to a real tile and never stored)
    const uint8_t *wbase[NT];
    const uint32_t *pbase[NT];
    bool tile_ok[NT];
#pragma unroll
    for (int t = 0; t < NT; t++) {
        tile_ok[t] = (nt0 + t) < ntiles_total;
        const int64_t tt = tile_ok[t] ? nt0 + t : ntiles_total - 1;
        wbase[t] = a.codes + tt * G * kTileBytes + 16 * l;
        pbase[t] = reinterpret_cast<const uint32_t *>(a.params) + (tt * (G4 / 4)) * 16 + c;
    }
    bool row_ok[MT];
    const int8_t *xbase[MT];
#pragma unroll
    for (int mt = 0; mt < MT; mt++) {
        const int r = 16 * mt + c;
        row_ok[mt] = r < mrows;
        xbase[mt] = a.qx + (m0 + (row_ok[mt] ? r : mrows - 1)) * a.K + 16 * kb;
    }

    v4i acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            acc[t][mt] = v4i{0, 0, 0, 0};

    // every load below is unconditional (addresses clamped), so the compiler
    // can keep the whole double buffer in flight with exact vmcnt waits
    auto load = [&](Chunk<MT, NT> &ch, int64_t pr) {
#pragma unroll
        for (int t = 0; t < NT; t++) {
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int64_t g = min<int64_t>(2 * pr + j, G - 1);
                ch.w[t][j] = load_nt16(wbase[t] + g * kTileBytes);
            }
            ch.p[t] = pbase[t][(2 * pr / 4) * 16];
        }
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int64_t g = min<int64_t>(2 * pr + j, G - 1);
                ch.x[mt][j][0] = *reinterpret_cast<const v4i *>(xbase[mt] + g * kGroup);
                ch.x[mt][j][1] = *reinterpret_cast<const v4i *>(xbase[mt] + g * kGroup + 64);
            }
    };

    auto compute = [&](const Chunk<MT, NT> &ch, int64_t pr) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t g = 2 * pr + j;
            if (g >= G)          // odd group count: the pair's second half is padding
                break;
            v4i xf[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; mt++)
#pragma unroll
                for (int h = 0; h < 2; h++)
                    xf[mt][h] = row_ok[mt] ? ch.x[mt][j][h] : v4i{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const uint32_t pb = (ch.p[t] >> (8 * (g & 3))) & 0xFFu;
                const uint32_t s1 = (pb & 15u) + 1u;
                const uint32_t zs = (pb >> 4) * s1;
                const unsigned short cc16 = (unsigned short)((128u - zs) * 257u);
                const us2 S = {(unsigned short)s1, (unsigned short)s1};
                const us2 C = {cc16, cc16};
                const v4i w = ch.w[t][j];
                v4i f0, f1;
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    const uint32_t x = (uint32_t)w[d];
                    f0[d] = (int)rebuild4(x & 0x0F0F0F0Fu, S, C);
                    f1[d] = (int)rebuild4((x >> 4) & 0x0F0F0F0Fu, S, C);
                }
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0, xf[mt][0], acc[t][mt], 0, 0, 0);
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f1, xf[mt][1], acc[t][mt], 0, 0, 0);
                }
            }
        }
    };

    if (pw1 > pw0) {
        Chunk<MT, NT> A, B;
        load(A, pw0);
        int64_t pr = pw0;
        for (; pr + 2 < pw1; pr += 2) {
            load(B, pr + 1);
            compute(A, pr);
            load(A, pr + 2);
            compute(B, pr + 1);
        }
        if (pr + 1 < pw1) {
            load(B, pr + 1);
            compute(A, pr);
            compute(B, pr + 1);
        } else {
            compute(A, pr);
        }
    }

    // ---- sum the four waves' partials through LDS ----------------------------
    v4i *red = reinterpret_cast<v4i *>(smem);   // [kWaves][NT*MT][64]
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            red[(wv * NT * MT + t * MT + mt) * 64 + l] = acc[t][mt];
    __syncthreads();

    const int64_t tile_id = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
    for (int i = wv; i < NT * MT; i += kWaves) {
        const int t = i / MT;
        const int mt = i - t * MT;
        v4i sum = red[i * 64 + l];
#pragma unroll
        for (int w = 1; w < kWaves; w++)
            sum += red[(w * NT * MT + i) * 64 + l];
        const int64_t m = m0 + 16 * mt + c;
        const int64_t n = (nt0 + t) * kTileN + 4 * kb;
        if (!((nt0 + t) < ntiles_total) || m >= a.M)
            continue;
        if (a.splitk > 1) {
#pragma unroll
            for (int r = 0; r < 4; r++)
                atomicAdd(a.ws_acc + m * a.N + n + r, sum[r]);
        } else {
            const float sa = a.s_a[m];
            const uint2 s0p = *reinterpret_cast<const uint2 *>(a.s0 + n);
            const uint32_t s0w[2] = {s0p.x, s0p.y};
            uint32_t out[2];
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
                float v0 = ((float)sum[r] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[r / 2] & 0xFFFF));
                float v1 = ((float)sum[r + 1] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[r / 2] >> 16));
                uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)v0);
                uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)v1);
                out[r / 2] = h0 | (h1 << 16);
            }
            *reinterpret_cast<uint2 *>(a.y + m * a.N + n) = make_uint2(out[0], out[1]);
            if (a.acc_out)
                *reinterpret_cast<v4i *>(a.acc_out + m * a.N + n) = sum;
        }
    }
    if (a.splitk <= 1)
        return;

    // ---- split-K: the last workgroup of the tile applies the epilogue --------
    __threadfence();
    __syncthreads();
    __shared__ uint32_t arrival;
    if (tid == 0)
        arrival = atomicAdd(a.ws_cnt + tile_id, 1u);
    __syncthreads();
    if (arrival != (uint32_t)(a.splitk - 1))
        return;
    __threadfence();
    const int ncols = (int)min<int64_t>(NT * kTileN, a.N - nt0 * kTileN);
    for (int i = tid; i < mrows * ncols / 4; i += kThreads) {
        const int r = i / (ncols / 4);
        const int q = i - r * (ncols / 4);
        const int64_t m = m0 + r;
        const int64_t n = nt0 * kTileN + 4 * q;
        int32_t *wp = a.ws_acc + m * a.N + n;
        v4i sum;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            sum[e] = __hip_atomic_load(wp + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(wp + e, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const float sa = a.s_a[m];
        const uint2 s0p = *reinterpret_cast<const uint2 *>(a.s0 + n);
        const uint32_t s0w[2] = {s0p.x, s0p.y};
        uint32_t out[2];
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            float v0 = ((float)sum[e] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[e / 2] & 0xFFFF));
            float v1 = ((float)sum[e + 1] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[e / 2] >> 16));
            uint32_t h0 = __builtin_bit_cast(uint16_t, (_Float16)v0);
            uint32_t h1 = __builtin_bit_cast(uint16_t, (_Float16)v1);
            out[e / 2] = h0 | (h1 << 16);
        }
        *reinterpret_cast<uint2 *>(a.y + m * a.N + n) = make_uint2(out[0], out[1]);
        if (a.acc_out)
            *reinterpret_cast<v4i *>(a.acc_out + m * a.N + n) = sum;
    }
    if (tid == 0)
        __hip_atomic_store(a.ws_cnt + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int NT>
hipError_t launch_decode_t(const GemmPlan &p, const DecodeArgs &a, size_t lds, hipStream_t st)
{
    dim3 grid((unsigned)p.n_blocks, (unsigned)p.splitk, (unsigned)p.m_blocks);
    hipLaunchKernelGGL((gemm_decode_kernel<MT, NT>), grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

}  // namespace

// Dynamic LDS of one decode workgroup: the cross-wave reduction buffer.
size_t decode_lds_bytes(int64_t M, int64_t K, int mt, int nt, int splitk)
{
    (void)M;
    (void)K;
    (void)splitk;
    return (size_t)kWaves * nt * mt * 64 * 16;
}

hipError_t launch_gemm_decode(const GemmPlan &p, const int8_t *qx, const float *s_a,
                              const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                              int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *ws,
                              hipStream_t st)
{
    DecodeArgs a;
    a.qx = qx;
    a.s_a = s_a;
    a.codes = stream_bytes;
    a.params = stream_bytes + code_bytes(N, K);
    a.s0 = s0;
    a.M = M;
    a.N = N;
    a.K = K;
    a.splitk = p.splitk;
    a.y = y;
    a.acc_out = acc_out;
    a.ws_acc = nullptr;
    a.ws_cnt = nullptr;
    if (p.splitk > 1) {
        a.ws_acc = reinterpret_cast<int32_t *>(ws);
        size_t acc_bytes = ((size_t)M * N * 4 + 255) / 256 * 256;
        a.ws_cnt = reinterpret_cast<uint32_t *>(reinterpret_cast<uint8_t *>(ws) + acc_bytes);
    }
    const size_t lds = decode_lds_bytes(M, K, p.mt, p.nt, p.splitk);
#define W4A8_DECODE_CASE(MT_, NT_) \
    if (p.mt == MT_ && p.nt == NT_) return launch_decode_t<MT_, NT_>(p, a, lds, st);
    W4A8_DECODE_CASE(1, 1)
    W4A8_DECODE_CASE(1, 2)
    W4A8_DECODE_CASE(1, 4)
    W4A8_DECODE_CASE(2, 1)
    W4A8_DECODE_CASE(2, 2)
    W4A8_DECODE_CASE(2, 4)
    W4A8_DECODE_CASE(4, 1)
    W4A8_DECODE_CASE(4, 2)
    W4A8_DECODE_CASE(4, 4)
#undef W4A8_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace w4a8
