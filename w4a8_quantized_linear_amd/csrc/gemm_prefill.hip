// gemm_prefill.hip -- W4A8 GEMM for many tokens (prefill shapes), gfx950.
//
// Same computation as the decode kernel (QServe talk summary, "Quantized
// Matrix Multiplication (GEMM) Kernel on GPUs" and "Challenges and Design
// Details of QServe GEMM Kernel"; Lecture 15 notes, 15.5-15.6):
//   acc[m,n] = sum_k qx[m,k] * (q4[n,k] s1 - z s1)        (exact INT32)
//   y[m,n]   = fp16((float(acc) * s_a[m]) * float(s0[n]))
// but in the regime where the INT8 matrix cores, not HBM, set the pace
// (Lecture 15 notes, Exercise 4: prefill is a compute problem).
//
// Tiling.  A 256-thread workgroup (2 x 2 waves) owns a BM x BN output tile
// and walks K one quantization group (128 k) at a time.  Per step it loads
// the BM x 128 INT8 activation tile and the BN x 128 packed UINT4 weight tile
// (16-byte loads, one device tile lane chunk per load), rebuilds the weights
// to INT8 once for the whole workgroup -- the same packed multiply-add and
// xor as the decode kernel, amortised over BM tokens -- and stores both
// tiles in LDS, double buffered, so the global loads of step g+1 overlap the
// matrix-core work of step g.  Each wave computes a (BM/2) x (BN/2) block with
// v_mfma_i32_32x32x32_i8 (tokens as the A operand, channels as the B
// operand), reading 16-byte operand chunks from LDS; the LDS rows are 128
// bytes with the eight 16-byte chunks of a row XOR-swizzled by the row index
// so that 32 rows read at one chunk position spread over the banks.
//
// XCD-aware order.  Workgroup b runs on XCD b % 8 (round-robin dispatch);
// it takes output tile (b % 8) * per + b / 8, so each XCD works through a
// contiguous, m-block-major range of tiles and its workgroups share the same
// activation rows in that XCD's L2.
#include <algorithm>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBufFlags = 0x00020000;   // raw buffer resource, dword 3 (gfx9 family)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *p, int64_t bytes)
{
    const int64_t lim = bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)lim, kBufFlags);
}

__device__ inline uint32_t rebuild4(uint32_t nib, us2 S, us2 C)
{
    us2 v = __builtin_bit_cast(us2, nib);
    v = v * S + C;
    return __builtin_bit_cast(uint32_t, v) ^ 0x80808080u;
}

// byte offset of 16-byte chunk `ch` (0..7) of LDS row `row` (128-byte rows)
__device__ inline int swz(int row, int ch) { return row * 128 + ((ch ^ (row & 7)) << 4); }

struct PrefillArgs {
    const int8_t *qx;
    const float *s_a;
    const uint8_t *codes;
    const uint8_t *params;
    const uint16_t *s0;
    int64_t M, N, K;
    int mblocks, nblocks, per_xcd;
    uint16_t *y;
    int32_t *acc_out;
};

template <int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_prefill_kernel(PrefillArgs a)
{
    constexpr int WM = BM / 2, WN = BN / 2;          // per-wave block
    constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA tiles per wave
    constexpr int ALD = BM * 128 / (kThreads * 16);  // activation 16-byte loads per thread
    constexpr int BLD = BN / 64;                     // weight 16-byte loads per thread
    constexpr int STAGE = (BM + BN) * 128;           // bytes of one LDS stage

    extern __shared__ __align__(16) uint8_t smem[];
    float *sa_lds = reinterpret_cast<float *>(smem + 2 * STAGE);
    float *s0_lds = sa_lds + BM;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;

    // ---- which tile ----------------------------------------------------------
    const int b = blockIdx.x;
    const int tile = (b % kXcds) * a.per_xcd + b / kXcds;
    if (tile >= a.mblocks * a.nblocks)
        return;
    const int mb = tile / a.nblocks;
    const int nb = tile - mb * a.nblocks;
    const int M = (int)a.M;
    const int K = (int)a.K;
    const int G = K / kGroup;
    const int G4 = (G + 3) / 4 * 4;
    const int ntiles = (int)(a.N / kTileN);
    const int m0 = mb * BM;
    const int nt0 = nb * (BN / 16);

    const __amdgpu_buffer_rsrc_t rx = rsrc(a.qx, (int64_t)a.M * a.K);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));

    // per-thread load assignment: one per-lane base offset, the rest scalar.
    // Rows past M and n-tiles past N fall outside the buffer descriptors'
    // ranges and load as zeros (their outputs are never stored).
    // activations: load i covers block row 32 i + tid / 8, 16-byte chunk tid % 8
    const int xrow0 = tid >> 3, xch = tid & 7;
    const int xoff = (m0 + xrow0) * K + xch * 16;
    // weights: load j covers device tile (4 j + wave) of the block, lane l
    const int cch = l & 15, kb = l >> 4;
    const int woff = (nt0 + wv) * G * kTileBytes + 16 * l;
    const int poff = ((nt0 + wv) * (G4 / 4) * 16 + cch) * 4;

    // epilogue scales of the block into LDS
    for (int i = tid; i < BM; i += kThreads)
        sa_lds[i] = a.s_a[min(m0 + i, M - 1)];
    for (int i = tid; i < BN; i += kThreads)
        s0_lds[i] = (float)__builtin_bit_cast(_Float16, a.s0[min(nt0 * 16 + i, ntiles * 16 - 1)]);

    v4i xr[ALD];
    v4i wr[BLD];
    uint32_t pr[BLD];
    auto gload = [&](int g) {
#pragma unroll
        for (int i = 0; i < ALD; i++)
            xr[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, i * 32 * K + g * kGroup, 0);
#pragma unroll
        for (int j = 0; j < BLD; j++) {
            wr[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff, (4 * j * G + g) * kTileBytes, 2);
            pr[j] = __builtin_amdgcn_raw_buffer_load_b32(rp, poff, (4 * j * (G4 / 4) + (g >> 2)) * 64, 0);
        }
    };
    auto lstore = [&](int stage, int g) {
        uint8_t *As = smem + stage * STAGE;
        uint8_t *Bs = As + BM * 128;
#pragma unroll
        for (int i = 0; i < ALD; i++)
            *reinterpret_cast<v4i *>(As + swz(32 * i + xrow0, xch)) = xr[i];
#pragma unroll
        for (int j = 0; j < BLD; j++) {
            const uint32_t p = (pr[j] >> (8 * (g & 3))) & 0xFFu;
            const uint32_t s1 = (p & 15u) + 1u;
            const unsigned short c16 = (unsigned short)((128u - (p >> 4) * s1) * 257u);
            const us2 S = {(unsigned short)s1, (unsigned short)s1};
            const us2 C = {c16, c16};
            v4i f0, f1;
#pragma unroll
            for (int d = 0; d < 4; d++) {
                const uint32_t x = (uint32_t)wr[j][d];
                f0[d] = (int)rebuild4(x & 0x0F0F0F0Fu, S, C);
                f1[d] = (int)rebuild4((x >> 4) & 0x0F0F0F0Fu, S, C);
            }
            // f0 holds k = 16 kb .. +15 of the group, f1 holds k = 64 + 16 kb .. +15
            const int nrow = (4 * j + wv) * 16 + cch;
            *reinterpret_cast<v4i *>(Bs + swz(nrow, kb)) = f0;
            *reinterpret_cast<v4i *>(Bs + swz(nrow, 4 + kb)) = f1;
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
            acc[i][j] = v16i{};

    // operand rows of this lane inside the stage
    const int lr = l & 31;          // row within a 32-row MFMA tile
    const int lk = l >> 5;          // which 16-byte half of a 32-k chunk

    gload(0);
    lstore(0, 0);
    __syncthreads();

    for (int g = 0; g < G; g++) {
        const int stage = g & 1;
        if (g + 1 < G)
            gload(g + 1);
        const uint8_t *As = smem + stage * STAGE;
        const uint8_t *Bs = As + BM * 128;
#pragma unroll
        for (int kc = 0; kc < 4; kc++) {
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                af[i] = *reinterpret_cast<const v4i *>(As + swz(wm * WM + 32 * i + lr, 2 * kc + lk));
#pragma unroll
            for (int j = 0; j < TN; j++)
                bf[j] = *reinterpret_cast<const v4i *>(Bs + swz(wn * WN + 32 * j + lr, 2 * kc + lk));
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (g + 1 < G)
            lstore(stage ^ 1, g + 1);
        __syncthreads();
    }

    // ---- epilogue: lane l holds column l%32 and rows 8(r/4) + 4(l/32) + r%4 of each tile
#pragma unroll
    for (int i = 0; i < TM; i++) {
#pragma unroll
        for (int j = 0; j < TN; j++) {
            const int nl = wn * WN + 32 * j + lr;           // column within the block
            const int64_t n = (int64_t)nt0 * 16 + nl;
            if (n >= (int64_t)ntiles * 16)
                continue;
            const float s0f = s0_lds[nl];
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int ml = wm * WM + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
                const int64_t m = (int64_t)m0 + ml;
                if (m < a.M) {
                    const int32_t v = acc[i][j][r];
                    const float t = ((float)v * sa_lds[ml]) * s0f;
                    a.y[m * a.N + n] = __builtin_bit_cast(uint16_t, (_Float16)t);
                    if (a.acc_out)
                        a.acc_out[m * a.N + n] = v;
                }
            }
            // one output tile at a time: keeps the scheduler from hoisting the
            // reads of all 256 accumulators at once
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

}  // namespace

size_t prefill_lds_bytes(int bm, int bn) { return (size_t)2 * (bm + bn) * 128 + (bm + bn) * 4; }

template <int BM, int BN>
hipError_t launch_prefill_t(const PrefillArgs &a, hipStream_t st)
{
    static bool attr_set = false;
    const size_t lds = prefill_lds_bytes(BM, BN);
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&gemm_prefill_kernel<BM, BN>),
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    const dim3 grid((unsigned)(a.per_xcd * kXcds));
    hipLaunchKernelGGL((gemm_prefill_kernel<BM, BN>), grid, dim3(kThreads), lds, st, a);
    return hipGetLastError();
}

// The kernel addresses activations with 32-bit buffer offsets, so M is cut
// into launches of at most 2^31 activation bytes each.
hipError_t launch_gemm_prefill(const GemmPlan &p, const int8_t *qx, const float *s_a,
                               const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                               int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, hipStream_t st)
{
    const int bm = p.mt * 16, bn = p.nt * 16;
    const int64_t rows_max = (0x7FFFFFFF / K) / bm * bm;
    for (int64_t r0 = 0; r0 < M; r0 += rows_max) {
        const int64_t mr = std::min<int64_t>(rows_max, M - r0);
        PrefillArgs a;
        a.qx = qx + r0 * K;
        a.s_a = s_a + r0;
        a.codes = stream_bytes;
        a.params = stream_bytes + code_bytes(N, K);
        a.s0 = s0;
        a.M = mr;
        a.N = N;
        a.K = K;
        a.y = y + r0 * N;
        a.acc_out = acc_out ? acc_out + r0 * N : nullptr;
        a.mblocks = (int)((mr + bm - 1) / bm);
        a.nblocks = (int)((N / kTileN * kTileN + bn - 1) / bn);
        const int tiles = a.mblocks * a.nblocks;
        a.per_xcd = (tiles + kXcds - 1) / kXcds;
        hipError_t e;
        if (bm == 256 && bn == 256)
            e = launch_prefill_t<256, 256>(a, st);
        else if (bm == 128 && bn == 128)
            e = launch_prefill_t<128, 128>(a, st);
        else if (bm == 256 && bn == 128)
            e = launch_prefill_t<256, 128>(a, st);
        else if (bm == 128 && bn == 256)
            e = launch_prefill_t<128, 256>(a, st);
        else
            e = hipErrorInvalidValue;
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace w4a8
