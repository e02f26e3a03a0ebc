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
// Tiling.  A workgroup of 4 waves (one per SIMD, each with the full 512-entry
// register file) owns a 256-token x 256-channel output tile and walks K one
// quantization group (128 k) at a time.  Wave w computes all 256 tokens x
// channels [64 w, 64 w + 64) of the tile with v_mfma_i32_16x16x64_i8; its 64
// 16x16 INT32 accumulator tiles fill the 256 accumulation registers.
//   * Weights never touch LDS.  The device weight stream is already in the
//     operand order of this MFMA (one 16-byte lane load = the two 64-k B
//     operands of one 16-channel tile), so each wave streams its four tiles
//     per group straight into a ring of registers several groups ahead of
//     use and rebuilds them to INT8 there (mask/shift, packed multiply-add,
//     xor: the QServe talk summary's register-level rebuild with subtraction
//     after multiplication).  Every weight byte is read once per workgroup.
//   * Activations go through LDS: the 256 x 128 INT8 tile of group g + 3 is
//     loaded into registers during group g and stored during group g + 1
//     into a three-stage LDS ring, so the stage group g + 1 reads is complete
//     a whole group before it is needed and its first operand reads can be
//     issued before the barrier that ends group g.  Rows are 128 bytes whose
//     eight 16-byte chunks are XOR-swizzled with (row / 2) so the rows one
//     operand load touches spread over the banks.
//   * A group is two phases, one per 64-k half, of 16 row steps each.  A row
//     step issues the LDS read of the activation operand three steps ahead,
//     four MFMAs, and the VALU rebuild of one dword of the next phase's B
//     operands, so the rebuild and the LDS latency hide under the matrix
//     cores.  With one wave per SIMD, all latency is hidden by issuing work
//     ahead, never by other waves.
//
// The MFMAs are issued through inline assembly with the accumulator tied in
// place in the accumulation registers: the compiler's own lowering of this
// MFMA copies accumulators between register files on every step.  The
// compiler does not see these as MFMAs, so the hazards it would pad are
// padded here: a VALU write of a B operand is separated from its first MFMA
// read by a phase boundary plus s_nop, and the accumulators are read only
// after s_nop padding that covers the MFMA result latency.
//
// Tile order.  Workgroup b runs on XCD b % 8 (round-robin dispatch) and takes
// output tile (b % 8) * per + b / 8, so each XCD works through a contiguous
// range of tiles.  Tiles are numbered in bands of four m-blocks, n-block
// major inside a band, so the workgroups an XCD runs at once cover a few
// m-blocks by several n-blocks and share both operands in that XCD's L2.
#include <algorithm>

#include "w4a8_internal.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBufFlags = 0x00020000;   // raw buffer resource, dword 3 (gfx9 family)
constexpr int kXcds = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int BM = 256, BN = 256;         // workgroup tile
constexpr int TM = 16, TN = 4;            // 16x16 MFMA tiles per wave (256 x 64)
constexpr int kAStage = BM * 128;         // bytes of one activation stage
constexpr int kAStages = 3;               // activation stages in LDS (ring)
constexpr int kXChunks = kAStage / 16 / kThreads;   // 16-byte activation loads per thread per group
constexpr int kBandM = 4;                 // m-blocks per band of the tile order
constexpr int kBDepth = 4;                // weight groups in flight per wave (ring slots)
constexpr int kAhead = 3;                 // activation operand reads in flight
static_assert(TM == 4 * TN, "one B-operand dword is rebuilt per row step");
static_assert(kXChunks + kXChunks / 2 + TN <= TM, "phase 1 has a row step for every transfer");
static_assert(TM % (kAhead + 1) == 0, "the operand-read ring lines up with the phases");

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *p, int64_t bytes)
{
    const int64_t lim = bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)lim, kBufFlags);
}

// byte offset of 16-byte chunk `ch` (0..7) of activation row `row` (128-byte rows)
__device__ inline int swz(int row, int ch) { return row * 128 + ((ch ^ ((row >> 1) & 7)) << 4); }

// acc += A * B on the matrix cores, accumulator in place in AGPRs
__device__ inline void mfma_acc(v4i &acc, const v4i &a, const v4i &b)
{
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

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

struct BSlot {
    v4i w[TN];         // packed codes of the wave's four channel tiles for one group
    uint32_t p[TN];    // group-parameter dword (four groups) of the lane's channel
};

// The accumulators, as two arrays of 32 tiles: kept under the size past which
// the compiler leaves a private array in scratch memory.
struct Acc {
    v4i lo[TM / 2][TN], hi[TM / 2][TN];
    __device__ v4i &operator()(int i, int t) { return i < TM / 2 ? lo[i][t] : hi[i - TM / 2][t]; }
};

__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(PrefillArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    float *sa_lds = reinterpret_cast<float *>(smem + kAStages * kAStage);

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = l & 15, lk = l >> 4;      // operand row / 16-byte k-block of this lane

    const int b = blockIdx.x;
    const int tile = (b % kXcds) * a.per_xcd + b / kXcds;
    if (tile >= a.mblocks * a.nblocks)
        return;
    const int band = tile / (kBandM * a.nblocks);
    const int bm0 = band * kBandM;
    const int bh = min(kBandM, a.mblocks - bm0);
    const int rt = tile - band * kBandM * a.nblocks;
    const int nb = rt / bh;
    const int mb = bm0 + (rt - nb * bh);
    const int K = (int)a.K;
    const int G = K / kGroup;
    const int G4 = (G + 3) / 4 * 4;
    const int ntiles = (int)(a.N / kTileN);
    const int m0 = mb * BM;
    const int nt0 = nb * (BN / 16) + wv * TN;   // first device tile of this wave

    // Rows past M and tiles past N fall outside the descriptors' ranges and
    // load as zeros; their outputs are never stored.
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.qx, a.M * a.K);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));

    // activation tile loads: load j covers block row 32 j + tid / 8, chunk tid % 8
    const int xrow0 = tid >> 3, xch = tid & 7;
    const int xoff = (m0 + xrow0) * K + xch * 16;
    // weight loads: tile nt0 + t, lane l; parameter dword of channel lr
    const int woff = nt0 * G * kTileBytes + 16 * l;
    const int poff = (nt0 * (G4 / 4) * 16 + lr) * 4;

    for (int i = tid; i < BM; i += kThreads)
        sa_lds[i] = a.s_a[min<int64_t>(m0 + i, a.M - 1)];

    v4i xr[kXChunks];
    auto aload = [&](int g) {
        g = min(g, G - 1);                   // the last loads re-read a real group
#pragma unroll
        for (int j = 0; j < kXChunks; j++)
            xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, j * (kThreads / 8) * K + g * kGroup, 0);
    };
    auto astore = [&](int stage) {
        uint8_t *As = smem + stage * kAStage;
#pragma unroll
        for (int j = 0; j < kXChunks; j++)
            *reinterpret_cast<v4i *>(As + swz(j * (kThreads / 8) + xrow0, xch)) = xr[j];
    };
    auto bload = [&](BSlot &s, int g) {
        g = min(g, G - 1);
#pragma unroll
        for (int t = 0; t < TN; t++) {
            s.w[t] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff, (t * G + g) * kTileBytes, 2);
            s.p[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, poff, (t * (G4 / 4) + (g >> 2)) * 64, 0);
        }
    };
    Acc acc;
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int t = 0; t < TN; t++)
            acc(i, t) = v4i{0, 0, 0, 0};

    // lane's activation operand of row tile i, k-half h: row 16 i + lr, chunk
    // 4 h + lk; the swizzle depends only on lr, so tile i is at + 2048 i
    const int aoff[2] = {swz(lr, lk), swz(lr, 4 + lk)};
    // byte offsets of the LDS stages read in this group, read next and
    // written now; they rotate by one stage per group (uniform, in SGPRs)
    int so_r = 0, so_n = kAStage, so_w = 2 * kAStage;
    static_assert(kAStages == 3, "three rotating stage offsets");

    // Per-lane (s1, C) of the four tiles for the group being rebuilt:
    // s1 = (p & 15) + 1 and C = 257 (128 - z s1) mod 2^16 from the parameter
    // byte p = (s1 - 1) | (z << 4).  Each group's pair is computed once, in
    // two halves (sc_a, sc_b) placed in different row steps.
    uint32_t S1[TN], C16[TN], sc_p = 0, sc_s1 = 0;
    auto sc_a = [&](const BSlot &s, int g, int t) {
        sc_p = (s.p[t] >> (8 * (g & 3))) & 0xFFu;
        sc_s1 = (sc_p & 15u) + 1u;
    };
    auto sc_b = [&](int t) {
        S1[t] = sc_s1;
        C16[t] = ((128u - (sc_p >> 4) * sc_s1) * 257u) & 0xFFFFu;
    };

    v4i af[kAhead + 1];   // activation operands in flight (one per row step)

    // One phase: the MFMAs of k-half h of group g against B operands fc,
    // interleaved one by one with the VALU rebuild of fn = the B operands of
    // the next phase (k-half 1 of group g, then k-half 0 of group g + 1, from
    // ring slot sb), the (s1, C) pairs of group g + 1 (from slot sn), and in
    // phase 1 with the LDS stores of group g + 2's activations, the loads of
    // group g + 3's and the loads of group g + kBDepth's weights into slot s.
    // Rebuild of dword (t, d): mask, packed multiply-add, xor 0x80, i.e.
    // (q4 s1 + 128 - z s1) ^ 0x80 per byte.  The operand reads run kAhead
    // row steps ahead, across phase and group boundaries.  sched_barrier
    // keeps the program order, so the matrix cores always have the next MFMA
    // while the VALU works.
    auto phase = [&](const int h, const v4i (&fc)[TN], v4i (&fn)[TN], const BSlot &sb,
                     const BSlot &sn, int g, BSlot *refill) {
        const uint8_t *As = smem + so_r + aoff[h];
        const uint8_t *An = h ? smem + so_n + aoff[0] : smem + so_r + aoff[1];
        uint8_t *Ad = smem + so_w;
        const int hn = 1 - h;
        // fc was last written by VALU before the previous phase boundary
        asm volatile("s_nop 4");
#pragma unroll
        for (int i = 0; i < TM; i++) {
            const int t = i >> 2, d = i & 3;
            const v4i &a = af[i % (kAhead + 1)];
            mfma_acc(acc(i, 0), a, fc[0]);
            {
                const int ir = i + kAhead;
                af[ir % (kAhead + 1)] = *reinterpret_cast<const v4i *>(
                    ir < TM ? As + 2048 * ir : An + 2048 * (ir - TM));
            }
            // (s1, C) of group g + 1: tile 0 at the end of phase 0, tile
            // t + 1 during tile t's steps of phase 1
            if (h == 0 && i == TM - 3)
                sc_a(sn, g + 1, 0);
            if (h == 1 && d == 1 && t + 1 < TN)
                sc_a(sn, g + 1, t + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_acc(acc(i, 1), a, fc[1]);
            const uint32_t u = ((uint32_t)sb.w[t][d] >> (4 * hn)) & 0x0F0F0F0Fu;
            if (h == 0 && i == TM - 2)
                sc_b(0);
            if (h == 1 && d == 2 && t + 1 < TN)
                sc_b(t + 1);
            __builtin_amdgcn_sched_barrier(0);
            mfma_acc(acc(i, 2), a, fc[2]);
            const us2 S = {(unsigned short)S1[t], (unsigned short)S1[t]};
            const us2 C = {(unsigned short)C16[t], (unsigned short)C16[t]};
            const us2 v = __builtin_bit_cast(us2, u) * S + C;
            if (h == 1) {
                if (i < kXChunks) {
                    *reinterpret_cast<v4i *>(Ad + swz(i * (kThreads / 8) + xrow0, xch)) = xr[i];
                } else if (i < kXChunks + kXChunks / 2) {
                    const int j = 2 * (i - kXChunks);
                    const int ga = min(g + 3, G - 1);
                    xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, j * (kThreads / 8) * K + ga * kGroup, 0);
                    xr[j + 1] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, (j + 1) * (kThreads / 8) * K + ga * kGroup, 0);
                } else if (refill) {
                    const int tb = i - (kXChunks + kXChunks / 2);
                    if (tb < TN) {
                        const int gb = min(g + kBDepth, G - 1);
                        refill->w[tb] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff, (tb * G + gb) * kTileBytes, 2);
                        refill->p[tb] = __builtin_amdgcn_raw_buffer_load_b32(rp, poff, (tb * (G4 / 4) + (gb >> 2)) * 64, 0);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            mfma_acc(acc(i, 3), a, fc[3]);
            fn[t][d] = (int)(__builtin_bit_cast(uint32_t, v) ^ 0x80808080u);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // One group g on ring slot s (holding group g) and slot sn (group g + 1),
    // then the barrier.  Before it, this wave's LDS stores must be complete
    // (the oldest LDS operations: everything but the kAhead operand reads of
    // the next group, which read a stage completed a group earlier).  The
    // stores of group g land in stage (g + 2) % 3, first read at the end of
    // group g + 1; the stage read in group g is rewritten in group g + 1.
    v4i f0[TN], f1[TN];
    auto group = [&](BSlot &s, const BSlot &sn, int g, bool refill) {
        phase(0, f0, f1, s, sn, g, nullptr);
        phase(1, f1, f0, sn, sn, g, refill ? &s : nullptr);
        asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(kAhead) : "memory");
        const int so = so_r;
        so_r = so_n;
        so_n = so_w;
        so_w = so;
    };

    // prologue: groups 0 and 1's activations into LDS, group 2's in
    // registers, the first kBDepth groups of weights in flight, group 0's
    // (s1, C), first operands and first activation operand reads
    BSlot ring[kBDepth];
    aload(0);
    astore(0);
    aload(1);
    astore(1);
    aload(2);
#pragma unroll
    for (int u = 0; u < kBDepth; u++)
        bload(ring[u], u);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TN; t++) {
        sc_a(ring[0], 0, t);
        sc_b(t);
        const us2 S = {(unsigned short)S1[t], (unsigned short)S1[t]};
        const us2 C = {(unsigned short)C16[t], (unsigned short)C16[t]};
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const us2 v = __builtin_bit_cast(us2, (uint32_t)ring[0].w[t][d] & 0x0F0F0F0Fu) * S + C;
            f0[t][d] = (int)(__builtin_bit_cast(uint32_t, v) ^ 0x80808080u);
        }
    }
#pragma unroll
    for (int i = 0; i < kAhead; i++)
        af[i] = *reinterpret_cast<const v4i *>(smem + so_r + aoff[0] + 2048 * i);

    // main loop, unrolled by the ring size so every slot index is static; the
    // loads are unconditional (clamped at the end), so the waits are exact
    int g = 0;
    for (; g + kBDepth <= G; g += kBDepth) {
#pragma unroll
        for (int u = 0; u < kBDepth; u++)
            group(ring[u], ring[(u + 1) % kBDepth], g + u, true);
    }
#pragma unroll
    for (int u = 0; u < kBDepth - 1; u++) {
        if (g + u < G)
            group(ring[u], ring[(u + 1) % kBDepth], g + u, false);
    }
    // the operand reads issued for group G (past the end) are never used
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    // MFMA results are read by VALU below: cover the longest result latency
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");

    // ---- epilogue.  Lane l holds rows 16 i + 4 (l / 16) + r, column
    // 16 t + l % 16 of the wave's slice.  y = fp16((acc s_a) s0) goes through
    // LDS, half a tile (128 rows) at a time, so that global stores are whole
    // 16-byte pieces of output rows; the stages are free once every wave has
    // passed the barrier.  The INT32 accumulators (an optional output) are
    // stored directly.
    float s0f[TN];
#pragma unroll
    for (int t = 0; t < TN; t++)
        s0f[t] = (float)__builtin_bit_cast(_Float16, a.s0[min(nt0 + t, ntiles - 1) * 16 + lr]);
    if (a.acc_out) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
            for (int t = 0; t < TN; t++) {
                const int64_t n = (int64_t)(nt0 + t) * 16 + lr;
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int64_t m = (int64_t)m0 + 16 * i + 4 * lk + r;
                    if (nt0 + t < ntiles && m < a.M)
                        a.acc_out[m * a.N + n] = acc(i, t)[r];
                }
            }
        }
    }
    constexpr int kYRow = BN * 2 + 16;    // padded LDS row of the fp16 tile (bytes)
    constexpr int kHalf = BM / 2;
    static_assert(kHalf * kYRow <= kAStages * kAStage, "output half-tile fits in the stages");
    const int ncol0 = nb * BN;              // first output column of the tile
    __syncthreads();
#pragma unroll
    for (int half = 0; half < 2; half++) {
#pragma unroll
        for (int ii = 0; ii < TM / 2; ii++) {
            const int i = half * (TM / 2) + ii;
#pragma unroll
            for (int t = 0; t < TN; t++) {
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int ml = 16 * i + 4 * lk + r;
                    const float yv = ((float)acc(i, t)[r] * sa_lds[ml]) * s0f[t];
                    *reinterpret_cast<_Float16 *>(smem + (ml - half * kHalf) * kYRow +
                                                  (wv * 64 + 16 * t + lr) * 2) = (_Float16)yv;
                }
            }
        }
        __syncthreads();
        // 128 rows x 32 pieces of 16 bytes; N is a multiple of 16, so a
        // piece is wholly inside or wholly past the last column
#pragma unroll 4
        for (int c = tid; c < kHalf * (BN / 8); c += kThreads) {
            const int row = c / (BN / 8), pc = c % (BN / 8);
            const int64_t m = (int64_t)m0 + half * kHalf + row;
            const int64_t n = (int64_t)ncol0 + 8 * pc;
            if (m < a.M && n < a.N)
                *reinterpret_cast<v4i *>(a.y + m * a.N + n) =
                    *reinterpret_cast<const v4i *>(smem + row * kYRow + 16 * pc);
        }
        __syncthreads();
    }
}

}  // namespace

size_t prefill_lds_bytes() { return (size_t)kAStages * kAStage + BM * 4; }

// The kernel addresses activations with 32-bit buffer offsets, so M is cut
// into launches of at most 2^31 activation bytes each.
hipError_t launch_gemm_prefill(const GemmPlan &p, const int8_t *qx, const float *s_a,
                               const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                               int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, hipStream_t st)
{
    (void)p;
    static bool attr_set = false;
    const size_t lds = prefill_lds_bytes();
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&gemm_prefill_kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    // (rows of the last block may reach BM past M, whose offsets must not wrap)
    const int64_t rows_max = (0x7FFFFFFF / K - BM) / BM * BM;
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
        a.mblocks = (int)((mr + BM - 1) / BM);
        a.nblocks = (int)((N + BN - 1) / BN);
        const int tiles = a.mblocks * a.nblocks;
        a.per_xcd = (tiles + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(gemm_prefill_kernel, dim3((unsigned)(a.per_xcd * kXcds)),
                           dim3(kThreads), lds, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace w4a8
