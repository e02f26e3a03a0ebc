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
//     operand order of this MFMA (one 16-byte lane load = the two 64-k A
//     operands of one 16-channel tile), so each wave streams its four tiles
//     per group straight into a ring of registers several groups ahead of
//     use and rebuilds them to INT8 there (mask/shift, packed multiply-add,
//     xor: the QServe talk summary's register-level rebuild with subtraction
//     after multiplication).  Every weight byte is read once per workgroup.
//   * Activations go through LDS: the 256 x 128 INT8 tile of group g + 3 is
//     loaded during group g by buffer loads whose destination is the LDS
//     (no registers, no LDS store instructions) into a four-stage ring, and
//     waited for by counted vmcnt at the end of group g + 1, so the stage
//     group g + 2 reads is complete a whole group before it is needed and its
//     first operand reads can be issued before the barrier that ends group
//     g + 1.  Rows are 128 bytes whose eight 16-byte chunks are XOR-swizzled
//     with (row / 2) so the rows one operand load touches spread over the
//     banks; each lane of a load fetches the chunk the swizzle puts at its
//     fixed LDS position.
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
// padded here: a VALU write of a weight operand is separated from its first MFMA
// read by a phase boundary plus s_nop, and the accumulators are read only
// after s_nop padding that covers the MFMA result latency.
//
// Tile order.  Workgroup b runs on XCD b % 8 (round-robin dispatch) and takes
// output tile (b % 8) * per + b / 8, so each XCD works through a contiguous
// range of tiles.  Tiles are numbered in bands of four m-blocks, n-block
// major inside a band, so the workgroups an XCD runs at once cover a few
// m-blocks by several n-blocks and share both operands in that XCD's L2.
#include <algorithm>

#include "kernel_common.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

using dev::kBufFlags;
using dev::rsrc;
constexpr int kXcds = 8;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int TN = 4;                     // 16-channel tiles per wave
constexpr int BN = kWaves * TN * 16;      // channels per workgroup
constexpr int kAStages = 4;               // activation stages in LDS (ring)
constexpr int kAhead = 3;                 // activation operand reads in flight
constexpr int kBandM = 4;                 // m-blocks per band of the tile order

// Shape of one instantiation: TM 16-row tiles per wave (all waves share the
// rows), so a workgroup tile is 16 TM tokens x 256 channels.
template <int TM>
struct Cfg {
    static constexpr int BM = 16 * TM;
    static constexpr int kAStage = BM * 128;                     // bytes of one activation stage
    static constexpr int kXChunks = kAStage / 1024 / kWaves;     // 1 KB LDS loads per wave per group
    static constexpr int kBDepth = TM >= 8 ? 4 : 6;             // weight groups in flight (ring slots)
    static constexpr int kUnroll = TM >= 8 ? 4 : 12;            // groups per main-loop iteration
    static_assert(kUnroll % kBDepth == 0 && kUnroll % 4 == 0,
                  "ring, register and parameter-byte indices are static in the unrolled loop");
    static_assert(kXChunks % 2 == 0, "a wave's first LDS load starts an even 8-row block");
    static_assert(TM % (kAhead + 1) == 0 && TM > kAhead, "the operand-read ring lines up with the phases");
    static_assert(BM <= kThreads && BN == kThreads, "one token scale and one channel scale per thread");
};

// byte offset of 16-byte chunk `ch` (0..7) of activation row `row` (128-byte rows)
__device__ inline int swz(int row, int ch) { return row * 128 + ((ch ^ ((row >> 1) & 7)) << 4); }

// acc += A * B on the matrix cores, accumulator in place in AGPRs.  Both
// operands put row (of A) or column (of B) l % 16 and 16-byte k-block l / 16
// in lane l; the result puts rows 4 (l / 16) .. + 3 of column l % 16 in lane
// l.  The weights are A and the activations B, so the result tile is channels
// x tokens and a lane holds four consecutive channels of one token.
__device__ inline void mfma_acc(v4i &acc, const v4i &a, const v4i &b)
{
    asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Stream-K (a tile's K range split over workgroups) at TM = 4 and 8 only: at
// TM = 16 the accumulators fill the accumulation registers, and the fixup
// path's adds made the compiler spill accumulators inside the main loop.
template <int TM>
constexpr bool kStreamK = TM < 16;

struct PrefillArgs {
    const int8_t *qx;
    const float *s_a;
    const uint8_t *codes;
    const uint8_t *params;
    const uint16_t *s0;
    int64_t M, N, K;
    int mblocks, nblocks;
    int P;             // workgroups with work: each takes a balanced range of (tile, group) units
    int per_xcd;       // launch grid / 8
    uint16_t *y;
    int32_t *acc_out;
    uint32_t *cnt;     // one arrival counter per tile (zero between calls); null: P == tiles
    int32_t *part;     // two partial-accumulator slots per workgroup
};

struct BSlot {
    v4i w[TN];         // packed codes of the wave's four channel tiles for one group
    uint32_t p[TN];    // group-parameter dword (four groups) of the lane's channel
};

// The accumulators, as two arrays: each stays under the size past which the
// compiler leaves a private array in scratch memory.
template <int TM>
struct Acc {
    v4i lo[TM / 2][TN], hi[TM / 2][TN];
    __device__ v4i &operator()(int i, int t) { return i < TM / 2 ? lo[i][t] : hi[i - TM / 2][t]; }
};

template <int TM>
__global__ __launch_bounds__(kThreads, 1) void gemm_prefill_kernel(PrefillArgs a)
{
    using C = Cfg<TM>;
    constexpr int BM = C::BM, kAStage = C::kAStage, kXChunks = C::kXChunks,
                  kBDepth = C::kBDepth, kUnroll = C::kUnroll;
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kDummy = kAStages * kAStage;   // 1 KB never read
    // the tile's token scales and channel scales, for the epilogue
    float *sa_lds = reinterpret_cast<float *>(smem + kDummy + 1024);   // [BM]
    float *s0_lds = sa_lds + BM;                                        // [BN]
    __shared__ uint32_t arrival;

    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);

    // Workgroup b runs on XCD b % 8; it takes range w of the P balanced
    // ranges of (tile, group) units, so each XCD works through contiguous
    // ranges.  With P equal to the tile count every range is one whole tile.
    const int b = blockIdx.x;
    const int w = (b % kXcds) * a.per_xcd + b / kXcds;
    if (w >= a.P)
        return;
    const int K = (int)a.K;
    const int G = K / kGroup;
    const int G4 = (G + 3) / 4 * 4;
    const int ntiles = (int)(a.N / kTileN);
    const int64_t units = (int64_t)a.mblocks * a.nblocks * G;
    auto range_lo = [&](int64_t ww) { return ww * units / a.P; };
    // workgroup whose range holds unit x: the largest ww with range_lo(ww) <= x
    auto owner = [&](int64_t x) { return (int)(((x + 1) * a.P - 1) / units); };
    const int64_t u_lo = range_lo(w), u_hi = range_lo(w + 1);

    // Rows past M and tiles past N fall outside the descriptors' ranges and
    // load as zeros; their outputs are never stored.
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.qx, a.M * a.K);
    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));

    // One segment per tile the range touches: groups [gs, ge) of the tile.
    for (int64_t x = u_lo; x < u_hi;) {
        const int tile = (int)(x / G);
        const int gs = (int)(x - (int64_t)tile * G);
        const int ge = (int)min<int64_t>(G, u_hi - (int64_t)tile * G);
        x = (int64_t)tile * G + ge;

        const int band = tile / (kBandM * a.nblocks);
        const int bm0 = band * kBandM;
        const int bh = min(kBandM, a.mblocks - bm0);
        const int rt = tile - band * kBandM * a.nblocks;
        const int nb = rt / bh;
        const int mb = bm0 + (rt - nb * bh);
        const int m0 = mb * BM;
        const int nt0 = nb * (BN / 16) + wv * TN;   // first device tile of this wave
        const int glast = ge - 1;                    // loads past the segment re-read its last group

        // Lane indices, made opaque per segment so that the compiler derives
        // the per-lane offsets inside the loop instead of keeping dozens of
        // them live (and spilled) across all segments.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int l = tid & 63;
        const int lr = l & 15, lk = l >> 4;      // operand row / 16-byte k-block of this lane

        // Activation tiles go from HBM straight into LDS (buffer loads with
        // the LDS as destination: no registers, no LDS store instructions).
        // Load j of wave wv fills rows 8 J .. 8 J + 7 of a stage (J = kXChunks
        // wv + j), lane l writing position l % 8 of row 8 J + l / 8, so it
        // fetches the chunk the swizzle puts there: (l % 8) ^ ((row / 2) % 8),
        // which depends on J only through its parity.
        const int xq = l >> 3, xp = l & 7;
        const int xoff[2] = {(m0 + xq) * K + 16 * (xp ^ (xq >> 1)),
                             (m0 + xq) * K + 16 * (xp ^ (4 + (xq >> 1)))};
        // weight loads: tile nt0 + t, lane l; parameter dword of channel lr
        const int woff = nt0 * G * kTileBytes + 16 * l;
        const int poff = (nt0 * (G4 / 4) * 16 + lr) * 4;

        __syncthreads();   // the previous segment is done with the LDS
        // this thread's token scale and channel scale (stored to LDS after
        // the loads below)
        const float sa_t = a.s_a[min<int64_t>(m0 + min(tid, BM - 1), a.M - 1)];
        const float s0_t = (float)__builtin_bit_cast(_Float16, a.s0[min<int64_t>((int64_t)nb * BN + tid, a.N - 1)]);

        // Loads of groups past the segment are still issued (so that every
        // group issues the same number of loads and no branch splits the
        // main loop), from the last group into a 1 KB scratch area that
        // nothing reads.
        auto xdma = [&](int stage, bool live, int g, int j) {
            const int J = wv * kXChunks + j;
            const int dst = live ? stage + 1024 * J : kDummy;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(smem + dst), 16, xoff[j & 1],
                8 * J * K + min(g, glast) * kGroup, 0, 0);
        };
        auto bload_t = [&](BSlot &sl, int g, int t) {
            g = min(g, glast);
            sl.w[t] = __builtin_amdgcn_raw_buffer_load_b128(rw, woff, (t * G + g) * kTileBytes, 2);
            sl.p[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, poff, (t * (G4 / 4) + (g >> 2)) * 64, 0);
        };

        Acc<TM> acc;
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int t = 0; t < TN; t++)
                acc(i, t) = v4i{0, 0, 0, 0};

        // lane's activation operand of row tile i, k-half h: row 16 i + lr, chunk
        // 4 h + lk; the swizzle depends only on lr, so tile i is at + 2048 i
        const int aoff[2] = {swz(lr, lk), swz(lr, 4 + lk)};
        // byte offsets of the LDS stages of groups g .. g + 3 (read now, read
        // next, in flight, being loaded); they rotate by one stage per group
        // (uniform, in SGPRs)
        int so_r = 0, so_n = kAStage, so_2 = 2 * kAStage, so_w = 3 * kAStage;
        static_assert(kAStages == 4, "four rotating stage offsets");

        // Per-lane (s1, C) of the four tiles, for groups of either parity:
        // s1 = (p & 15) + 1 and C = 257 (128 - z s1) mod 2^16 from the
        // parameter byte p = (s1 - 1) | (z << 4) (byte g % 4 of the dword).
        // Group g + 1's pairs are computed during group g's first phase.
        uint32_t S1[2][TN], C16[2][TN], sc_p = 0, sc_s1 = 0;

        v4i af[kAhead + 1];   // activation operands in flight (one per row step)
        v4i f0[TN], f1[TN];   // weight operands: current phase / next phase
        uint32_t ru = 0;      // rebuild in progress: masked codes of one dword
        us2 rv = {0, 0};      // ... after the packed multiply-add

        // One phase: the TM x TN MFMAs of k-half h of group g against B
        // operands fc, with three instruction streams spread evenly over the
        // MFMA slots (sched_barrier keeps the program order, so the matrix
        // cores always have the next MFMA while the VALU and memory pipes work):
        //   * rebuild of fn, the next phase's operands (k-half 1 of group g,
        //     then k-half 0 of group g + 1), one dword in three steps: mask,
        //     packed multiply-add, xor 0x80, i.e. (q4 s1 + 128 - z s1) ^ 0x80;
        //   * phase 0: the LDS loads of group g + 3's activations, then group
        //     g + 1's (s1, C) pairs, from ring slot sn;
        //   * phase 1: loads of group g + kBDepth's weights into slot s (loads
        //     leave in the order they are waited for; vmcnt is in-order).
        // The activation operand of row i + kAhead is read at the start of
        // row step i, across phase and group boundaries.  u is the group's
        // position in the unrolled loop; ring and register indices follow it.
        auto phase = [&](const int h, const int u, const v4i (&fc)[TN], v4i (&fn)[TN], BSlot &s,
                         const BSlot &sn, int g) {
            constexpr int kSlots = TM * TN;
            constexpr int kRebuild = 3 * 4 * TN;
            constexpr int kSc = kXChunks + 2 * TN;
            constexpr int kMem = TN;
            const uint8_t *As = smem + so_r + aoff[h];
            const uint8_t *An = h ? smem + so_n + aoff[0] : smem + so_r + aoff[1];
            const bool dma = g + 3 < ge;   // group g + 3 is inside the segment
            // operands being rebuilt: half hn, from slot sb, pairs of parity pr
            const int hn = 1 - h;
            const BSlot &sb = h ? sn : s;
            const int pr = h ? (u + 1) & 1 : u & 1;
            // fc was last written by VALU before the previous phase boundary
            // (or in the prologue: nothing before this point may sink past it)
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("s_nop 4");
#pragma unroll
            for (int k = 0; k < kSlots; k++) {
                const int i = k / TN, t = k % TN;
                const v4i &av = af[i % (kAhead + 1)];
                mfma_acc(acc(i, t), fc[t], av);
                if (t == 0) {
                    const int ir = i + kAhead;
                    af[ir % (kAhead + 1)] = *reinterpret_cast<const v4i *>(
                        ir < TM ? As + 2048 * ir : An + 2048 * (ir - TM));
                }
                // (slot k runs ops [k n / kSlots, (k + 1) n / kSlots) of a
                // stream of n ops: at most ceil(n / kSlots), a constant bound)
#pragma unroll
                for (int q = 0; q < (kRebuild + kSlots - 1) / kSlots; q++) {
                    const int o = k * kRebuild / kSlots + q;
                    if (o >= (k + 1) * kRebuild / kSlots)
                        break;
                    const int j = o / 3, tt = j >> 2, d = j & 3;
                    if (o % 3 == 0) {
                        ru = ((uint32_t)sb.w[tt][d] >> (4 * hn)) & 0x0F0F0F0Fu;
                    } else if (o % 3 == 1) {
                        const us2 Sv = {(unsigned short)S1[pr][tt], (unsigned short)S1[pr][tt]};
                        const us2 Cv = {(unsigned short)C16[pr][tt], (unsigned short)C16[pr][tt]};
                        rv = __builtin_bit_cast(us2, ru) * Sv + Cv;
                    } else {
                        fn[tt][d] = (int)(__builtin_bit_cast(uint32_t, rv) ^ 0x80808080u);
                    }
                }
                if (h == 0) {
#pragma unroll
                    for (int q = 0; q < (kSc + kSlots - 1) / kSlots; q++) {
                        const int o = k * kSc / kSlots + q;
                        if (o >= (k + 1) * kSc / kSlots)
                            break;
                        if (o < kXChunks) {
                            xdma(so_w, dma, g + 3, o);
                            continue;
                        }
                        const int tt = (o - kXChunks) >> 1;
                        if (((o - kXChunks) & 1) == 0) {
                            sc_p = (sn.p[tt] >> (8 * ((g + 1) & 3))) & 0xFFu;
                            sc_s1 = (sc_p & 15u) + 1u;
                        } else {
                            S1[(u + 1) & 1][tt] = sc_s1;
                            C16[(u + 1) & 1][tt] = ((128u - (sc_p >> 4) * sc_s1) * 257u) & 0xFFFFu;
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < (kMem + kSlots - 1) / kSlots; q++) {
                        const int o = k * kMem / kSlots + q;
                        if (o >= (k + 1) * kMem / kSlots)
                            break;
                        bload_t(s, g + kBDepth, o);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // One group g (position u in the unrolled loop) on ring slot s
        // (holding group g) and slot sn (group g + 1), then the barrier.
        // Before it, this wave's LDS loads of group g + 2 (issued in group
        // g - 1, first read at the end of group g + 1) must be complete:
        // vmcnt retires in order, and after them this wave issued group g -
        // 1's weight loads (2 TN), group g + 3's LDS loads (kXChunks) and
        // group g's weight loads (2 TN), so waiting until at most that many
        // remain suffices (more in flight, e.g. right after the
        // prologue, only makes the wait stricter).  Its LDS reads must be
        // complete too, except the kAhead operand reads of the next group,
        // which read a stage completed a group earlier.  The stage read in
        // group g is reloaded in group g + 1, after this barrier.
        auto group = [&](const int u, BSlot &s, BSlot &sn, int g) {
            phase(0, u, f0, f1, s, sn, g);
            phase(1, u, f1, f0, s, sn, g);   // past the segment's end the rebuild is unused
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(%1)\n\ts_barrier" ::"n"(kXChunks + 4 * TN), "n"(kAhead)
                         : "memory");
            const int so = so_r;
            so_r = so_n;
            so_n = so_2;
            so_2 = so_w;
            so_w = so;
        };

        // prologue: groups gs .. gs + 2's activations into LDS, the first
        // kBDepth groups of weights in flight, group gs's (s1, C), first
        // operands and first operand reads.  Each group's weights follow its
        // activations, so the wait below covers only what the first group
        // needs (a wait for three stages and then the first weights made
        // every CU of a round wait for more of the start-up burst)
        BSlot ring[kBDepth];
#pragma unroll
        for (int q = 0; q < 3; q++) {
#pragma unroll
            for (int j = 0; j < kXChunks; j++)
                xdma(q * kAStage, gs + q < ge, gs + q, j);
#pragma unroll
            for (int t = 0; t < TN; t++)
                bload_t(ring[q], gs + q, t);
        }
#pragma unroll
        for (int u = 3; u < kBDepth; u++)
#pragma unroll
            for (int t = 0; t < TN; t++)
                bload_t(ring[u], gs + u, t);
        if (tid < BM)
            sa_lds[tid] = sa_t;
        s0_lds[tid] = s0_t;
        // groups gs and gs + 1 in LDS with group gs's weights (group gs + 1's
        // weights, group gs + 2's LDS loads and the later weights, kXChunks +
        // 2 TN (kBDepth - 1) loads, may still be in flight); the scales
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kXChunks + 2 * TN * (kBDepth - 1))
                     : "memory");
#pragma unroll
        for (int t = 0; t < TN; t++) {
            const uint32_t p = (ring[0].p[t] >> (8 * (gs & 3))) & 0xFFu;
            S1[0][t] = (p & 15u) + 1u;
            C16[0][t] = ((128u - (p >> 4) * S1[0][t]) * 257u) & 0xFFFFu;
            const us2 Sv = {(unsigned short)S1[0][t], (unsigned short)S1[0][t]};
            const us2 Cv = {(unsigned short)C16[0][t], (unsigned short)C16[0][t]};
#pragma unroll
            for (int d = 0; d < 4; d++) {
                const us2 v = __builtin_bit_cast(us2, (uint32_t)ring[0].w[t][d] & 0x0F0F0F0Fu) * Sv + Cv;
                f0[t][d] = (int)(__builtin_bit_cast(uint32_t, v) ^ 0x80808080u);
            }
        }
#pragma unroll
        for (int i = 0; i < kAhead; i++)
            af[i] = *reinterpret_cast<const v4i *>(smem + so_r + aoff[0] + 2048 * i);

        // main loop, unrolled so every ring index is static; the loads are
        // unconditional (clamped to the segment's last group), also in the
        // tail, whose groups may still need weights refilled kBDepth back
        int g = gs;
        for (; g + kUnroll <= ge; g += kUnroll) {
#pragma unroll
            for (int u = 0; u < kUnroll; u++)
                group(u, ring[u % kBDepth], ring[(u + 1) % kBDepth], g + u);
        }
#pragma unroll
        for (int u = 0; u < kUnroll - 1; u++) {
            if (g + u < ge)
                group(u, ring[u % kBDepth], ring[(u + 1) % kBDepth], g + u);
        }
        // the operand reads issued past the segment's end are never used
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

        // MFMA results are read by VALU below: cover the longest result latency
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int t = 0; t < TN; t++)
                asm volatile("" : "+a"(acc(i, t)));

        // ---- a tile split over several ranges: every contributor stores its
        // partial accumulators; the last to arrive adds the others' and runs
        // the epilogue.  Partials move through agent-coherent (sc1) stores and
        // loads; each wave waits for its stores before the barrier, the
        // arrival count is taken after it, and the last arriver's loads are
        // issued after it has seen the final count.  No workgroup waits on
        // another.
        const int c_lo = owner((int64_t)tile * G), c_hi = owner((int64_t)tile * G + G - 1);
        if (kStreamK<TM> && c_lo != c_hi) {
            constexpr int kSlotInts = TM * TN * kWaves * 64 * 4;
            auto slot_of = [&](int ww) {
                const int first = (int)(range_lo(ww) / G);
                return a.part + (size_t)(2 * ww + (first == tile ? 0 : 1)) * kSlotInts;
            };
            const int pbase = ((wv * TM) * TN * 64 + l) * 16;   // lane's bytes in a slot
            {
                const __amdgpu_buffer_rsrc_t rs = rsrc(slot_of(w), (int64_t)kSlotInts * 4);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int t = 0; t < TN; t++)
                        __builtin_amdgcn_raw_buffer_store_b128(acc(i, t), rs, pbase, (i * TN + t) * 1024, 16);
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0)
                arrival = __hip_atomic_fetch_add(a.cnt + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (arrival != (uint32_t)(c_hi - c_lo))
                continue;
            for (int ww = c_lo; ww <= c_hi; ww++) {
                if (ww == w)
                    continue;
                const __amdgpu_buffer_rsrc_t rs = rsrc(slot_of(ww), (int64_t)kSlotInts * 4);
#pragma unroll
                for (int i = 0; i < TM; i++)
#pragma unroll
                    for (int t = 0; t < TN; t++)
                        acc(i, t) += __builtin_amdgcn_raw_buffer_load_b128(rs, pbase, (i * TN + t) * 1024, 16);
            }
            if (tid == 0)
                __hip_atomic_store(a.cnt + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- epilogue.  Lane l holds token row 16 i + l % 16 and channels
        // 16 t + 4 (l / 16) .. + 3 of the wave's slice, so y = fp16((acc s_a)
        // s0) leaves as one 8-byte store of four consecutive channels per
        // (i, t), straight from the registers (the caches merge the four
        // lane groups' 8-byte pieces of a row into whole lines).  The INT32
        // accumulators (an optional output) leave as 16-byte stores.  N is a
        // multiple of 16, so a channel tile is wholly inside or past N.
        const int tn = min(TN, ntiles - nt0);                // the wave's tiles inside N
        const int64_t n0 = (int64_t)nt0 * 16 + 4 * lk;       // lane's first channel in tile 0
        if (a.acc_out) {
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int64_t m = (int64_t)m0 + 16 * i + lr;
#pragma unroll
                for (int t = 0; t < TN; t++)
                    if (t < tn && m < a.M)
                        *reinterpret_cast<v4i *>(a.acc_out + m * a.N + n0 + 16 * t) = acc(i, t);
            }
        }
        // the scales come from LDS: a global load waited for between the
        // stores would also wait for every store issued before it
        v4f s0f[TN];
        float sa[TM];
#pragma unroll
        for (int t = 0; t < TN; t++)
            s0f[t] = *reinterpret_cast<const v4f *>(s0_lds + wv * 64 + 16 * t + 4 * lk);
#pragma unroll
        for (int i = 0; i < TM; i++)
            sa[i] = sa_lds[16 * i + lr];
        auto yval = [&](int i, int t) {
            // the tile stays in the accumulation registers up to here: the
            // compiler would otherwise copy all of them to VGPRs (and spill)
            // right after the main loop
            asm volatile("" : "+a"(acc(i, t)));
            h4 v;
#pragma unroll
            for (int r = 0; r < 4; r++)
                v[r] = (_Float16)(((float)acc(i, t)[r] * sa[i]) * s0f[t][r]);
            return v;
        };
        if (m0 + BM <= a.M && tn == TN) {
            // a whole tile: straight-line code, one row tile at a time (the
            // scheduler would otherwise move every accumulator read up front)
#pragma unroll
            for (int i = 0; i < TM; i++) {
                uint16_t *yr = a.y + ((int64_t)m0 + 16 * i + lr) * a.N + n0;
#pragma unroll
                for (int t = 0; t < TN; t++)
                    *reinterpret_cast<h4 *>(yr + 16 * t) = yval(i, t);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int64_t m = (int64_t)m0 + 16 * i + lr;
#pragma unroll
                for (int t = 0; t < TN; t++)
                    if (t < tn && m < a.M)
                        *reinterpret_cast<h4 *>(a.y + m * a.N + n0 + 16 * t) = yval(i, t);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

template <int TM>
size_t lds_bytes()
{
    return (size_t)kAStages * Cfg<TM>::kAStage + 1024 + (Cfg<TM>::BM + BN) * 4;
}

// The kernel addresses activations with 32-bit buffer offsets, so M is cut
// into launches of at most 2^31 activation bytes each.  P = 0 runs one
// workgroup per tile; P > 0 splits the (tile, group) units into P balanced
// ranges (stream-K), which needs the workspace laid out by prefill_ws_bytes.
template <int TM>
hipError_t launch_tm(int P, const int8_t *qx, const float *s_a, const uint8_t *stream_bytes,
                     const uint16_t *s0, int64_t M, int64_t N, int64_t K, uint16_t *y,
                     int32_t *acc_out, void *ws, hipStream_t st)
{
    constexpr int BM = Cfg<TM>::BM;
    const size_t lds = lds_bytes<TM>();
    const hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(&gemm_prefill_kernel<TM>), (int)lds);
    if (e != hipSuccess)
        return e;
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
        const int64_t tiles = (int64_t)a.mblocks * a.nblocks;
        const int64_t units = tiles * (K / kGroup);
        if (kStreamK<TM> && P > 0 && ws != nullptr && tiles <= kWsCounters) {
            a.P = (int)std::min<int64_t>(P, units);
            a.cnt = reinterpret_cast<uint32_t *>(ws);
            a.part = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(ws) + kWsPartOffset);
        } else {
            a.P = (int)tiles;
            a.cnt = nullptr;
            a.part = nullptr;
        }
        a.per_xcd = (a.P + kXcds - 1) / kXcds;
        hipLaunchKernelGGL(gemm_prefill_kernel<TM>, dim3((unsigned)(a.per_xcd * kXcds)),
                           dim3(kThreads), lds, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace

bool prefill_tm_supported(int tm) { return tm == 4 || tm == 8 || tm == 16; }

size_t prefill_lds_bytes(int tm)
{
    switch (tm) {
    case 4: return lds_bytes<4>();
    case 8: return lds_bytes<8>();
    case 16: return lds_bytes<16>();
    }
    return 0;
}

// Stream-K workspace: the counters (one per tile; at most kWsCounters tiles
// per launch), then two partial-accumulator slots of 16 TM x 256 INT32 per range.
size_t prefill_ws_bytes(int tm, int P, int64_t M, int64_t N, int64_t K)
{
    if (P <= 0 || !prefill_tm_supported(tm) || tm == 16)   // no stream-K at TM = 16
        return 0;
    const int64_t bm = 16 * tm;
    const int64_t rows_max = (0x7FFFFFFF / K - bm) / bm * bm;
    const int64_t tiles = (std::min<int64_t>(M, rows_max) + bm - 1) / bm * ((N + BN - 1) / BN);
    if (tiles > kWsCounters)
        return 0;
    return (size_t)kWsPartOffset + (size_t)2 * P * bm * BN * 4;
}

hipError_t launch_gemm_prefill(const GemmPlan &p, const int8_t *qx, const float *s_a,
                               const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                               int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *ws,
                               hipStream_t st)
{
    const int P = p.splitk > 1 ? p.splitk : 0;
    switch (p.mt) {
    case 4: return launch_tm<4>(P, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
    case 8: return launch_tm<8>(P, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
    case 16: return launch_tm<16>(P, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace w4a8
