// gemm_decode_ns.hip -- decode GEMM whose waves split N, gfx950.
//
// Same arithmetic as gemm_decode.hip (QServe talk summary, "Quantized Matrix
// Multiplication (GEMM) Kernel on GPUs"; the rebuild q4 s1 - z s1 in packed
// 16-bit lanes, INT8 matrix cores, both scales in the epilogue), with another
// work split for several token tiles.  There every wave of a workgroup takes a
// share of the K groups and loads its own activation operands next to its
// weights, so with 2-4 token tiles half of each wave's registers and of its
// memory traffic are activations.  Here the four waves of a workgroup split
// the workgroup's n-tiles (NTW each) and all walk the whole K slice in step:
//  * the activation rows of the workgroup's tokens are copied into LDS, one
//    window of two group pairs (512 bytes per row) at a time, by direct-to-
//    LDS loads shared by the four waves (one 1 KB copy fills two rows),
//    double-buffered: window j + 1 is in flight while window j is used;
//  * each wave streams only weight tiles through its register ring (DEPTH
//    pairs ahead) and keeps only its own accumulators, so no cross-wave
//    reduction is needed;
//  * a window row is stored with its 16-byte chunks XOR-swizzled by the row
//    (chunk k of row r at chunk k ^ (r & 15)), so the 16 token rows a wave
//    reads at one k land in 16 different bank groups.
// Each pair's group-parameter dword (four groups of the lane's channel) rides
// in the weight ring next to the pair's codes and is decoded in registers.
// Split-K across workgroups uses the workspace protocol of gemm_decode.hip:
// per-split partial tiles stored with agent-coherent stores, an arrival
// counter per tile, the last arriver sums the slots in split order.
#include <algorithm>

#include "kernel_common.h"

namespace w4a8 {
namespace {

using namespace dev;

constexpr int kWaves = 4;
constexpr int kWin = 2;                 // group pairs per activation window: 512 bytes per row
constexpr int kRowBytes = 2 * kWin * kGroup;
constexpr int kRowChunks = kRowBytes / 16;

struct NsArgs {
    const int8_t *qx;
    const float *s_a;
    const uint8_t *codes;
    const uint8_t *params;
    const uint16_t *s0;
    int64_t M, N, K;
    int splitk;
    uint16_t *y;
    int32_t *acc_out;
    int32_t *ws_part;
    uint32_t *ws_cnt;
};

// LDS bytes: two activation windows
__host__ __device__ inline int ns_lds_bytes(int MT) { return 2 * 16 * MT * kRowBytes; }

template <int MT, int NTW, int DEPTH>
__global__ __launch_bounds__(64 * kWaves) void gemm_decode_ns_kernel(NsArgs a)
{
    constexpr int NT = kWaves * NTW;          // n-tiles of the workgroup
    constexpr int kRows = 16 * MT;
    constexpr int kWinBytes = kRows * kRowBytes;
    static_assert(kWin % DEPTH == 0, "the ring must cycle within a window");
    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int c = l & 15;
    const int kb = l >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

    const int K = (int)a.K;
    const int G = K / kGroup;
    const int G4 = (G + 3) / 4 * 4;
    const int P = (G + 1) / 2;
    const int ntiles = (int)(a.N / kTileN);
    const int nt0 = (int)blockIdx.x * NT;
    const int64_t m0 = (int64_t)blockIdx.z * kRows;
    const int mrows = (int)min<int64_t>(kRows, a.M - m0);

    const int ps0 = (int)((uint32_t)P * blockIdx.y / (uint32_t)a.splitk);
    const int ps1 = (int)((uint32_t)P * (blockIdx.y + 1) / (uint32_t)a.splitk);
    const int npairs = ps1 - ps0;

    int8_t *win = reinterpret_cast<int8_t *>(smem);

    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.qx + m0 * a.K, (int64_t)mrows * a.K);
    // direct-to-LDS copies use the buffer form: the compiler adds no wait for
    // them before LDS reads (it cannot tell the two window buffers apart), so
    // the waits are the counted ones below

    // one window: row r (a token of the block, clamped to the last real one)
    // takes groups [2 (ps0 + j kWin), +2 kWin) of the slice (clamped to the
    // last group).  Copy i fills rows 2i and 2i + 1 (lanes 0-31, 32-63); the
    // lane that writes chunk k of row r loads source chunk k ^ (r & 15).
    auto window_copy = [&](int j, int buf) {
#pragma unroll
        for (int i0 = 0; i0 < kRows / 2; i0 += kWaves) {
            const int i = i0 + wv;
            const int r = 2 * i + (l >> 5);
            const int srow = min(r, mrows - 1);
            const int chunk = (l & (kRowChunks - 1)) ^ (r & 15);
            const int g = min(2 * (ps0 + j * kWin) + chunk / 8, G - 1);
            lds_copy16(rx, win + buf * kWinBytes + 2 * i * kRowBytes, srow * K + g * kGroup + 16 * (chunk & 7));
        }
    };

    // ---- 1. staging: the first window, then the weight prologue
    window_copy(0, 0);
    __builtin_amdgcn_sched_barrier(0);    // the copies stay ahead of the weight prologue

    int vw[NTW], vp[NTW];
#pragma unroll
    for (int t = 0; t < NTW; t++) {
        vw[t] = min(nt0 + wv * NTW + t, ntiles - 1) * G * kTileBytes + 16 * l;
        vp[t] = min(nt0 + wv * NTW + t, ntiles - 1) * (G4 / 4) * 64 + 4 * c;
    }
    v4i ring[DEPTH][NTW][2];
    uint32_t pring[DEPTH][NTW];       // the pairs' parameter dwords (both groups of a pair in one)
    auto load = [&](v4i (&slot)[NTW][2], uint32_t (&ps)[NTW], int pr) {
        const int q = __builtin_amdgcn_readfirstlane(min(2 * pr, G - 1) >> 2);
#pragma unroll
        for (int t = 0; t < NTW; t++)
            ps[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, vp[t], q * 64, 0);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = __builtin_amdgcn_readfirstlane(min(2 * pr + j, G - 1));
#pragma unroll
            for (int t = 0; t < NTW; t++)
                slot[t][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[t], g * kTileBytes, kLoadNT);
        }
    };
#pragma unroll
    for (int u = 0; u < DEPTH; u++)
        load(ring[u], pring[u], min(ps0 + u, ps1 - 1));

    // this thread's window copies were issued before its weight prologue:
    // they have landed once only the prologue is outstanding
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DEPTH * NTW * 3) : "memory");
    lds_barrier();

    // ---- 2. main loop: windows of kWin pairs ---------------------------------
    v4i acc[NTW][MT];
#pragma unroll
    for (int t = 0; t < NTW; t++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            acc[t][mt] = v4i{0, 0, 0, 0};

    auto compute = [&](const v4i (&slot)[NTW][2], const uint32_t (&ps)[NTW], int pr, const int8_t *wbuf) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = 2 * pr + j;
            if (g >= G)
                break;
            const int gw = g - 2 * ps0;                           // group within the slice
            const int gl = gw % (2 * kWin);                       // group within the window
            v4i xf[MT][2];
#pragma unroll
            for (int mt = 0; mt < MT; mt++) {
                const int8_t *row = wbuf + (16 * mt + c) * kRowBytes;
                xf[mt][0] = *reinterpret_cast<const v4i *>(row + 16 * ((gl * 8 + kb) ^ c));
                xf[mt][1] = *reinterpret_cast<const v4i *>(row + 16 * ((gl * 8 + 4 + kb) ^ c));
            }
#pragma unroll
            for (int t = 0; t < NTW; t++) {
                const uint32_t sc = decode_param((ps[t] >> (8 * (g & 3))) & 0xFFu);
                const us2 S = {(unsigned short)(sc & 0xFFFFu), (unsigned short)(sc & 0xFFFFu)};
                const us2 C = {(unsigned short)(sc >> 16), (unsigned short)(sc >> 16)};
                v4i f0, f1;
                rebuild_tile(slot[t][j], S, C, f0, f1);
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0, xf[mt][0], acc[t][mt], 0, 0, 0);
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f1, xf[mt][1], acc[t][mt], 0, 0, 0);
                }
            }
        }
    };

    const int nwin = (npairs + kWin - 1) / kWin;
    for (int j = 0; j < nwin; j++) {
        const int buf = j & 1;
        // the next window goes into the buffer the previous window used; every
        // wave has left that window (barrier at the end of the last iteration)
        if (j + 1 < nwin)
            window_copy(j + 1, buf ^ 1);
        __builtin_amdgcn_sched_barrier(0);
        const int8_t *wbuf = win + buf * kWinBytes;
#pragma unroll
        for (int u = 0; u < kWin; u++) {
            const int pr = ps0 + j * kWin + u;
            if (pr < ps1)
                compute(ring[u % DEPTH], pring[u % DEPTH], pr, wbuf);
            load(ring[u % DEPTH], pring[u % DEPTH], min(pr + DEPTH, ps1 - 1));
        }
        // window j + 1 (issued before this window's refills) has landed once
        // only the last DEPTH pairs of weights and parameters are outstanding
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DEPTH * NTW * 3) : "memory");
        lds_barrier();
    }

    // ---- 3. outputs: each wave's own tiles ---------------------------------------
    const int64_t tile_id = (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
    SplitTile st;
    st.part = a.ws_part + tile_id * a.splitk * (256 * MT * NT);
    st.cnt = a.ws_cnt + tile_id;
    st.splitk = a.splitk;
    st.slot_elems = 256 * MT * NT;
    st.row_stride = 16 * NT;
    st.m0 = m0;
    st.n0 = (int64_t)nt0 * kTileN;
    st.rows = mrows;
    st.cols = (int)min<int64_t>(NT * kTileN, a.N - st.n0);
#pragma unroll
    for (int t = 0; t < NTW; t++) {
#pragma unroll
        for (int mt = 0; mt < MT; mt++) {
            const int tt = wv * NTW + t;
            const int64_t m = m0 + 16 * mt + c;
            const int64_t n = (int64_t)(nt0 + tt) * kTileN + 4 * kb;
            if (nt0 + tt >= ntiles || m >= a.M)
                continue;
            if (a.splitk > 1)
                splitk_store(st, blockIdx.y, 16 * mt + c, 16 * tt + 4 * kb, acc[t][mt]);
            else
                store_out4(acc[t][mt], a.s_a[m], *reinterpret_cast<const uint2 *>(a.s0 + n), a.y, a.acc_out, m, n,
                           a.N);
        }
    }
    // ---- 4. split-K: the last workgroup of the tile applies the epilogue -------
    if (a.splitk > 1)
        splitk_finish<64 * kWaves>(st, a.s_a, a.s0, a.y, a.acc_out, a.N, tid);
}

template <int MT, int NTW, int DEPTH>
hipError_t launch_ns_t(const GemmPlan &p, const NsArgs &a, size_t lds, hipStream_t st)
{
    if (lds > 64 * 1024) {
        const hipError_t e = raise_lds_limit(reinterpret_cast<const void *>(&gemm_decode_ns_kernel<MT, NTW, DEPTH>),
                                             (int)kDecodeLdsMax);
        if (e != hipSuccess)
            return e;
    }
    dim3 grid((unsigned)p.n_blocks, (unsigned)p.splitk, (unsigned)p.m_blocks);
    hipLaunchKernelGGL((gemm_decode_ns_kernel<MT, NTW, DEPTH>), grid, dim3(64 * kWaves), lds, st, a);
    return hipGetLastError();
}

}  // namespace

// Instantiated (mt, n-tiles per wave, depth) variants of the N-split kernel.
#define W4A8_DECODE_NS_VARIANTS(X) X(1, 1, 2) X(1, 2, 2) X(2, 1, 2) X(2, 2, 2) X(2, 4, 2) X(4, 1, 2) X(4, 2, 2)

bool decode_ns_variant_exists(int mt, int ntw, int depth)
{
#define W4A8_NS_HAS(MT_, NTW_, D_) \
    if (mt == MT_ && ntw == NTW_ && depth == D_) return true;
    W4A8_DECODE_NS_VARIANTS(W4A8_NS_HAS)
#undef W4A8_NS_HAS
    return false;
}

size_t decode_ns_lds_bytes(const GemmPlan &p, int64_t K)
{
    (void)K;
    return (size_t)ns_lds_bytes(p.mt);
}

hipError_t launch_gemm_decode_ns(const GemmPlan &p, const int8_t *qx, const float *s_a, const uint8_t *stream_bytes,
                                 const uint16_t *s0, int64_t M, int64_t N, int64_t K, uint16_t *y, int32_t *acc_out,
                                 void *ws, hipStream_t st)
{
    NsArgs a;
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
    a.ws_part = nullptr;
    a.ws_cnt = nullptr;
    if (p.splitk > 1) {
        a.ws_cnt = reinterpret_cast<uint32_t *>(ws);
        a.ws_part = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(ws) + kWsPartOffset);
    }
    const size_t lds = decode_ns_lds_bytes(p, K);
    if (p.nt % kWaves != 0 || lds == 0 || lds > kDecodeLdsMax)
        return hipErrorInvalidValue;
    const int ntw = p.nt / kWaves;
#define W4A8_NS_CASE(MT_, NTW_, D_)                                 \
    if (p.mt == MT_ && ntw == NTW_ && p.depth == D_ && p.waves == kWaves) \
        return launch_ns_t<MT_, NTW_, D_>(p, a, lds, st);
    W4A8_DECODE_NS_VARIANTS(W4A8_NS_CASE)
#undef W4A8_NS_CASE
    return hipErrorInvalidValue;
}

}  // namespace w4a8
