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
// Work decomposition.  A workgroup of WAVES waves owns NT n-tiles of 16
// channels, up to MT m-tiles of 16 tokens, and one K slice (split-K across
// workgroups is optional).  The waves split the slice into runs of group
// pairs.  At the start every thread issues its share of the small loads --
// the epilogue scales and, for few tokens, the tokens' activation rows,
// copied straight into LDS -- then the first DEPTH pairs of its wave's
// weight tiles.  Each pair's group-parameter dword (four groups of the lane's
// channel) is loaded with the pair's weights and decoded in registers, so no
// workgroup waits for a parameter table before its first MFMA: a table staged
// in LDS had put an HBM round trip and two barriers in front of every
// workgroup's main loop, and all workgroups of a decode launch run that
// prologue at the same time.  Activation operands for more tokens are loaded
// with the weights as well.  Weight
// tiles are read with 16-byte buffer loads (scalar base and offset, one
// per-lane offset register) DEPTH pairs ahead of use; every load is
// unconditional, so the compiler's vmcnt waits are exact.  An unstaged
// activation operand is the 16 bytes of row c at k-block kb, four lanes per
// row 16 lanes apart: as loaded, the 64 lanes touch 16 rows in 64 separate
// cache accesses.  With more than 8 tokens the lanes instead load the block
// row by row (lane 4 r + q takes row r, 16-byte piece q, so four neighbouring
// lanes read 64 contiguous bytes) and ds_bpermute hands each lane the piece
// its MFMA position needs, four dwords per operand.  Each 16-byte lane
// load is the operand pair of two v_mfma_i32_16x16x64_i8 (the device layout
// puts the codes in that order): mask/shift, one packed 16-bit multiply-add
// and one xor per 4 weights, then the MFMA with the weights as the A operand
// (rows = channels) and the tokens as the B operand (columns = tokens; columns
// past M carry whatever row their lane loads and are never stored).  The
// waves' partial accumulators meet in LDS through LDS atomics; with split-K
// each workgroup of a tile stores its partial into its own workspace slot and
// the last to arrive adds the slots in split order and applies the epilogue
// (kernel_common.h, splitk_finish).  The packed rebuild and its byte-lane
// arithmetic are described at rebuild4 in kernel_common.h.
#include <algorithm>
#include <cstdlib>

#include "kernel_common.h"

namespace w4a8 {
namespace {

using namespace dev;

__device__ inline int sgpr(int64_t v) { return __builtin_amdgcn_readfirstlane((int)v); }

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
    int32_t *ws_part;    // split-K partial tiles: slot (tile, split) of 16 MT x 16 NT int32
    uint32_t *ws_cnt;    // one arrival counter per (m-block, n-block)
    int cx;             // unstaged activation operands: row-contiguous loads, lanes exchanged
};

// One ring slot: the loads of one pair of groups (2 x 128 k).
template <int MT, int NT, bool XS>
struct Chunk {
    v4i w[NT][2];                    // weight operands: 16 B per lane per (n-tile, group)
    uint32_t p[NT];                  // parameter dword of the lane's channel (four groups)
    v4i x[XS ? 1 : MT][2][2];        // activation operands when not staged in LDS
};

template <int MT, int NT, int WAVES, int DEPTH, bool XS>
__global__ __launch_bounds__(64 * WAVES) void gemm_decode_kernel(DecodeArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kThreads = 64 * WAVES;

    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int c = l & 15;                    // channel row (A) / token column (B) of this lane
    const int kb = l >> 4;                   // 16-byte k-block within a 64-k MFMA step
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);

    // index arithmetic in 32 bits (shapes are validated on the host: K < 2^24,
    // N < 2^30, weight stream < 2^31 bytes); 64-bit division would cost
    // hundreds of instructions before the first load
    const int K = (int)a.K;
    const int G = K / kGroup;
    const int G4 = (G + 3) / 4 * 4;
    const int P = (G + 1) / 2;               // pairs of groups
    const int ntiles = (int)(a.N / kTileN);
    const int nt0 = (int)blockIdx.x * NT;
    const int64_t m0 = (int64_t)blockIdx.z * (16 * MT);
    const int mrows = (int)min<int64_t>(16 * MT, a.M - m0);

    // K slice of this workgroup and this wave's pairs (all uniform)
    const int ps0 = (int)((uint32_t)P * blockIdx.y / (uint32_t)a.splitk);
    const int ps1 = (int)((uint32_t)P * (blockIdx.y + 1) / (uint32_t)a.splitk);
    const int pw0 = ps0 + (ps1 - ps0) * wv / WAVES;
    const int pw1 = ps0 + (ps1 - ps0) * (wv + 1) / WAVES;
    const int gbase = 2 * ps0;                          // first group of the slice
    const int span = min(2 * (ps1 - ps0), G - gbase);   // groups in the slice

    // LDS: reduction [NT*MT][4][64] int32 | activation rows [mrows][span*128 + 16]
    // (rounded up to whole copy chunks)
    const int xstride = span * kGroup + 16;
    int32_t *red = reinterpret_cast<int32_t *>(smem);
    int8_t *xlds = reinterpret_cast<int8_t *>(smem + NT * MT * 1024);

    const __amdgpu_buffer_rsrc_t rw = rsrc(a.codes, code_bytes(a.N, a.K));
    const __amdgpu_buffer_rsrc_t rp = rsrc(a.params, param_bytes(a.N, a.K));
    const int8_t *xblk = a.qx + m0 * a.K;     // this block's first token row
    const __amdgpu_buffer_rsrc_t rx = rsrc(xblk, (int64_t)mrows * a.K);

    // ---- 1. staging: (few tokens) the activation rows go straight from
    // memory to LDS, exact counts, issued before the weights.  The copies are
    // the buffer form of the direct-to-LDS load: the compiler adds no wait for
    // them before LDS reads, so the counted wait below decides, and the
    // weights issued after them are not waited for.
    if constexpr (XS) {
        const int xbytes = mrows * xstride;
        for (int ch = wv; ch < (xbytes + 1023) / 1024; ch += WAVES) {
            const int o = ch * 1024 + 16 * l;
            const int row = o / xstride;
            const int col = o - row * xstride;
            const bool ok = row < mrows && col < span * kGroup;
            lds_copy16(rx, xlds + ch * 1024, ok ? row * K + gbase * kGroup + col : 0);
        }
    }
    // epilogue scales of this wave's first output tile (waves without a tile skip them)
    const int i0 = wv < NT * MT ? wv : 0;
    const int t_e = i0 / MT, mt_e = i0 - (i0 / MT) * MT;
    const int64_t m_e = min<int64_t>(m0 + 16 * mt_e + c, a.M - 1);
    const int64_t n_e = (int64_t)min(nt0 + t_e, ntiles - 1) * kTileN + 4 * kb;
    float sa_e = 0.0f;
    uint2 s0_e = make_uint2(0, 0);
    if (wv < NT * MT) {
        sa_e = a.s_a[m_e];
        s0_e = *reinterpret_cast<const uint2 *>(a.s0 + n_e);
    }
    __builtin_amdgcn_sched_barrier(0);    // all of the above is issued before the weights

    // ---- 2. the weight stream: DEPTH pairs in flight per wave -----------------
    int vw[NT];                         // per-lane byte offset of each tile's stream
    int vp[NT];                         // ... and of its parameter dwords (channel c)
#pragma unroll
    for (int t = 0; t < NT; t++) {
        vw[t] = min(nt0 + t, ntiles - 1) * G * kTileBytes + 16 * l;
        vp[t] = min(nt0 + t, ntiles - 1) * (G4 / 4) * 64 + 4 * c;
    }
    int vx[XS ? 1 : MT];                // per-lane offset of the activation operand row
#pragma unroll
    for (int mt = 0; mt < (XS ? 1 : MT); mt++)
        vx[mt] = a.cx ? min(16 * mt + (l >> 2), mrows - 1) * K + 16 * (l & 3)
                      : min(16 * mt + c, mrows - 1) * K + 16 * kb;
    const int xsrc = 4 * (4 * c + kb);      // cx: the lane that loaded this lane's operand

    // a pair's parameter bytes ride with its weights: both groups of a pair
    // are in one dword (four groups per dword, pairs start at even groups)
    auto load = [&](Chunk<MT, NT, XS> &ch, int pr) {
        const int q = sgpr(min(2 * pr, G - 1) >> 2);
#pragma unroll
        for (int t = 0; t < NT; t++)
            ch.p[t] = __builtin_amdgcn_raw_buffer_load_b32(rp, vp[t], q * 64, 0);
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = sgpr(min(2 * pr + j, G - 1));
#pragma unroll
            for (int t = 0; t < NT; t++)
                ch.w[t][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, vw[t], g * kTileBytes, kLoadNT);
            if constexpr (!XS) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    ch.x[mt][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, vx[mt], g * kGroup, 0);
                    ch.x[mt][j][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, vx[mt], g * kGroup + 64, 0);
                }
            }
        }
    };

    // unconditional, even for a wave without pairs (the loads then re-read a
    // real tile), so that the waits below are exact
    const int npairs = pw1 - pw0;
    Chunk<MT, NT, XS> ring[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; u++)
        load(ring[u], pw0 + max(min(u, npairs - 1), 0));

    // ---- 3. zero the reduction buffer; with staged rows, wait for them ------
    // Loads retire in order: once no more than the weight prologue is
    // outstanding, this thread's staging copies and scale loads have landed
    // (the count is capped at the counter's 6-bit range, which waits longer).
    constexpr int kPrologue = DEPTH * (3 * NT + (XS ? 0 : 4 * MT));
    for (int i = tid; i < NT * MT * 256; i += kThreads)
        red[i] = 0;
    if constexpr (XS)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kPrologue < 63 ? kPrologue : 63) : "memory");
    lds_barrier();                      // zeroed; staging copies have landed

    // ---- 4. main loop ----------------------------------------------------------
    v4i acc[NT][MT];
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
            acc[t][mt] = v4i{0, 0, 0, 0};

    // staged activations: the B-operand row of token 16 mt + c
    const int8_t *xrow[XS ? MT : 1];
#pragma unroll
    for (int mt = 0; mt < (XS ? MT : 1); mt++)
        xrow[mt] = xlds + (XS ? min(16 * mt + c, mrows - 1) : 0) * xstride + 16 * kb;

    auto compute = [&](const Chunk<MT, NT, XS> &ch, int pr) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int g = 2 * pr + j;
            if (g >= G)          // odd group count: the pair's second half is padding
                break;
            const int gr = g - gbase;
            v4i xf[MT][2];
            if constexpr (XS) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    xf[mt][0] = *reinterpret_cast<const v4i *>(xrow[mt] + gr * kGroup);
                    xf[mt][1] = *reinterpret_cast<const v4i *>(xrow[mt] + gr * kGroup + 64);
                }
            } else if (a.cx) {
#pragma unroll
                for (int mt = 0; mt < MT; mt++)
#pragma unroll
                    for (int h = 0; h < 2; h++)
#pragma unroll
                        for (int d = 0; d < 4; d++)
                            xf[mt][h][d] = __builtin_amdgcn_ds_bpermute(xsrc, ch.x[mt][j][h][d]);
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    xf[mt][0] = ch.x[mt][j][0];
                    xf[mt][1] = ch.x[mt][j][1];
                }
            }
#pragma unroll
            for (int t = 0; t < NT; t++) {
                const uint32_t sc = decode_param((ch.p[t] >> (8 * (g & 3))) & 0xFFu);
                const unsigned short s1 = (unsigned short)(sc & 0xFFFFu);
                const unsigned short c16 = (unsigned short)(sc >> 16);
                const us2 S = {s1, s1};
                const us2 C = {c16, c16};
                v4i f0, f1;
                rebuild_tile(ch.w[t][j], S, C, f0, f1);
#pragma unroll
                for (int mt = 0; mt < MT; mt++) {
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0, xf[mt][0], acc[t][mt], 0, 0, 0);
                    acc[t][mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(f1, xf[mt][1], acc[t][mt], 0, 0, 0);
                }
            }
        }
    };

    // Loads in the steady-state loop are all real; the prologue and the last
    // refill clamp to the wave's last pair (a re-read of data just fetched) so
    // that no load is conditional.
    if (npairs > 0) {
        int pr = pw0;
        for (; pr + 2 * DEPTH <= pw1; pr += DEPTH) {
#pragma unroll
            for (int u = 0; u < DEPTH; u++) {
                compute(ring[u], pr + u);
                load(ring[u], pr + u + DEPTH);
            }
        }
        int rem = pw1 - pr;
        if (rem > DEPTH) {
#pragma unroll
            for (int u = 0; u < DEPTH; u++) {
                compute(ring[u], pr + u);
                load(ring[u], min(pr + u + DEPTH, pw1 - 1));
            }
            pr += DEPTH;
            rem -= DEPTH;
        }
#pragma unroll
        for (int u = 0; u < DEPTH; u++)
            if (u < rem)
                compute(ring[u], pr + u);
    }

    // ---- 5. sum the waves' partials with LDS atomics ---------------------------
#pragma unroll
    for (int t = 0; t < NT; t++)
#pragma unroll
        for (int mt = 0; mt < MT; mt++)
#pragma unroll
            for (int r = 0; r < 4; r++)
                atomicAdd(red + ((t * MT + mt) * 4 + r) * 64 + l, acc[t][mt][r]);
    __syncthreads();

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
    for (int i = wv; i < NT * MT; i += WAVES) {
        const int t = i / MT;
        const int mt = i - t * MT;
        v4i sum;
#pragma unroll
        for (int r = 0; r < 4; r++)
            sum[r] = red[(i * 4 + r) * 64 + l];
        const int64_t m = m0 + 16 * mt + c;
        const int64_t n = (int64_t)(nt0 + t) * kTileN + 4 * kb;
        if (nt0 + t >= ntiles || m >= a.M)
            continue;
        if (a.splitk > 1) {
            // this split's partial: row 16 mt + c, columns 16 t + 4 kb .. + 3
            splitk_store(st, blockIdx.y, 16 * mt + c, 16 * t + 4 * kb, sum);
        } else {
            const float sa = (i == i0) ? sa_e : a.s_a[m];
            const uint2 s0p = (i == i0) ? s0_e : *reinterpret_cast<const uint2 *>(a.s0 + n);
            store_out4(sum, sa, s0p, a.y, a.acc_out, m, n, a.N);
        }
    }
    // ---- 6. split-K: the last workgroup of the tile applies the epilogue -------
    if (a.splitk > 1)
        splitk_finish<kThreads>(st, a.s_a, a.s0, a.y, a.acc_out, a.N, tid);
}

template <int MT, int NT, int WAVES, int DEPTH, bool XS>
hipError_t launch_decode_t(const GemmPlan &p, const DecodeArgs &a, size_t lds, hipStream_t st)
{
    // plans with staged activation rows may use more than the default 64 KB of
    // dynamic LDS: the first such plan raises this kernel's limit on the
    // device to the largest any decode plan may take
    if (lds > 64 * 1024) {
        const hipError_t e = raise_lds_limit(
            reinterpret_cast<const void *>(&gemm_decode_kernel<MT, NT, WAVES, DEPTH, XS>), (int)kDecodeLdsMax);
        if (e != hipSuccess)
            return e;
    }
    dim3 grid((unsigned)p.n_blocks, (unsigned)p.splitk, (unsigned)p.m_blocks);
    hipLaunchKernelGGL((gemm_decode_kernel<MT, NT, WAVES, DEPTH, XS>), grid, dim3(64 * WAVES), lds,
                       st, a);
    return hipGetLastError();
}

}  // namespace

// Instantiated (mt, nt, waves, depth, staged activations) variants.
#define W4A8_DECODE_VARIANTS(X)                                                                   \
    X(1, 1, 4, 2, true) X(1, 1, 4, 4, true) X(1, 2, 4, 2, true) X(1, 2, 4, 4, true)              \
    X(1, 1, 8, 2, true) X(1, 2, 8, 2, true) X(1, 1, 4, 2, false) X(1, 1, 4, 4, false)            \
    X(1, 2, 4, 2, false) X(1, 4, 4, 2, false) X(1, 1, 8, 2, false) X(1, 2, 8, 2, false)          \
    X(2, 1, 4, 2, false) X(2, 2, 4, 2, false) X(2, 4, 4, 2, false) X(2, 1, 8, 2, false)          \
    X(4, 1, 4, 2, false) X(4, 2, 4, 2, false) X(4, 4, 4, 2, false) X(4, 1, 8, 2, false)          \
    X(1, 1, 4, 8, true) X(1, 1, 4, 8, false) X(1, 2, 4, 4, false) X(1, 2, 4, 8, false)           \
    X(1, 4, 4, 4, false) X(2, 2, 4, 4, false) X(2, 4, 4, 4, false) X(4, 4, 4, 4, false)            \
    X(2, 1, 4, 2, true) X(2, 2, 4, 2, true) X(2, 4, 4, 2, true) X(2, 2, 8, 2, true)                \
    X(4, 2, 4, 2, true) X(4, 4, 4, 2, true) X(1, 4, 4, 2, true)

bool decode_variant_exists(int mt, int nt, int waves, int depth, bool xs)
{
#define W4A8_DECODE_HAS(MT_, NT_, WV_, D_, XS_) \
    if (mt == MT_ && nt == NT_ && waves == WV_ && depth == D_ && xs == XS_) return true;
    W4A8_DECODE_VARIANTS(W4A8_DECODE_HAS)
#undef W4A8_DECODE_HAS
    return false;
}

size_t decode_lds_bytes(const GemmPlan &p, int64_t M, int64_t K);

int decode_candidates(int64_t M, int64_t N, int64_t K, GemmPlan *out, int max)
{
    const int64_t ntiles = N / kTileN, G = num_groups(K), P = (G + 1) / 2;
    int n = 0;
    auto add = [&](int mt, int nt, int wv, int dp, bool xs) {
        for (int s : {1, 2, 4, 8}) {
            if (s > P)
                continue;
            GemmPlan p{};
            p.kind = 0;
            p.mt = mt;
            p.nt = nt;
            p.splitk = s;
            p.waves = wv;
            p.depth = dp;
            p.xstage = xs;
            p.m_blocks = (M + 16 * mt - 1) / (16 * mt);
            p.n_blocks = (ntiles + nt - 1) / nt;
            if (s > 1 && p.m_blocks * p.n_blocks > kWsCounters)
                continue;
            const size_t lds = decode_lds_bytes(p, M, K);
            if (lds == 0 || lds > kDecodeLdsMax)
                continue;
            if (n < max)
                out[n] = p;
            n++;
        }
    };
#define W4A8_DECODE_ADD(MT_, NT_, WV_, D_, XS_) add(MT_, NT_, WV_, D_, XS_);
    W4A8_DECODE_VARIANTS(W4A8_DECODE_ADD)
#undef W4A8_DECODE_ADD
    // the N-split kernel: four waves, NTW n-tiles each, activations staged
    for (int mt : {1, 2, 4})
        for (int ntw : {1, 2, 4})
            for (int dp : {2})
                for (int s : {1, 2, 4, 8}) {
                    if (!decode_ns_variant_exists(mt, ntw, dp) || s > P)
                        continue;
                    GemmPlan p{};
                    p.kind = 0;
                    p.mt = mt;
                    p.nt = 4 * ntw;
                    p.splitk = s;
                    p.waves = 4;
                    p.depth = dp;
                    p.xstage = true;
                    p.wave_n = 1;
                    p.m_blocks = (M + 16 * mt - 1) / (16 * mt);
                    p.n_blocks = (ntiles + p.nt - 1) / p.nt;
                    if (s > 1 && p.m_blocks * p.n_blocks > kWsCounters)
                        continue;
                    const size_t lds = decode_ns_lds_bytes(p, K);
                    if (lds == 0 || lds > kDecodeLdsMax)
                        continue;
                    if (n < max)
                        out[n] = p;
                    n++;
                }
    return n;
}

// Dynamic LDS of one decode workgroup (0 if the plan does not fit).
size_t decode_lds_bytes(const GemmPlan &p, int64_t M, int64_t K)
{
    const int64_t G = num_groups(K);
    const int64_t P = (G + 1) / 2;
    int64_t span = 0;
    for (int s = 0; s < p.splitk; s++) {
        const int64_t ps0 = P * s / p.splitk, ps1 = P * (s + 1) / p.splitk;
        span = std::max(span, std::min<int64_t>(2 * (ps1 - ps0), G - 2 * ps0));
    }
    const int64_t rows = std::min<int64_t>(16 * p.mt, M);
    int64_t bytes = (int64_t)p.nt * p.mt * 1024;
    if (p.xstage)
        bytes += (rows * (span * kGroup + 16) + 1023) / 1024 * 1024;
    return (size_t)bytes;
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
    a.ws_part = nullptr;
    a.ws_cnt = nullptr;
    if (p.splitk > 1) {
        a.ws_cnt = reinterpret_cast<uint32_t *>(ws);
        a.ws_part = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(ws) + kWsPartOffset);
    }
    // row-contiguous activation loads pay off from nine tokens on (below,
    // half the lanes of a block repeat the last row); W4A8_DECODE_CX=0|1
    // overrides, for sweeps
    a.cx = M > 8;
    if (const char *env = std::getenv("W4A8_DECODE_CX"))
        a.cx = std::atoi(env) != 0;
    const size_t lds = decode_lds_bytes(p, M, K);
    if (lds == 0 || lds > kDecodeLdsMax)
        return hipErrorInvalidValue;
#define W4A8_DECODE_CASE(MT_, NT_, WV_, D_, XS_)                                           \
    if (p.mt == MT_ && p.nt == NT_ && p.waves == WV_ && p.depth == D_ && p.xstage == XS_) \
        return launch_decode_t<MT_, NT_, WV_, D_, XS_>(p, a, lds, st);
    W4A8_DECODE_VARIANTS(W4A8_DECODE_CASE)
#undef W4A8_DECODE_CASE
    return hipErrorInvalidValue;
}

}  // namespace w4a8
