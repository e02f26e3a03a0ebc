// dispatch.hip -- shape-keyed choice of GEMM kernel, tile and split-K.
//
// The QFactory reading notes (6.1-6.2) make tile shapes compile-time template
// parameters and pick an instantiation per shape; here the pick is a small
// deterministic rule of (M, N, K), so the workspace size a caller queries and
// the plan gemm_w4a8 launches always agree.  W4A8_DECODE_PLAN=
// "mt,nt,splitk[,waves[,depth[,xstage[,wave_n]]]]" overrides the decode
// choice and sends every M <= 1024 to the decode kernels (for tuning sweeps);
// a plan that names no instantiated variant is replaced by the decode
// kernels' own plan for the shape.
#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <set>
#include <unordered_map>
#include <utility>

#include "w4a8_internal.h"

namespace w4a8 {

bool decode_variant_exists(int mt, int nt, int waves, int depth, bool xs);
size_t decode_lds_bytes(const GemmPlan &p, int64_t M, int64_t K);
bool prefill_tm_supported(int tm);
size_t prefill_ws_bytes(int tm, int P, int64_t M, int64_t N, int64_t K);
size_t prefill_lds_bytes(int tm);
GemmPlan launchable_fallback(int64_t M, int64_t N, int64_t K, bool split);
hipError_t launch_gemm_prefill(const GemmPlan &p, const int8_t *qx, const float *s_a,
                               const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                               int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *ws,
                               hipStream_t st);
hipError_t launch_gemm_decode(const GemmPlan &p, const int8_t *qx, const float *s_a,
                              const uint8_t *stream_bytes, const uint16_t *s0, int64_t M,
                              int64_t N, int64_t K, uint16_t *y, int32_t *acc_out, void *ws,
                              hipStream_t st);

// compute units of the current device (cached per device; several host
// threads may race to fill an entry, all with the same value)
int64_t num_cus()
{
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The dynamic-LDS limit of a kernel is a per-device function attribute.  It
// is raised once per (kernel, device) to the kernel's own maximum and never
// lowered, so no launch can run under a smaller limit that another host
// thread set between its check and its launch.  The mutex orders the first
// calls; later calls find the pair in the set.
hipError_t raise_lds_limit(const void *kernel, int bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(kernel, dev);
    if (done.count(key))
        return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess)
        done.insert(key);
    return e;
}

namespace {

// decode split-K: the counters, then one 16 mt x 16 nt INT32 slot per (tile, split)
size_t ws_size(const GemmPlan &p)
{
    const int64_t tiles = p.m_blocks * p.n_blocks;
    if (p.splitk <= 1 || tiles > kWsCounters)
        return 0;
    return (size_t)kWsPartOffset + (size_t)tiles * p.splitk * 256 * p.mt * p.nt * 4;
}

bool launchable(const GemmPlan &p, int64_t M, int64_t N, int64_t K)
{
    if (p.wave_n == 1) {
        const size_t lds = decode_ns_lds_bytes(p, K);
        return p.waves == 4 && p.nt % 4 == 0 && decode_ns_variant_exists(p.mt, p.nt / 4, p.depth) && lds > 0 &&
               lds <= kDecodeLdsMax;
    }
    const size_t lds = decode_lds_bytes(p, M, K);
    return decode_variant_exists(p.mt, p.nt, p.waves, p.depth, p.xstage) && lds > 0 &&
           lds <= kDecodeLdsMax;
}

// The selector's choice for (M, N, K) on a device with `cus` compute units:
// the candidate with the highest predicted utilization when that prediction
// beats the fixed rule's plan by more than kSelMargin, else the rule's plan.
// The margin is chosen on held-out measurements (random shapes and the 7B /
// 70B decode shapes); for the current model no margin does best.
// Ranking all candidates costs tens of microseconds of host time, so the
// choice is kept per shape (at most 4096 shapes; the table restarts when
// full).  Guarded by a mutex: calls may come from several host threads.
GemmPlan selected_plan(int64_t M, int64_t N, int64_t K, const GemmPlan &fallback)
{
    struct Key {
        int64_t M, N, K, cus;
        bool operator==(const Key &o) const { return M == o.M && N == o.N && K == o.K && cus == o.cus; }
    };
    struct Hash {
        size_t operator()(const Key &k) const
        {
            uint64_t h = 1469598103934665603ull;
            for (int64_t v : {k.M, k.N, k.K, k.cus})
                h = (h ^ (uint64_t)v) * 1099511628211ull;
            return (size_t)h;
        }
    };
    static std::mutex mu;
    static std::unordered_map<Key, GemmPlan, Hash> table;
    const int64_t cus = num_cus();
    const Key key{M, N, K, cus};
    {
        std::lock_guard<std::mutex> lock(mu);
        const auto it = table.find(key);
        if (it != table.end())
            return it->second;
    }
    GemmPlan cand[256];
    const int nc = std::min(decode_candidates(M, N, K, cand, 256), 256);
    GemmPlan top = fallback;
    float best = -1.0f;
    for (int i = 0; i < nc; i++) {
        if (!selector_knows_wave_n(cand[i].wave_n))
            continue;
        float x[kSelFeatures];
        selector_features(cand[i], M, N, K, cus, x);
        const float u = selector_predict(x);
        if (u > best) {
            best = u;
            top = cand[i];
        }
    }
    // the rule's plan stays unless the model expects more than kSelMargin
    // better utilization from its top candidate
    float xf[kSelFeatures];
    selector_features(fallback, M, N, K, cus, xf);
    const GemmPlan p = best > selector_predict(xf) * (1.0f + kSelMargin) ? top : fallback;
    std::lock_guard<std::mutex> lock(mu);
    if (table.size() >= 4096)
        table.clear();
    table[key] = p;
    return p;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K)
{
    GemmPlan p{};
    p.kind = 0;
    const int64_t ntiles = N / kTileN;
    const int64_t G = num_groups(K);
    const int64_t P = (G + 1) / 2;
    // Rules fitted to rocprofv3 sweeps of the decode plans over the 7B and 70B
    // shapes (M = 1..64) on MI355X.  Few tokens: one n-tile per workgroup,
    // the activation rows staged in LDS when they fit.  Large weight streams
    // (>= 512 n-tiles, or >= 100 MB at 2..8 tokens): two n-tiles per workgroup
    // and a 2-way K split, which doubles the weight bytes in flight per CU.
    // 17..32 tokens: two m-tiles, wide n-blocks (each activation operand
    // feeds more weight tiles) and a 4-way K split for long K.  33..64
    // tokens: four m-tiles and four n-tiles for long K and wide N, else two
    // m-blocks of two m-tiles; the widest N goes to the matrix-core kernel.
    const double wbytes = (double)N * K / 2;
    p.splitk = 1;
    p.waves = 4;
    p.depth = 2;
    p.xstage = false;
    if (M <= 16) {
        p.mt = 1;
        p.nt = 1;
        if (M > 1 && ((M > 8 && ntiles >= 512) || (M <= 8 && wbytes >= 100e6))) {
            p.nt = 2;
            p.splitk = 2;
        }
    } else if (M <= 32) {
        p.mt = 2;
        p.nt = ntiles >= 512 ? 4 : (ntiles >= 384 ? 2 : 1);
        if (G >= 86) {
            p.nt = 4;
            p.splitk = 4;
        }
    } else if (M > 128) {
        // 129..1024 tokens (layers with at most 2^20 outputs, below): a small
        // decision tree over the weight size, N, K and the workgroup counts
        // of the plan families, fitted (least total log-time over the best
        // plan) to graph-timed sweeps of every decode plan on MI355X at
        // 129..256 tokens: 150 random shapes (N = 512..7296, K = 2048..28672),
        // 60 more and 15 layers of the 7B / 70B family.  Re-timed live, its
        // plan runs at 1.04-1.07x the best plan's time on average over each
        // set (at most 1.3x); at 257..1024 tokens on narrow layers, 1.1x.
        const int64_t cus = num_cus();
        const int64_t nk_cap = M <= 256 ? INT64_MAX : (M <= 512 ? int64_t{1} << 25 : int64_t{1} << 23);
        auto wg = [&](int mt, int nt) { return (M + 16 * mt - 1) / (16 * mt) * ((ntiles + nt - 1) / nt); };
        auto use = [&](int mt, int nt, int s, int waves, bool xstage, int wave_n) {
            p.mt = mt;
            p.nt = nt;
            p.splitk = s;
            p.waves = waves;
            p.xstage = xstage;
            p.wave_n = wave_n;
        };
        if (N * K > nk_cap) {
            // past 256 tokens, weights above the tree's range (taken only
            // when these workgroups fit one round): four m-tiles, unsplit.
            // Against the matrix-core kernel's best run on 41 such shapes
            // with 257..1024 tokens: 0.99-1.58x its speed
            use(4, 4, 1, 4, false, 0);
        } else if (N * K <= (int64_t{1} << 25)) {
            if (wg(1, 2) <= cus)
                use(1, 2, 1, 8, K <= 8192, 0);             // one m-tile, the token rows staged when short
            else if (wg(2, 4) <= cus + cus / 2 && K >= 12288)
                use(2, 4, 4, 4, true, 1);                  // few workgroups, long K: split K four ways
            else if (wg(2, 4) <= cus + cus / 2)
                use(2, 2, 1, 4, false, 0);
            else
                use(2, 4, 1, 4, true, 1);                  // waves splitting N
        } else if (N <= 2560) {
            if (wg(2, 4) <= cus * 3 / 4)
                use(2, 4, 4, 4, true, 1);
            else
                use(4, 4, 2, 4, false, 0);
        } else if (wg(4, 4) <= cus) {
            use(4, 4, 1, 4, false, 0);
        } else {
            use(2, 4, 1, 4, false, 0);
        }
        if (!launchable(p, M, N, K)) {   // staged and N-split forms need LDS that grows with K
            p.xstage = false;
            p.wave_n = 0;
        }
    } else if (M > 64) {
        // 65..128 tokens (where the decode kernels take them, below): a
        // decision tree over the workgroup counts of the (1, 2), (2, 4) and
        // (4, 4) tilings, N x K and K, fitted like the one above to
        // graph-timed sweeps of every decode plan: 210 random shapes
        // (M = 65..128, N = 512..16384, K = 2048..28672) and 26 7B / 70B and
        // narrow layers at 72..128 tokens.  Re-timed live, its plan runs at
        // 1.06x the best plan's time on average over each set (at most
        // 1.3x); the selector's picks ran at 1.12x (at most 1.7x).
        const int64_t cus = num_cus();
        auto wg = [&](int mt, int nt) { return (M + 16 * mt - 1) / (16 * mt) * ((ntiles + nt - 1) / nt); };
        p.splitk = 1;
        if (wg(1, 2) <= 2 * cus) {
            p.mt = wg(1, 2) <= cus ? 1 : 2;
            p.nt = wg(1, 2) <= cus / 2 ? 1 : 2;
            p.waves = wg(1, 2) <= cus / 2 || (p.mt == 2 && N * K < (int64_t{1} << 23)) ? 8 : 4;
            p.xstage = p.mt == 2 && N * K < (int64_t{1} << 23);
        } else if (wg(2, 4) <= 2 * cus) {
            p.mt = wg(2, 4) <= cus || wg(4, 4) > cus ? 2 : 4;   // four m-tiles only in one round
            p.nt = 4;
        } else {
            p.mt = 4;
            p.nt = K <= 10240 ? 4 : 8;
            p.splitk = K <= 10240 ? 1 : 2;
            p.xstage = true;
            p.wave_n = 1;   // waves splitting N
        }
        if (!launchable(p, M, N, K)) {
            p.xstage = false;
            p.wave_n = 0;
        }
    } else if (K >= 8192 && N >= 8192) {
        p.mt = 4;
        p.nt = 4;
        p.splitk = K >= 16384 ? 2 : 1;
    } else {
        p.mt = 2;
        p.nt = 4;
        p.splitk = ntiles <= 256 ? 2 : 1;
    }
    p.splitk = (int)std::min<int64_t>(p.splitk, P);
    p.m_blocks = (M + 16 * p.mt - 1) / (16 * p.mt);
    p.n_blocks = (ntiles + p.nt - 1) / p.nt;
    if (M <= 64 && p.mt == 1 && p.splitk == 1) {
        GemmPlan q = p;
        q.xstage = true;
        if (launchable(q, M, N, K) && decode_lds_bytes(q, M, K) <= 64 * 1024)
            p = q;
    }
    // 65..128 tokens stay on the decode kernels while the matrix-core
    // kernel's smallest tiles (64 tokens x 256 channels) would leave more than
    // half of the CUs idle, unless the weights are very large (N x K above
    // 3 x 2^25, about 10^8) and four-m-tile workgroups would take two rounds.
    // Measured on MI355X (graph-timed) against the matrix-core kernel's best
    // TM and K split, M = 96: K = 4096, N = 11008: 19.0 against 25.1 us;
    // K = 11008, N = 4096: 18.2 against 34.3; K = 12288, N = 1536: 13.0
    // against 35.2.  At N = 22016 (172 tiles) the matrix-core kernel stays
    // ahead (27.1 against 28.1), and on the excluded large weights it ran up
    // to 1.35x faster (K = 19584, N = 8448, M = 122; K = 12544, N = 9344,
    // M = 111: 1.22x), while below the bound the decode plans stayed within
    // 6% or ahead (K = 8192, N = 10240, M = 72: 1.24x ahead)
    const int64_t cus = num_cus();
    const int64_t nblk = (ntiles * kTileN + 255) / 256;
    auto tiles_of = [&](int t) { return (M + 16 * t - 1) / (16 * t) * nblk; };
    // 129..1024 tokens stay on the decode kernels on layers with at most 2^20
    // outputs (M x N), unless the weights are large (N x K above 2^26) and
    // four-m-tile workgroups would not fit one round on the CUs.  Graph-timed
    // on MI355X against the matrix-core kernel's best TM and K split on the
    // 277 shapes of the plan rule above: on the 274 it sends to the decode
    // kernels their rule plan ran 0.90-4.5x the speed of the best matrix-core
    // run (K = 11008, N = 4096, M = 136: 25.7 against 34.9 us; K = 13824,
    // N = 5120, M = 160: 30.3 against 40.4); on the three it excludes, 0.64-
    // 0.89x (K = 16512, N = 5760, M = 165: 71.1 against 45.3).  Up to 2^21
    // outputs the decode kernels keep small weights (N x K <= 2^25): on 33 such
    // random shapes their plan ran 0.96-1.45x the speed of the best
    // matrix-core run (K = 2944, N = 5120, M = 254: 1.45x); past 2^25 the
    // matrix-core kernel was mostly ahead.  Wider layers stay on the
    // matrix-core kernel (K = 28672, N = 8192, M = 160: 79.5 against 88.7 for
    // the best decode plan).  Past 256 tokens only small weights (N x K <=
    // 2^25) stay: on 100 random shapes with 257..512 tokens and the 7B / 70B
    // layers at 320..512, those ran 0.91-3.4x the speed of the best
    // matrix-core run (geomean 1.5-1.8x; K = 4096, N = 1024, M = 512: 9.8
    // against 22.5 us).  Past 512 tokens the tree's plans hold to
    // N x K <= 2^23 (K = 4096, N = 1024, M = 1024: 15.3 against 24.0 us).
    // Past those caps the tree's long-K plans lost up to 1.25x, so there the
    // decode kernels run four m-tiles unsplit, and only where those
    // workgroups fit one round (at 294 workgroups that plan lost 1.6x)
    const int64_t wg44 = (M + 63) / 64 * ((ntiles + 3) / 4);
    const int64_t nk_cap = M <= 256 ? INT64_MAX : (M <= 512 ? int64_t{1} << 25 : int64_t{1} << 23);
    const bool decode_m = M <= 64 ||
                          (M <= 128 && tiles_of(4) * 2 < cus &&
                           (N * K <= (int64_t{3} << 25) || wg44 <= cus)) ||
                          (M <= kDecodeMaxM && M * N <= (int64_t{1} << 20) && tiles_of(4) * 2 < cus &&
                           (N * K <= (int64_t{1} << 26) || wg44 <= cus) && (N * K <= nk_cap || wg44 <= cus)) ||
                          (M <= kDecodeMaxM && M * N <= (int64_t{1} << 21) &&
                           N * K <= std::min<int64_t>(int64_t{1} << 25, nk_cap));

    // the learned selector, when a model is compiled in: the candidate with
    // the highest predicted bandwidth utilization (remembered per shape);
    // its model was trained on 1..64 tokens, and past 64 its picks ran
    // 1.1x the best plan's time on average (up to 1.7x), so the trees above
    // keep those
    if (decode_m && M <= 64 && selector_enabled())
        p = selected_plan(M, N, K, p);

    // many tokens: the matrix-core kernel with (16 TM) x 256 workgroup tiles.
    // Rules fitted to graph-timed sweeps on MI355X (TM x splits per tile,
    // M = 96..768, K = 4096..28672, the 7B and 70B layers):
    //  * when TM 4 tiles fit one round (at most one per CU): split every tile
    //    into s equal K ranges, s = CUs / tiles (at most 4, and at least 16
    //    groups per range), so that P = tiles x s workgroups still fit one
    //    round and no range straddles two tiles.  Where TM 4 allows no split
    //    (s = 1) but TM 8 tiles split in two still fit one round and K has
    //    at least 80 groups, TM 8 with two ranges per tile (at 64 groups TM 4
    //    unsplit stayed 8-10% ahead).  Measured against
    //    P = CUs ranges (which straddle tiles): K = 11008, N = 4096, M = 160
    //    36.2 against 50.7 us, M = 384 39.8 against 53.7; K = 8192, N = 10240,
    //    M = 160 34.6 against 48.2; K = 28672, N = 8192, M = 384 112.6 against
    //    145.4 (TM 8, two ranges); with whole tiles past one round,
    //    splitting lost everywhere;
    //  * otherwise one workgroup per tile, TM minimising workgroup rounds x
    //    TM x the relative time per MFMA at that TM (1.0, 1.23, 1.75 for
    //    TM 16, 8, 4: smaller tiles rebuild each weight for fewer tokens).
    // W4A8_PREFILL_TM=4|8|16 forces this kernel and its TM (at any M);
    // W4A8_PREFILL_P=n forces n stream-K ranges (0: one workgroup per tile).
    int tm = 0;
    int64_t ranges = 0;
    if (const char *env = std::getenv("W4A8_PREFILL_TM"))
        tm = std::atoi(env);
    const bool force_decode = M <= kDecodeMaxM && std::getenv("W4A8_DECODE_PLAN") != nullptr;
    if (!prefill_tm_supported(tm) && !force_decode) {
        tm = 0;
        if (M > 32 && M <= 64 && N >= 32768)
            tm = 4;   // 33..64 tokens on the widest N: activations shared through LDS
        else if (!decode_m) {
            const int64_t t4 = tiles_of(4), t8 = tiles_of(8);
            if (t4 <= cus) {
                const int64_t s4 = std::max<int64_t>(1, std::min<int64_t>({cus / t4, G / 16, 4}));
                if (s4 == 1 && G >= 80 && t8 * 2 <= cus) {
                    tm = 8;
                    ranges = t8 * 2;
                } else {
                    tm = 4;
                    ranges = s4 > 1 ? t4 * s4 : 0;
                }
            } else {
                const struct { int tm; double rel; } cand[] = {{16, 1.0}, {8, 1.23}, {4, 1.75}};
                double best = 0;
                for (const auto &c : cand) {
                    const double cost = (double)((tiles_of(c.tm) + cus - 1) / cus) * c.tm * c.rel;
                    if (tm == 0 || cost < best) {
                        tm = c.tm;
                        best = cost;
                    }
                }
            }
        }
    }
    if (prefill_tm_supported(tm)) {
        GemmPlan q{};
        q.kind = 1;
        q.mt = tm;
        q.nt = 16;
        q.m_blocks = (M + 16 * tm - 1) / (16 * tm);
        q.n_blocks = nblk;
        if (const char *env = std::getenv("W4A8_PREFILL_P"))
            ranges = std::max<int64_t>(0, std::min<int64_t>(std::atoll(env), tiles_of(tm) * G));
        q.ws_bytes = prefill_ws_bytes(tm, (int)ranges, M, N, K);
        q.splitk = q.ws_bytes > 0 ? (int)ranges : 0;
        return q;
    }

    if (const char *env = std::getenv("W4A8_DECODE_PLAN")) {
        int mt = 0, nt = 0, s = 0, wv = 4, dp = 2, xs = 0, wn = 0;
        int got = std::sscanf(env, "%d,%d,%d,%d,%d,%d,%d", &mt, &nt, &s, &wv, &dp, &xs, &wn);
        GemmPlan q = p;
        q.mt = mt;
        q.nt = nt;
        q.splitk = s;
        q.waves = wv;
        q.depth = dp;
        q.xstage = xs != 0 || wn != 0;
        q.wave_n = wn != 0 ? 1 : 0;
        if (got >= 3 && nt > 0 && s >= 1 && s <= P && (mt == 1 || mt == 2 || mt == 4)) {
            q.m_blocks = (M + 16 * mt - 1) / (16 * mt);
            q.n_blocks = (ntiles + nt - 1) / nt;
            if (launchable(q, M, N, K))
                p = q;
        }
    }
    if (p.splitk > 1 && p.m_blocks * p.n_blocks > kWsCounters)
        return plan_without_workspace(p, M, N, K);   // more tiles than counters: run unsplit
    if (!launchable(p, M, N, K))
        return launchable_fallback(M, N, K, true);   // very long K: the plan's LDS does not fit
    p.ws_bytes = ws_size(p);
    return p;
}

namespace {

// The many-token kernel with the smallest tile, one workgroup per tile: its
// LDS does not depend on K, so it runs every shape the C ABI accepts.
GemmPlan prefill_unsplit(int64_t M, int64_t N)
{
    GemmPlan q{};
    q.kind = 1;
    q.mt = 4;
    q.nt = 16;
    q.m_blocks = (M + 63) / 64;
    q.n_blocks = (N + 255) / 256;
    return q;
}

}  // namespace

// The best-scored decode candidate that can launch (unsplit ones only unless
// `split` is set), or the many-token kernel when no decode plan fits.
GemmPlan launchable_fallback(int64_t M, int64_t N, int64_t K, bool split)
{
    GemmPlan cand[256];
    const int nc = std::min(decode_candidates(M, N, K, cand, 256), 256);
    const int64_t cus = num_cus();
    const bool rank = selector_enabled();
    int pick = -1;
    float best = -2.0f;
    for (int i = 0; i < nc; i++) {
        if ((!split && cand[i].splitk != 1) || (rank && !selector_knows_wave_n(cand[i].wave_n)))
            continue;
        float u = 0.0f;
        if (rank) {
            float x[kSelFeatures];
            selector_features(cand[i], M, N, K, cus, x);
            u = selector_predict(x);
        }
        if (pick < 0 || u > best) {
            pick = i;
            best = u;
        }
    }
    if (pick < 0)
        return prefill_unsplit(M, N);
    GemmPlan p = cand[pick];
    p.ws_bytes = ws_size(p);
    return p;
}

GemmPlan plan_without_workspace(GemmPlan p, int64_t M, int64_t N, int64_t K)
{
    p.ws_bytes = 0;
    if (p.kind == 1) {
        p.splitk = 0;
        return p;
    }
    p.splitk = 1;
    // an N-split or staged plan keeps the whole K slice's parameters (and
    // activation rows) in LDS, which an unsplit long K may not fit
    if (launchable(p, M, N, K))
        return p;
    return launchable_fallback(M, N, K, false);
}

size_t plan_lds_bytes(const GemmPlan &p, int64_t M, int64_t N, int64_t K)
{
    if (p.kind == 1)
        return prefill_lds_bytes(p.mt);
    return p.wave_n == 1 ? decode_ns_lds_bytes(p, K) : decode_lds_bytes(p, M, K);
}

hipError_t launch_gemm(const GemmPlan &p, const int8_t *qx, const float *s_a,
                       const uint8_t *stream_bytes, const uint16_t *s0, int64_t M, int64_t N,
                       int64_t K, uint16_t *y, int32_t *acc_out, void *ws, hipStream_t st)
{
    if (std::getenv("W4A8_LOG"))
        std::fprintf(stderr,
                     "w4a8: gemm M=%lld N=%lld K=%lld kind=%d mt=%d nt=%d splitk=%d waves=%d "
                     "depth=%d xstage=%d wave_n=%d grid=%lldx%dx%lld\n",
                     (long long)M, (long long)N, (long long)K, p.kind, p.mt, p.nt, p.splitk,
                     p.waves, p.depth, (int)p.xstage, (int)p.wave_n, (long long)p.n_blocks, p.splitk,
                     (long long)p.m_blocks);
    if (p.kind == 1)
        return launch_gemm_prefill(p, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
    if (p.wave_n == 1)
        return launch_gemm_decode_ns(p, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
    return launch_gemm_decode(p, qx, s_a, stream_bytes, s0, M, N, K, y, acc_out, ws, st);
}

}  // namespace w4a8
