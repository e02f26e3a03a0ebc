// kernel_common.h -- device helpers shared by the W4A8 GEMM kernels of
// libw4a8 (private to the library): buffer resources, the packed UINT4 ->
// INT8 rebuild, the group-parameter decode, the fp32 epilogue and the
// split-K / stream-K reduction through the workspace.
#pragma once

#include "w4a8_internal.h"

namespace w4a8 {
namespace dev {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

constexpr int kBufFlags = 0x00020000;   // raw buffer resource, dword 3 (gfx9 family)
constexpr int kLoadNT = 2;              // non-temporal (streaming) load policy
constexpr int kCoherent = 16;           // sc1: loads and stores coherent across the XCDs' L2s

// A raw buffer resource over [p, p + bytes) (clamped to the 31-bit range the
// GEMMs validate); loads past the range return zero.
__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void *p, int64_t bytes)
{
    const int64_t lim = bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)lim, kBufFlags);
}

// The packed rebuild (QServe talk summary, "Efficient INT4 to INT8
// Dequantization": multiply by the scale, then subtract the scaled zero).
// For a dword holding four codes b in [0, 15], one per byte,
// v_pk_mad_u16(x, s1, C) with C = 257 (128 - z s1) mod 2^16 computes in each
// byte b s1 - z s1 + 128, which the protective range keeps in [1, 255], so no
// carry or borrow crosses a byte; xor 0x80808080 then turns each byte into
// the signed INT8 value b s1 - z s1.  Subtracting the zero first would put
// negative values into the packed lanes and borrow across bytes.
__device__ inline uint32_t rebuild4(uint32_t nib, us2 S, us2 C)
{
    us2 v = __builtin_bit_cast(us2, nib);
    v = v * S + C;
    return __builtin_bit_cast(uint32_t, v) ^ 0x80808080u;
}

// Both MFMA fragments of one 16-byte lane load: low nibbles (first 64-k half
// of the group) and high nibbles (second half).
__device__ inline void rebuild_tile(const v4i &w, us2 S, us2 C, v4i &f0, v4i &f1)
{
#pragma unroll
    for (int d = 0; d < 4; d++) {
        const uint32_t x = (uint32_t)w[d];
        f0[d] = (int)rebuild4(x & 0x0F0F0F0Fu, S, C);
        f1[d] = (int)rebuild4((x >> 4) & 0x0F0F0F0Fu, S, C);
    }
}

// A group's parameter byte (s1 - 1) | z << 4 -> s1 in the low half, 257 (128 - z s1)
// in the high half.
__device__ inline uint32_t decode_param(uint32_t p)
{
    const uint32_t s1 = (p & 15u) + 1u;
    const uint32_t c16 = ((128u - (p >> 4) * s1) * 257u) & 0xFFFFu;
    return s1 | (c16 << 16);
}

// Epilogue of four consecutive output channels of one token:
// fp16_rne((float(acc) * s_a) * float(s0)), in that order (no contraction).
__device__ inline uint2 epilogue4(const v4i &sum, float sa, uint2 s0p)
{
    const uint32_t s0w[2] = {s0p.x, s0p.y};
    uint32_t out[2];
#pragma unroll
    for (int r = 0; r < 4; r += 2) {
        const float v0 = ((float)sum[r] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[r / 2] & 0xFFFF));
        const float v1 = ((float)sum[r + 1] * sa) * (float)__builtin_bit_cast(_Float16, (uint16_t)(s0w[r / 2] >> 16));
        out[r / 2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                     ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
    }
    return make_uint2(out[0], out[1]);
}

// y[m, n..n+3] (and acc_out) for one lane's four accumulators.
__device__ inline void store_out4(const v4i &sum, float sa, uint2 s0p, uint16_t *y, int32_t *acc_out, int64_t m,
                                  int64_t n, int64_t N)
{
    *reinterpret_cast<uint2 *>(y + m * N + n) = epilogue4(sum, sa, s0p);
    if (acc_out)
        *reinterpret_cast<v4i *>(acc_out + m * N + n) = sum;
}

// One output tile (rows x cols of the GEMM) split over `splitk` workgroups.
struct SplitTile {
    int32_t *part;       // the tile's slots: splitk x slot_elems INT32, each [rows_max][row_stride]
    uint32_t *cnt;       // the tile's arrival counter (zero between calls)
    int splitk;
    int slot_elems;
    int row_stride;      // INT32 per slot row (the tile's column count)
    int64_t m0, n0;      // first row and column of the tile in the output
    int rows, cols;      // real rows and columns (cols a multiple of 4)
};

// Store this workgroup's partial accumulators (four consecutive columns of
// one row) into its own slot, coherently across XCDs.
__device__ inline void splitk_store(const SplitTile &t, int split, int row, int col, const v4i &sum)
{
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        t.part + (int64_t)split * t.slot_elems, (short)0, t.slot_elems * 4, kBufFlags);
    __builtin_amdgcn_raw_buffer_store_b128(sum, rs, (row * t.row_stride + col) * 4, 0, kCoherent);
}

// After every thread's splitk_store: the last of the tile's workgroups to
// arrive adds the slots in split order (exact INT32, so the bits do not
// depend on the arrival order), applies the epilogue and resets the counter.
// The stores are coherent (sc1) and bypass the XCD's L2, so no cache
// writeback or invalidate is needed: each wave waits until its stores are
// acknowledged before the barrier, the counter increment is issued after the
// barrier, and the last arriver's coherent loads of the other slots are
// issued after it has seen the final count.  Nobody waits on another
// workgroup.  Must be reached by every thread of the workgroup.
template <int THREADS>
__device__ inline void splitk_finish(const SplitTile &t, const float *s_a, const uint16_t *s0, uint16_t *y,
                                     int32_t *acc_out, int64_t N, int tid)
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ uint32_t arrival;
    if (tid == 0)
        arrival = __hip_atomic_fetch_add(t.cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrival != (uint32_t)(t.splitk - 1))
        return;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(t.part, (short)0,
                                                                        t.splitk * t.slot_elems * 4, kBufFlags);
    const int q4 = t.cols / 4;
    for (int i = tid; i < t.rows * q4; i += THREADS) {
        const int r = i / q4;
        const int q = i - r * q4;
        const int64_t m = t.m0 + r;
        const int64_t n = t.n0 + 4 * q;
        v4i sum = {0, 0, 0, 0};
        for (int sp = 0; sp < t.splitk; sp++)
            sum += __builtin_amdgcn_raw_buffer_load_b128(rs, (r * t.row_stride + 4 * q) * 4, sp * (t.slot_elems * 4),
                                                         kCoherent);
        store_out4(sum, s_a[m], *reinterpret_cast<const uint2 *>(s0 + n), y, acc_out, m, n, N);
    }
    if (tid == 0)
        __hip_atomic_store(t.cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A workgroup barrier that waits only for this wave's LDS operations:
// __syncthreads() would also wait for every outstanding global load.  Callers
// first wait (counted vmcnt) for their own direct-to-LDS copies that the
// barrier must publish.
__device__ inline void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct-to-LDS copy of 16 / 4 bytes per lane, buffer form: lane i writes
// dst + i * size; the compiler adds no wait for it before LDS reads, so the
// caller's counted waits decide.
__device__ inline void lds_copy16(const __amdgpu_buffer_rsrc_t &r, void *dst, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, 0, 0, 0);
}

__device__ inline void lds_copy4(const __amdgpu_buffer_rsrc_t &r, void *dst, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 4, voff, 0, 0, 0);
}

}  // namespace dev
}  // namespace w4a8
