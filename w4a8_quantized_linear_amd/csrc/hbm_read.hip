// hbm_read.hip -- the streaming-read ceiling the decode GEMM is measured
// against (measurement aid, not part of the W4A8 computation).
//
// Lecture 15 notes (15.1 and "Numbers worth memorizing"): a decode-size
// linear layer cannot finish faster than its weight bytes take to stream from
// HBM.  The published 8 TB/s is not what one kernel launch reaches on bytes
// of this size: the launch, the first loads' latency and the drain of the last
// ones cost a fixed time per call.  This kernel reads a buffer once, the way
// the GEMM reads its weight stream (16-byte non-temporal buffer loads, 32 KB
// per workgroup of four waves, each wave's eight 1 KB loads in flight at
// once), and does nothing else, so its duration on the same bytes is the
// ceiling a streaming kernel can reach on this chip.
#include <cstdint>

#include "kernel_common.h"
#include "w4a8.h"

namespace w4a8 {
namespace {

using namespace dev;

constexpr int kChunk = 32 * 1024;     // bytes per workgroup
constexpr int kSteps = kChunk / 4 / 1024;   // 1 KB loads per wave

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint8_t *p, uint32_t bytes, uint32_t *sink)
{
    const __amdgpu_buffer_rsrc_t r = rsrc(p, bytes);
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t base = blockIdx.x * (uint32_t)kChunk + wv * (kChunk / 4) + 16 * l;
    v4i v[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; u++)          // past the end the buffer range returns zeros
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, base + u * 1024, 0, kLoadNT);
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < kSteps; u++)
        x ^= (uint32_t)(v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3]);
    // consume the data without writing: a store only for one fixed value
    if (x == 0x9E3779B9u)
        sink[0] = x;
}

}  // namespace
}  // namespace w4a8

extern "C" w4a8_status w4a8_hbm_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t stream)
{
    if (bytes == 0)
        return W4A8_OK;
    if (bytes % 16 != 0 || bytes > 0x7FFFFFFFu)
        return W4A8_E_SHAPE;
    if (!buf || !sink)
        return W4A8_E_NULL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
        return W4A8_E_ALIGN;
    const unsigned grid = (unsigned)((bytes + w4a8::kChunk - 1) / w4a8::kChunk);
    hipLaunchKernelGGL(w4a8::hbm_read_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(buf), (uint32_t)bytes, sink);
    return hipGetLastError() == hipSuccess ? W4A8_OK : W4A8_E_HIP;
}
