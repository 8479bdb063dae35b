// Plain 16-byte copy: the achievable-bandwidth ceiling (one HBM read and one
// write per byte) that the row kernels are measured against, and the kernel of
// known traffic that calibrates the HBM byte counters.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// Four independent 16-byte vectors per thread per step, non-temporal loads
// and stores: the fastest plain copy measured on MI355X.
constexpr int kCopyU = 4;

__global__ __launch_bounds__(256) void probe_copy(const u32x4_t *__restrict__ src,
                                                  u32x4_t *__restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * kCopyU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * kCopyU + threadIdx.x; base < n;
         base += stride) {
        u32x4_t q[kCopyU];
#pragma unroll
        for (int u = 0; u < kCopyU; ++u)
            if (base + u * 256 < n)
                q[u] = ld<kStreaming>(src + base + u * 256);
#pragma unroll
        for (int u = 0; u < kCopyU; ++u)
            if (base + u * 256 < n)
                st<kStreaming>(dst + base + u * 256, q[u]);
    }
}

hipError_t probe_copy_run(const void *src, void *dst, size_t bytes, int max_wg,
                          hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(bytes / 16);
    int64_t blocks = (n + 256 * kCopyU - 1) / (256 * kCopyU);
    if (blocks > 65536)
        blocks = 65536;
    if (max_wg > 0 && blocks > max_wg)
        blocks = max_wg;
    if (blocks < 1)
        blocks = 1;
    return launch(probe_copy, dim3(static_cast<unsigned>(blocks)), dim3(256), stream,
                  static_cast<const u32x4_t *>(src), static_cast<u32x4_t *>(dst), n);
}

}  // namespace rk
