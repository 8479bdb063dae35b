// Plain 16-byte copy: the achievable-bandwidth ceiling (one HBM read and one
// write per byte) that the row kernels are measured against, and the kernel of
// known traffic that calibrates the HBM byte counters.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

__global__ __launch_bounds__(256) void probe_copy(const uint4 *__restrict__ src,
                                                  uint4 *__restrict__ dst, int64_t n)
{
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

hipError_t probe_copy_run(const void *src, void *dst, size_t bytes, int max_wg,
                          hipStream_t stream)
{
    const int64_t n = static_cast<int64_t>(bytes / 16);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    if (max_wg > 0 && blocks > max_wg)
        blocks = max_wg;
    if (blocks < 1)
        blocks = 1;
    return launch(probe_copy, dim3(static_cast<unsigned>(blocks)), dim3(256), stream,
                  static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
}

}  // namespace rk
