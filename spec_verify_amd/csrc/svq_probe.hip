// Streaming probe: a read-only kernel that moves a buffer's bytes from HBM to
// the compute units and does nothing else. It measures the bandwidth a plain
// read of a given number of bytes reaches on this chip in a given launch shape,
// the ceiling against which the GEMM kernels' weight streams are judged (the
// AWQ card "Qwen3.8-27B-AWQ-INT4-MTP-LowLatency" ties decode latency to the
// bytes each token reads, in its head-precision section).
//
// Workgroup b of the grid reads the b-th of `grid` equal contiguous shares of
// the 16-byte units; each lane keeps eight 16-byte loads in flight, and the
// XOR of everything read decides a store to sink[b] that never happens for
// ordinary data but keeps every load live.
#include "svq_launch.h"

namespace svq {

__global__ __launch_bounds__(1024) void stream_probe_kernel(const uint4 *__restrict__ src, uint64_t n16,
                                                            uint32_t *__restrict__ sink) {
    constexpr int U = 8;
    const uint64_t b = blockIdx.x, g = gridDim.x, nt = blockDim.x;
    const uint64_t beg = b * n16 / g, end = (b + 1) * n16 / g;
    uint32_t acc = 0;
    for (uint64_t i = beg + threadIdx.x; i < end; i += U * nt) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + u * nt;
            v[u] = j < end ? src[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x5EED5EEDu) sink[b] = acc;
}

hipError_t launch_stream_probe(const void *src, size_t bytes, uint32_t grid, uint32_t threads, uint32_t *sink,
                               hipStream_t stream) {
    hipLaunchKernelGGL(stream_probe_kernel, dim3(grid), dim3(threads), 0, stream, (const uint4 *)src,
                       (uint64_t)(bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace svq
