// Probes: ceilings for the GEMM kernels, measured on this chip.
//
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

// Matrix-core probe: every wave of `grid` workgroups of `threads` threads runs
// `per_wave` v_mfma_f32_16x16x32_bf16 (a multiple of 8) as eight independent
// accumulator chains on register operands, with no memory traffic. Its time is
// the floor that MFMA issue alone sets for a kernel doing the same number of
// MFMAs per wave in the same launch shape (batched verify: "FP8 decode is the
// more compute-bound path", autobench "Qwen3.8-27B · vLLM · FP8 + MTP").
//
// Two operand sets. Constant: every A and B register holds one small value, so
// the multipliers' inputs never change. Random: each chain has its own
// operands, A random bf16 values (random sign and mantissa, magnitude in
// [2^-2, 2^2)) like activations, B the bf16 of 128 + q for random nibbles q,
// the W4A16 kernels' weight operand; consecutive MFMAs then switch every input
// bit the data switches. The matrix cores' power draw depends on that
// switching, and the chip lowers its shader clock under it, so the random set
// gives the floor for real data. Either way the accumulator totals decide a
// store to sink[b] that never happens but keeps every MFMA live.
__device__ __forceinline__ uint32_t probe_mix(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(1024) void mfma_probe_kernel(uint32_t per_wave, int random, float *__restrict__ sink) {
    const uint32_t lane = threadIdx.x & 63;
    uint4 a[8], b[8];
    if (!random) {
        // bf16 pairs of 2^-4 * (1 + lane/128) and 2^-4: exact, small
        const uint32_t ha = 0x3D80u + (lane & 15u), hb = 0x3D80u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            a[j] = make_uint4(ha | (ha << 16), ha | (ha << 16), ha | (ha << 16), ha | (ha << 16));
            b[j] = make_uint4(hb | (hb << 16), hb | (hb << 16), hb | (hb << 16), hb | (hb << 16));
        }
    } else {
        const uint32_t seed = (blockIdx.x * 1024u + threadIdx.x) * 64u;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t wa[4], wb[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t h = probe_mix(seed + (uint32_t)(8 * j + 2 * e));
                const uint32_t k = probe_mix(seed + (uint32_t)(8 * j + 2 * e + 1));
                // sign and 7 mantissa bits from the hash, exponent 125..128
                const uint32_t lo = (h & 0x807Fu) | ((0x7Du + ((h >> 8) & 3u)) << 7);
                const uint32_t hi = ((h >> 16) & 0x807Fu) | ((0x7Du + ((h >> 24) & 3u)) << 7);
                wa[e] = lo | (hi << 16);
                wb[e] = (0x4300u | (k & 15u)) | ((0x4300u | ((k >> 16) & 15u)) << 16);
            }
            a[j] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
            b[j] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        asm volatile("" : "+v"(a[j].x), "+v"(a[j].y), "+v"(a[j].z), "+v"(a[j].w));
        asm volatile("" : "+v"(b[j].x), "+v"(b[j].y), "+v"(b[j].z), "+v"(b[j].w));
    }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (uint32_t i = 0; i < per_wave; i += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma16x16x32(a[j], b[j], acc[j]);
    }
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (t == -1.0f) sink[blockIdx.x] = t;
}

hipError_t launch_mfma_probe(uint32_t grid, uint32_t threads, uint32_t per_wave, int random, float *sink,
                             hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(grid), dim3(threads), 0, stream, per_wave, random, sink);
    return hipGetLastError();
}

hipError_t launch_stream_probe(const void *src, size_t bytes, uint32_t grid, uint32_t threads, uint32_t *sink,
                               hipStream_t stream) {
    hipLaunchKernelGGL(stream_probe_kernel, dim3(grid), dim3(threads), 0, stream, (const uint4 *)src,
                       (uint64_t)(bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace svq
