// One-time repack of GPTQ INT4 words into the 16-column x 128-row tile layout
// read by the W4A16 kernels. A pure bit permutation: each GPTQ word [j][n]
// (rows 8j..8j+7 of column n) becomes exactly one tile word, with its nibbles
// reordered so that rows (2s, 2s+1) land in nibble slots (s, s+4).
// The Eole recipe "Qwen3.8-27B and native MTP speculative decoding" repacks
// packed weights once during inference setup (section "Pack inference
// projections"); this is that step for the tile layout defined in svq.h.
#include "svq_launch.h"

namespace svq {

// Even source nibbles -> slots 0..3, odd source nibbles -> slots 4..7.
__device__ __forceinline__ uint32_t gptq_to_slot_order(uint32_t v) {
    uint32_t r = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        r |= ((v >> (8 * p)) & 0xFu) << (4 * p);            // nibble 2p   -> slot p
        r |= ((v >> (8 * p + 4)) & 0xFu) << (16 + 4 * p);    // nibble 2p+1 -> slot p+4
    }
    return r;
}

// Thread (row j of the GPTQ array, column n): n is fastest, so reads coalesce.
__global__ __launch_bounds__(256) void q4_repack_kernel(const uint32_t *__restrict__ src,
                                                       uint32_t *__restrict__ dst, int64_t N,
                                                       int64_t K8, int64_t KT) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K8 * N) return;
    const int64_t j = idx / N;         // GPTQ word row: rows 8j..8j+7
    const int64_t n = idx - j * N;
    const int64_t kt = j >> 4;         // 16 word rows per 128-row tile
    const int64_t r = j & 15;          // = 4 * (row group) + word index
    const int64_t nb = n >> 4;
    const int64_t lane = (r >> 2) * 16 + (n & 15);
    const int64_t w = ((nb * KT + kt) * 64 + lane) * 4 + (r & 3);
    dst[w] = gptq_to_slot_order(src[idx]);
}

hipError_t launch_q4_repack(const int32_t *src, int32_t *dst, int64_t N, int64_t K,
                            hipStream_t stream) {
    const int64_t total = (K / 8) * N;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(q4_repack_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                       (const uint32_t *)src, (uint32_t *)dst, N, K / 8, K / 128);
    return hipGetLastError();
}

}  // namespace svq
