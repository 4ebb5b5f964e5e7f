// Setup-time layout kernels. One-time repack of GPTQ INT4 words into the
// 16-column x 128-row tile layout read by the W4A16 kernels. A pure bit permutation: each GPTQ word [j][n]
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

// The 16 bytes lane l of tile (nb, kt) owns: the words of GPTQ rows
// 4q .. 4q+3 of column n, q = 4*kt + l/16, n = 16*nb + l%16, word i in slot i.
__device__ __forceinline__ uint4 repack_quad(const uint32_t *__restrict__ src, int64_t q, int64_t n,
                                             int64_t ld) {
    const uint32_t *p = src + 4 * q * ld + n;
    return make_uint4(gptq_to_slot_order(p[0]), gptq_to_slot_order(p[ld]),
                      gptq_to_slot_order(p[2 * ld]), gptq_to_slot_order(p[3 * ld]));
}

// Thread (quad q of GPTQ word rows, column n), n fastest: the four word reads
// coalesce across the wave, and the wave writes 256-byte runs of whole lane
// slots (four 4-byte stores per slot, each from another workgroup, doubled the
// written bytes: 89 MB for 44.6 MB at K = 5120, N = 17408).
__global__ __launch_bounds__(256) void q4_repack_kernel(const uint32_t *__restrict__ src,
                                                       uint4 *__restrict__ dst, int64_t N,
                                                       int64_t K32, int64_t KT) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= K32 * N) return;
    const int64_t q = idx / N;         // GPTQ word rows 4q..4q+3 = K rows 32q..32q+31
    const int64_t n = idx - q * N;
    const int64_t lane = (q & 3) * 16 + (n & 15);
    dst[((n >> 4) * KT + (q >> 2)) * 64 + lane] = repack_quad(src, q, n, N);
}

hipError_t launch_q4_repack(const int32_t *src, int32_t *dst, int64_t N, int64_t K,
                            hipStream_t stream) {
    const int64_t total = (K / 32) * N;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(q4_repack_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream,
                       (const uint32_t *)src, (uint4 *)dst, N, K / 32, K / 128);
    return hipGetLastError();
}

// ---- projection fusion at setup ----------------------------------------------
// Projections that read the same x are concatenated along N before the repack
// (Eole recipe, section "Pack inference projections"; no requantization). Part p
// covers fused columns [col_off[p], col_off[p+1]). Because the tile layout is
// column-block-major and every width is a multiple of 16, part p's tiles are
// its own repack placed at word col_off[p]*K/8; its scales are columns
// col_off[p].. of the fused [K/G][N] array. One launch covers all parts: part p
// owns workgroups [blk_off[p], blk_off[p+1]), one thread per 16-byte lane slot
// (four GPTQ words, int4) or per 16 bytes of int8 codes, the threads below
// (K/G)*N_p also moving one scale each (K/G <= K/32 slots per column).
struct FuseTable {
    const void *w[kMaxFuseParts];
    const uint16_t *s[kMaxFuseParts];
    int64_t col_off[kMaxFuseParts + 1];
    int64_t blk_off[kMaxFuseParts + 1];
    int parts;
};

template <int BITS>
__global__ __launch_bounds__(256) void fuse_pack_kernel(FuseTable t, void *__restrict__ dst_w,
                                                        uint16_t *__restrict__ dst_s, int64_t K,
                                                        int G) {
    const int64_t b = blockIdx.x;
    int p = 0;
    while (p + 1 < t.parts && b >= t.blk_off[p + 1]) ++p;   // wave-uniform
    const int64_t n0 = t.col_off[p], Np = t.col_off[p + 1] - n0, Nt = t.col_off[t.parts];
    const int64_t idx = (b - t.blk_off[p]) * 256 + threadIdx.x;
    if (BITS == 4) {
        const int64_t K32 = K / 32, KT = K / 128;
        if (idx < K32 * Np) {
            const int64_t q = idx / Np, n = idx - q * Np, nf = n0 + n;
            const int64_t lane = (q & 3) * 16 + (nf & 15);
            ((uint4 *)dst_w)[((nf >> 4) * KT + (q >> 2)) * 64 + lane] =
                repack_quad((const uint32_t *)t.w[p], q, n, Np);
        }
    } else {
        if (idx < Np * (K / 16))
            ((uint4 *)dst_w)[n0 * (K / 16) + idx] = ((const uint4 *)t.w[p])[idx];
    }
    if (idx < (K / G) * Np) {
        const int64_t g = idx / Np, n = idx - g * Np;
        dst_s[g * Nt + n0 + n] = t.s[p][idx];
    }
}

hipError_t launch_fuse_pack(int bits, const void *const *w, const void *const *s,
                            const int64_t *widths, int parts, int64_t K, int G, void *dst_w,
                            void *dst_s, hipStream_t stream) {
    FuseTable t{};
    t.parts = parts;
    t.col_off[0] = t.blk_off[0] = 0;
    for (int p = 0; p < parts; ++p) {
        t.w[p] = w[p];
        t.s[p] = (const uint16_t *)s[p];
        const int64_t items = bits == 4 ? (K / 32) * widths[p] : widths[p] * (K / 16);
        t.col_off[p + 1] = t.col_off[p] + widths[p];
        t.blk_off[p + 1] = t.blk_off[p] + (items + 255) / 256;
    }
    const dim3 grid((uint32_t)t.blk_off[parts]);
    if (bits == 4)
        hipLaunchKernelGGL(fuse_pack_kernel<4>, grid, dim3(256), 0, stream, t, dst_w,
                           (uint16_t *)dst_s, K, G);
    else
        hipLaunchKernelGGL(fuse_pack_kernel<8>, grid, dim3(256), 0, stream, t, dst_w,
                           (uint16_t *)dst_s, K, G);
    return hipGetLastError();
}

// ---- compressed-tensors ingest -----------------------------------------------
// Compressed-tensors stores a W4A16 projection as words [N][K/8] and scales
// [N][K/G]; the GPTQ layout is their transpose, with each word unchanged (Eole
// recipe, section "Compressed-tensors INT4 layout"). A 64 x 64 tile transpose
// through LDS: reads run along a source row, writes along a destination row,
// and the padded LDS rows keep both phases free of bank conflicts. Words and
// scales go in one launch: the first `word_tiles` workgroups transpose word
// tiles, the rest scale tiles (a wave-uniform choice per workgroup).
template <typename T>
__device__ __forceinline__ void transpose_tile(const T *__restrict__ src, T *__restrict__ dst,
                                               int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                               uint32_t (*tile)[65]) {
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = (uint32_t)src[r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[c * rows + r] = (T)tile[tx][i];
    }
}

__global__ __launch_bounds__(256) void ct_transpose_kernel(const uint32_t *__restrict__ wp,
                                                           uint32_t *__restrict__ qw,
                                                           const uint16_t *__restrict__ ws,
                                                           uint16_t *__restrict__ s, int64_t N,
                                                           int64_t K8, int64_t KG, int64_t word_tiles) {
    __shared__ uint32_t tile[64][65];
    const int64_t tn = (N + 63) / 64;
    int64_t b = blockIdx.x;
    if (b < word_tiles) {
        transpose_tile<uint32_t>(wp, qw, N, K8, (b % tn) * 64, (b / tn) * 64, tile);
    } else {
        b -= word_tiles;
        transpose_tile<uint16_t>(ws, s, N, KG, (b % tn) * 64, (b / tn) * 64, tile);
    }
}

hipError_t launch_ct_to_gptq(const int32_t *wp, const void *ws, int32_t *qw, void *s, int64_t N,
                             int64_t K, int G, hipStream_t stream) {
    const int64_t K8 = K / 8, KG = K / G, tn = (N + 63) / 64;
    const int64_t word_tiles = tn * ((K8 + 63) / 64), scale_tiles = tn * ((KG + 63) / 64);
    hipLaunchKernelGGL(ct_transpose_kernel, dim3((uint32_t)(word_tiles + scale_tiles)), dim3(256), 0,
                       stream, (const uint32_t *)wp, (uint32_t *)qw, (const uint16_t *)ws,
                       (uint16_t *)s, N, K8, KG, word_tiles);
    return hipGetLastError();
}

}  // namespace svq
