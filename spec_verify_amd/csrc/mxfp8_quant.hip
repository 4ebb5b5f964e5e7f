// MXFP8 quantizer: dense bf16 weights [N][K] -> E4M3FN codes [N][K] and one
// E8M0 scale per 32 consecutive K-elements [N][K/32], the svq_mxfp8_gemm input.
//
// MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp": plain round-to-nearest
// (opening summary) and the optimized round-to-nearest of its notes on the
// quantizer's behaviour, which evaluates the baseline block scale together
// with the scales twice and half as large and keeps the best.
//
// Per block: the baseline exponent is the OCP MX one, X0 = floor(log2 amax) - 8
// (8 is E4M3's largest normal exponent), E8M0 b0 = clamp(X0 + 127, 0, 254), and
// an all-zero block takes b0 = 127. A candidate b (b0, then b0 + 1, then b0 - 1,
// each within 0..254) codes every element as E4M3_RNE(|v| / 2^(b-127)),
// saturating at 448, with the sign of v, and scores the squared differences
// between v and the decoded values, added in ascending element order in fp32.
// A later candidate replaces the kept one only with a strictly smaller score.
// The score is computed with explicit round-to-nearest subtract, multiply and
// add (no contraction), so the choice depends on nothing but these steps. The
// kernel scores only the candidates that can win (the reasons are given where
// the candidates are scored), which gives the same choice.
//
// One thread per block: 64 bytes of bf16 in, 32 code bytes and 1 scale byte
// out. Consecutive threads take consecutive blocks of a row, so loads, code
// stores and scale stores are contiguous across a wave. The three candidates
// cost ~2.4k VALU operations per block, which makes the kernel ALU-bound
// (about 5x the time of its HBM traffic); it runs once, when a model is
// quantized.
#include "svq_launch.h"

namespace svq {
namespace {

// |a| (finite, >= 0) -> E4M3FN magnitude code 0..0x7E, nearest value, ties to
// the even code, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_mag_rne(float a) {
    if (!(a < 448.0f)) return 0x7Eu;
    if (a < 0.015625f)                                   // below 2^-6: multiples of 2^-9
        return (uint32_t)rintf(a * 512.0f);              // 8 lands on code 0x08 = 2^-6
    const uint32_t u = __float_as_uint(a);
    const int e = (int)(u >> 23) - 127;                  // -6 .. 8
    const float mant = __uint_as_float((u & 0x7FFFFFu) | 0x3F800000u);
    const uint32_t m = (uint32_t)rintf((mant - 1.0f) * 8.0f);   // 0..8; 8 carries
    return ((uint32_t)(e + 7) << 3) + m;                 // a < 448 keeps this <= 0x7E
}

// E4M3FN magnitude code -> its value (exact in fp32).
__device__ __forceinline__ float e4m3_mag_value(uint32_t c) {
    const uint32_t e = c >> 3, m = c & 7u;
    return e == 0 ? (float)m * 0.001953125f : ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
}

// floor(log2 a) of a finite a > 0 (fp32 subnormals included).
__device__ __forceinline__ int floor_log2(float a) {
    const uint32_t u = __float_as_uint(a);
    const int e = (int)(u >> 23);
    if (e > 0) return e - 127;
    return (31 - __clz((int)(u & 0x7FFFFFu))) - 149;
}

// Codes of the block at E8M0 code b, packed 4 per word, and their fp32 score.
__device__ __forceinline__ float mx_candidate(const float (&v)[32], int b, uint32_t (&codes)[8]) {
    const int X = b - 127;
    float err = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x = v[4 * w + j];
            const uint32_t neg = __float_as_uint(x) >> 31;
            const uint32_t mag = e4m3_mag_rne(ldexpf(fabsf(x), -X));
            const float d = ldexpf(e4m3_mag_value(mag), X);
            const float diff = __fsub_rn(x, neg ? -d : d);
            err = __fadd_rn(err, __fmul_rn(diff, diff));
            word |= (mag | (neg << 7)) << (8 * j);
        }
        codes[w] = word;
    }
    return err;
}

__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint4 *__restrict__ w,
                                                             uint4 *__restrict__ codes,
                                                             uint8_t *__restrict__ scales,
                                                             int64_t blocks, int optimized) {
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (b >= blocks) return;
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 p = w[b * 4 + q];
        const uint32_t d[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * q + 2 * j] = __uint_as_float(d[j] << 16);
            v[8 * q + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int b0 = 127;
    if (amax > 0.0f) b0 = min(max(floor_log2(amax) - 8 + 127, 0), 254);

    uint32_t best[8], cand[8];
    float best_err = mx_candidate(v, b0, best);
    int best_b = b0;
    // Of the other two candidates only twice the scale can win, and only when
    // the baseline saturates an element (amax / 2^X > 448), so only then is it
    // scored; the choice is the same as scoring both in order:
    //  * No element above 448 * 2^X: at twice the scale every element's nearest
    //    representable value is one the baseline also has, so each element's
    //    error is at least the baseline's, and the fp32 sum of element errors
    //    in the same order (rounded addition is monotonic) is not smaller.
    //  * Half the scale (b0 > 0, so amax / 2^X is in [256, 512)): the block
    //    maximum saturates and its error grows by at least 768 * 4^X, while only
    //    elements below the baseline's normal range (error < 2^(2X-10) each)
    //    can gain; fp32 rounding of the sums is far below the difference, and
    //    where 4^X is so small that it is not, those gains round to zero. So
    //    half the scale is never strictly better and is not scored.
    const bool sat = ldexpf(amax, 127 - b0) > 448.0f;
    if (optimized) {
        // the candidates in the definition's order, skipping those that cannot
        // win (the loop form keeps one copy of the scoring code)
#pragma unroll 1
        for (int k = 0; k < 2; ++k) {
            const int bc = k == 0 ? b0 + 1 : b0 - 1;
            const bool can_win = k == 0 && sat;
            if (bc < 0 || bc > 254 || !can_win) continue;
            const float e = mx_candidate(v, bc, cand);
            if (e < best_err) {
                best_err = e;
                best_b = bc;
#pragma unroll
                for (int i = 0; i < 8; ++i) best[i] = cand[i];
            }
        }
    }
    codes[b * 2] = make_uint4(best[0], best[1], best[2], best[3]);
    codes[b * 2 + 1] = make_uint4(best[4], best[5], best[6], best[7]);
    scales[b] = (uint8_t)best_b;
}

}  // namespace

hipError_t launch_mxfp8_quantize(const void *w, int optimized, uint8_t *codes, uint8_t *scales,
                                 int64_t N, int64_t K, hipStream_t stream) {
    const int64_t blocks = N * (K / 32);
    hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((uint32_t)((blocks + 255) / 256)), dim3(256), 0,
                       stream, (const uint4 *)w, (uint4 *)codes, scales, blocks, optimized);
    return hipGetLastError();
}

}  // namespace svq
