// W4A16 GEMV-class kernel for the smallest verify chunks (M = 1..8) on gfx950.
//
// What it computes: y[m][n] = sum_k x[m][k] * (q[k][n] - 8) * s[k/G][n] with fp32
// accumulation and a bf16 (round-to-nearest-even) result. Weight format: GPTQ
// INT4 card "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16", section "Quantization
// contract" (symmetric INT4, group 128, desc_act off); group sizes 32/64/128 as
// accepted by the Eole recipe "Qwen3.8-27B and native MTP speculative decoding",
// section "Compressed-tensors INT4 layout".
//
// Design (memory-bound: 0.5 B of weight per 2*M flops):
//  * A workgroup owns one 16-column block and all of K; its WAVES waves take
//    the block's 1 KiB tiles round-robin, so at any moment the workgroup streams
//    WAVES consecutive KiB. Each wave keeps 2*D tiles in flight.
//  * One 128-bit load per lane per tile (64 lanes x 16 B = one tile). Lane l
//    owns column l%16 and the 32 K-rows 32*(l/16).. of the tile: a split of K
//    across the four 16-lane rows of the wave.
//  * Dequant in registers: (w >> 4s) & 0x000F000F | 0x43004300 turns two nibbles
//    into the exact bf16 pair (128 + q0, 128 + q1).
//  * x is one 32-bit bf16 pair per lane per tile (lane L holds rows 2L, 2L+1);
//    v_dot2c_f32_bf16 with a DPP row_newbcast hands lane i's pair to the whole
//    16-lane row, so no lane ever loads or stores a copy of x. The dot chain of
//    a tile is one generated asm block (dot2_asm.h) that keeps the gfx950 DPP
//    and DOT wait states itself.
//  * The 128 + q bias is removed per tile: the partial starts at -136 * (sum of
//    the 32 x values of the row), then the fp16 group scale multiplies it into
//    the fp32 accumulator.
//  * Epilogue: the four 16-lane rows are summed with permlane16/permlane32
//    swaps (a wavefront reduction), the waves through LDS, in a fixed order.
#include "svq_launch.h"
#include "dot2_asm.h"

namespace svq {

template <int M>
struct Dot2Stage {
    uint4 w;         // this lane's 16 bytes of the tile
    uint32_t x[M];   // bf16 pair (rows 2*lane, 2*lane+1 of the tile) of each x row
    uint16_t s;      // fp16 scale of this lane's group and column
};

template <int M, int WAVES, int D, int GSHIFT>
__global__ __launch_bounds__(64 * WAVES) void w4a16_dot2_kernel(
    const uint32_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, int N, int K) {
    constexpr int NG = 128 >> GSHIFT;  // groups per 128-row tile
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = lane >> 4;
    const int nb = blockIdx.x;
    const int KT = K >> 7;
    const int col = nb * 16 + (lane & 15);
    const size_t KH = (size_t)K >> 1;
    const uint4 *tp = wt + (size_t)nb * KT * 64 + lane;
    const uint32_t *xp = x + lane;
    const uint16_t *sp = sc + col;
    const int gsub = (rg * 32) >> GSHIFT;
    const int ntile = wave < KT ? (KT - 1 - wave) / WAVES + 1 : 0;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;

    // Loads are unconditional (tile index clamped to the wave's last tile) so
    // the compiler can count outstanding loads statically; out-of-range tiles
    // are loaded again and skipped.
    auto load = [&](Dot2Stage<M>(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            int i = i0 + d;
            i = i < ntile ? i : ntile - 1;
            const int kt = wave + i * WAVES;
            S[d].w = load_stream16(tp + (size_t)kt * 64);
#pragma unroll
            for (int m = 0; m < M; ++m) S[d].x[m] = xp[m * KH + (size_t)kt * 64];
            S[d].s = sp[(size_t)(kt * NG + gsub) * N];
        }
    };

    auto tile = [&](const Dot2Stage<M> &S) {
        float p[M];
#pragma unroll
        for (int m = 0; m < M; ++m) p[m] = -136.f * row16_sum(dot2_bf16(S.x[m], kBf16OnePair, 0.f));
        const uint32_t wj[4] = {S.w.x, S.w.y, S.w.z, S.w.w};
        w4a16_tile_dots<M>(p, S.x, wj, kNibblePairMask, kMagic128Pair);
        const float sf = fp16_bits_to_f32(S.s);
#pragma unroll
        for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(sf, p[m], acc[m]);
    };

    auto compute = [&](const Dot2Stage<M>(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (i0 + d < ntile) tile(S[d]);
    };

    if (ntile > 0) {
        Dot2Stage<M> A[D], B[D];
        load(A, 0);
        for (int i0 = 0; i0 < ntile; i0 += 2 * D) {
            load(B, i0 + D);
            compute(A, i0);
            load(A, i0 + 2 * D);
            compute(B, i0 + D);
        }
    }

    __shared__ float red[WAVES][M][16];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float v = rows4_sum(acc[m]);
        if (lane < 16) red[wave][m][lane] = v;
    }
    __syncthreads();
    for (int t = threadIdx.x; t < M * 16; t += 64 * WAVES) {
        const int m = t >> 4, c = t & 15;
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) s += red[w][m][c];
        out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(s);
    }
}

namespace {
constexpr int kDot2Waves = 8;
constexpr int kDot2Depth = 4;

template <int M, int GS>
hipError_t dot2_launch(const void *x, const int32_t *wt, const void *sc, void *out, int64_t N,
                       int64_t K, hipStream_t stream) {
    hipLaunchKernelGGL((w4a16_dot2_kernel<M, kDot2Waves, kDot2Depth, GS>), dim3((uint32_t)(N / 16)),
                       dim3(64 * kDot2Waves), 0, stream, (const uint32_t *)x, (const uint4 *)wt,
                       (const uint16_t *)sc, (uint16_t *)out, (int)N, (int)K);
    return hipGetLastError();
}

template <int GS>
hipError_t dot2_by_m(int M, const void *x, const int32_t *wt, const void *sc, void *out,
                     int64_t N, int64_t K, hipStream_t stream) {
    switch (M) {
    case 1: return dot2_launch<1, GS>(x, wt, sc, out, N, K, stream);
    case 2: return dot2_launch<2, GS>(x, wt, sc, out, N, K, stream);
    case 3: return dot2_launch<3, GS>(x, wt, sc, out, N, K, stream);
    case 4: return dot2_launch<4, GS>(x, wt, sc, out, N, K, stream);
    case 5: return dot2_launch<5, GS>(x, wt, sc, out, N, K, stream);
    case 6: return dot2_launch<6, GS>(x, wt, sc, out, N, K, stream);
    case 7: return dot2_launch<7, GS>(x, wt, sc, out, N, K, stream);
    case 8: return dot2_launch<8, GS>(x, wt, sc, out, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_w4a16_dot2(const void *x, const int32_t *wt, const void *scales, void *out,
                             int M, int64_t N, int64_t K, int G, hipStream_t stream) {
    switch (G) {
    case 32: return dot2_by_m<5>(M, x, wt, scales, out, N, K, stream);
    case 64: return dot2_by_m<6>(M, x, wt, scales, out, N, K, stream);
    case 128: return dot2_by_m<7>(M, x, wt, scales, out, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace svq
