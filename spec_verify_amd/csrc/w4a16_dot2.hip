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
#include "svq_streamk.h"

namespace svq {

template <int M, int WAVES, int D, int GSHIFT>
__global__ __launch_bounds__(64 * WAVES) void w4a16_dot2_kernel(
    const uint32_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int N, int K, int splits, int S) {
    constexpr int NG = 128 >> GSHIFT;  // groups per 128-row tile
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int rg = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int nb = lb / splits, sp = lb % splits;
    const int KT = K >> 7;
    // buffer views rebased on this workgroup's column block; tile kt of the
    // block is at byte kt*1024 of `wr`, x row m at byte m*2K of `xr`, and the
    // scale of group g for this lane's column at byte g*2N + 2*(lane%16) of `sr`
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt + (size_t)nb * KT * 64, (uint32_t)KT * 1024);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * K * 2);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + nb * 16, (uint32_t)(((size_t)(K >> GSHIFT) * N - nb * 16) * 2));
    const uint32_t w_vo = lane * 16;
    const uint32_t x_vo = lane * 4;
    // scales are loaded as the aligned dword holding this lane's fp16 and the
    // neighbouring column's; s_sh selects the half
    const uint32_t s_vo = ((rg * 32) >> GSHIFT) * N * 2 + (lane & 14) * 2;
    const int s_sh = (lane & 1) * 16;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = wave < kcnt ? (kcnt - 1 - wave) / WAVES + 1 : 0;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;

    uint4 wA[D], wB[D];
    uint32_t xA[D][M], xB[D][M], sA[D], sB[D];

    // Two register stages of D tiles each: the loads of one stage are in flight
    // while the other is computed. Every branch below is wave-uniform.
#define SVQ_LOAD(W, X, S, I0)                                                        \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wave + ((I0) + d) * WAVES;                                    \
        W[d] = bload16(wr, w_vo, kt * 1024);                                         \
        _Pragma("unroll") for (int m = 0; m < M; ++m) X[d][m] = bload4(xr, x_vo, m * K * 2 + kt * 256); \
        S[d] = bload4(sr, s_vo, kt * NG * N * 2);                                    \
    }
#define SVQ_COMPUTE(W, X, S, I0)                                                     \
    _Pragma("unroll") for (int d = 0; d < D; ++d) {                                  \
        float p[M];                                                                  \
        _Pragma("unroll") for (int m = 0; m < M; ++m)                                \
            p[m] = -136.f * row16_sum(dot2_bf16(X[d][m], kBf16OnePair, 0.f));        \
        const uint32_t wj[4] = {W[d].x, W[d].y, W[d].z, W[d].w};                     \
        w4a16_tile_dots<M>(p, X[d], wj, kNibblePairMask, kMagic128Pair);             \
        if ((I0) + d < ntile) {                                                      \
            const float sf = fp16_bits_to_f32((uint16_t)(S[d] >> s_sh));                       \
            _Pragma("unroll") for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(sf, p[m], acc[m]); \
        }                                                                            \
    }

    if (ntile > 0) {
        SVQ_LOAD(wA, xA, sA, 0)
        for (int i0 = 0;; i0 += 2 * D) {
            SVQ_LOAD(wB, xB, sB, i0 + D)
            SVQ_COMPUTE(wA, xA, sA, i0)
            if (i0 + D >= ntile) break;
            SVQ_LOAD(wA, xA, sA, i0 + 2 * D)
            SVQ_COMPUTE(wB, xB, sB, i0 + D)
            if (i0 + 2 * D >= ntile) break;
        }
    }
#undef SVQ_LOAD
#undef SVQ_COMPUTE

    __shared__ float red[WAVES][M][16];
#pragma unroll
    for (int m = 0; m < M; ++m) {
        const float v = rows4_sum(acc[m]);
        if (lane < 16) red[wave][m][lane] = v;
    }
    __syncthreads();
    __shared__ int s_flag;
    float v = 0.f;
    if (threadIdx.x < 16 * M) {
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[w][threadIdx.x >> 4][threadIdx.x & 15];
    }
    smallm_finish(v, M, N, nb, sp, splits, out, cnt, part, &s_flag);
}

namespace {
constexpr int kDot2Depth = 4;

template <int M, int WAVES, int GS>
hipError_t dot2_launch_w(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                         int64_t N, int64_t K, void *ws, hipStream_t stream) {
    hipLaunchKernelGGL((w4a16_dot2_kernel<M, WAVES, kDot2Depth, GS>),
                       dim3((uint32_t)(N / 16 * p.splits)), dim3(64 * WAVES), 0, stream,
                       (const uint32_t *)x, (const uint4 *)wt, (const uint16_t *)sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), (int)N, (int)K, p.splits, p.S);
    return hipGetLastError();
}

template <int M, int GS>
hipError_t dot2_launch(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                       int64_t N, int64_t K, void *ws, hipStream_t stream) {
    static const int r16 = resident_blocks(w4a16_dot2_kernel<M, 16, kDot2Depth, GS>, 1024);
    static const int r8 = resident_blocks(w4a16_dot2_kernel<M, 8, kDot2Depth, GS>, 512);
    switch (pick_waves(N / 16 * p.splits, p.cus, r16, r8)) {
    case 16: return dot2_launch_w<M, 16, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 8: return dot2_launch_w<M, 8, GS>(p, x, wt, sc, out, N, K, ws, stream);
    default: return dot2_launch_w<M, 4, GS>(p, x, wt, sc, out, N, K, ws, stream);
    }
}

template <int GS>
hipError_t dot2_by_m(const SmallPlan &p, int M, const void *x, const int32_t *wt, const void *sc,
                     void *out, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    switch (M) {
    case 1: return dot2_launch<1, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 2: return dot2_launch<2, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 3: return dot2_launch<3, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 4: return dot2_launch<4, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 5: return dot2_launch<5, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 6: return dot2_launch<6, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 7: return dot2_launch<7, GS>(p, x, wt, sc, out, N, K, ws, stream);
    case 8: return dot2_launch<8, GS>(p, x, wt, sc, out, N, K, ws, stream);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_w4a16_dot2(const SmallPlan &plan, const void *x, const int32_t *wt,
                             const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                             void *workspace, hipStream_t stream) {
    switch (G) {
    case 32: return dot2_by_m<5>(plan, M, x, wt, scales, out, N, K, workspace, stream);
    case 64: return dot2_by_m<6>(plan, M, x, wt, scales, out, N, K, workspace, stream);
    case 128: return dot2_by_m<7>(plan, M, x, wt, scales, out, N, K, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace svq
