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
        _Pragma("unroll") for (int m = 0; m < M; ++m) X[d][m] = bload4(xr, x_vo, m * K * 2 + kt * 256); \
        W[d] = bload16(wr, w_vo, kt * 1024);                                         \
        S[d] = bload4(sr, s_vo, kt * NG * N * 2);                                    \
    }
#define SVQ_COMPUTE(W, X, S, I0)                                                     \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        float p[M];                                                                  \
        _Pragma("unroll") for (int m = 0; m < M; ++m)                                \
            p[m] = -136.f * row16_sum(dot2_bf16(X[d][m], kBf16OnePair, 0.f));        \
        const uint32_t wj[4] = {W[d].x, W[d].y, W[d].z, W[d].w};                     \
        w4a16_tile_dots<M>(p, X[d], wj, kNibblePairMask, kMagic128Pair);             \
        const float sf = fp16_bits_to_f32((uint16_t)(S[d] >> s_sh));                 \
        _Pragma("unroll") for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(sf, p[m], acc[m]); \
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

// Narrow-unit GEMV for M = 1..2 where the matrix has fewer 16-column blocks
// than the chip has CUs (a decode projection with N = 1024 has 64 blocks: the
// kernel above would leave three quarters of the CUs idle, and splitting K
// across workgroups costs a cross-workgroup handoff). The work unit is 4
// output columns over all of K, so N/4 units spread over all the CUs with no
// split of K. Measured on the MI355X, M = 1, K = 5120: N = 1024 took 4.4 us
// against 5.0 us for the block kernel when this kernel was introduced (3.35 us
// now, with four waves per unit); with N >= 16 x CUs the block kernel is as
// fast or faster, so it keeps those shapes.
//  * A workgroup owns `upw` consecutive units; `wpu` waves share each unit's
//    128-row tiles, four tiles per load: lane l reads the 16 bytes of tile
//    4g + l/16 that hold rows 32*((l/4)%4).. of the unit's column l%4 (four
//    lanes read one contiguous 64-byte run), so one wave load covers four
//    tiles of the unit and every byte is read once.
//  * x (M rows, zero-padded to whole groups of four tiles) is staged in LDS
//    once per workgroup with the sums of each 32-row run (for the -136*sum(x)
//    bias); each lane then reads its 32 rows of x from LDS.
//  * All of a wave's weight and scale loads are issued before x is staged, so
//    the HBM stream starts at once; the x loads are issued before them, so the
//    wait for x leaves the weight loads in flight.
//  * Reduction: the 16 lanes of a column (4 tiles x 4 row runs) with row
//    rotations and permlane swaps, the waves of a unit through LDS, in a fixed
//    order.
constexpr int kNarrowCols = 4;      // output columns per unit
constexpr int kNarrowXChunks = 4;   // most 16-byte x chunks one thread stages

template <int M, int CW, int LPW, int GSHIFT>
__global__ __launch_bounds__(1024) void w4a16_narrow_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt, const uint16_t *__restrict__ sc,
    uint16_t *__restrict__ out, int N, int K, int upw, int wpu) {
    extern __shared__ __align__(16) unsigned char narrow_lds[];
    constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every operand: reads zero
    constexpr int TPL = 16 / CW;  // tiles per wave load
    const int KT = K >> 7;
    const int TG = (KT + TPL - 1) / TPL;  // groups of TPL tiles
    const int KTp = TG * TPL;
    uint16_t *xs = (uint16_t *)narrow_lds;                    // [M][KTp * 128] bf16
    float *xsum = (float *)(narrow_lds + (size_t)M * KTp * 256);  // [M][KTp * 4]
    float *red = xsum + M * KTp * 4;                           // [waves][M][CW]

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int units = N / CW;
    const int unit = lb * upw + wave / wpu;
    const int sub = wave % wpu;
    const bool live = unit < units;
    const int nb = unit / TPL, c0 = (unit % TPL) * CW;
    const int u = lane / (4 * CW), rg = (lane / CW) & 3, c = lane % CW;
    const int n = nb * 16 + c0 + c;

    // x chunks first (16 bytes each; past K or past the stage: zero, no traffic)
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)(M * K * 2));
    const int xchunks = M * KTp * 16;
    uint4 xv[kNarrowXChunks];
#pragma unroll
    for (int i = 0; i < kNarrowXChunks; ++i) {
        const int ch = threadIdx.x + i * blockDim.x;
        const int m = ch / (KTp * 16), k0 = (ch - m * KTp * 16) * 8;
        const uint32_t vo = (ch < xchunks && k0 < K) ? (uint32_t)((m * K + k0) * 2) : kOob;
        xv[i] = bload16(xr, vo, 0);
    }
    // then every weight and scale load of this wave, in the order they are
    // used (the scheduling barriers keep the issue order: waits are in order)
    __builtin_amdgcn_sched_barrier(0);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt, (uint32_t)((size_t)N * K / 2));
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc, (uint32_t)((size_t)(K >> GSHIFT) * N * 2));
    uint4 w[LPW];
    uint32_t s[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int t = (sub + i * wpu) * TPL + u;
        const bool ok = live && t < KT;
        const uint32_t wvo = ok ? (uint32_t)((nb * KT + t) * 1024 + rg * 256 + (c0 + c) * 16) : kOob;
        const int g = (t * 128 + rg * 32) >> GSHIFT;
        const uint32_t svo = ok ? (uint32_t)(((g * N + n) * 2) & ~3) : kOob;
        w[i] = bload16(wr, wvo, 0);
        s[i] = bload4(sr, svo, 0);
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // stage x and the sums of its 32-row runs (four consecutive chunks, which
    // sit in four consecutive lanes)
#pragma unroll
    for (int i = 0; i < kNarrowXChunks; ++i) {
        const int ch = threadIdx.x + i * blockDim.x;
        const uint32_t wd[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) v += bits_f32(wd[j] << 16) + bits_f32(wd[j] & 0xFFFF0000u);
        v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
        v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
        if (ch < xchunks) {
            *(uint4 *)(xs + (size_t)ch * 8) = xv[i];
            if ((ch & 3) == 0) xsum[ch >> 2] = v;
        }
    }
    lds_barrier();

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int tg = sub + i * wpu;
        if (!live || tg >= TG) break;
        const int t = tg * TPL + u;
        const uint32_t wj[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
        const float sf = fp16_bits_to_f32((uint16_t)(s[i] >> ((n & 1) * 16)));
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const u32x4 *xp = (const u32x4 *)(xs + (size_t)m * KTp * 128 + t * 128 + rg * 32);
            const u32x4 xa = xp[0], xb = xp[1], xc = xp[2], xd = xp[3];
            const uint32_t xq[16] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w,
                                     xc.x, xc.y, xc.z, xc.w, xd.x, xd.y, xd.z, xd.w};
            // two interleaved chains (pairs of even and odd word index)
            float p0 = -136.f * xsum[m * KTp * 4 + t * 4 + rg], p1 = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 pw = word_to_pairs(wj[j]);
                const uint32_t pr[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (j & 1) p1 = dot2_bf16(pr[q], xq[4 * j + q], p1);
                    else p0 = dot2_bf16(pr[q], xq[4 * j + q], p0);
                }
            }
            acc[m] = __builtin_fmaf(sf, p0 + p1, acc[m]);
        }
    }

    // column sums: over the four row runs (rotations by 4 and 8 within a row),
    // then over the four tiles (the 16-lane rows)
#pragma unroll
    for (int m = 0; m < M; ++m) {
        float v = acc[m];
        if constexpr (CW == 4)
            v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x124, 0xF, 0xF, true));  // row_ror:4
        v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x128, 0xF, 0xF, true));  // row_ror:8
        v = rows4_sum(v);
        if (lane < CW) red[(wave * M + m) * CW + lane] = v;
    }
    lds_barrier();
    const int tid = threadIdx.x;
    if (tid < upw * M * CW) {
        const int ul = tid / (M * CW), m = (tid / CW) % M, cc = tid % CW;
        const int un = lb * upw + ul;
        float v = 0.f;
        for (int q = 0; q < wpu; ++q) v += red[((ul * wpu + q) * M + m) * CW + cc];
        if (un < units) out[(size_t)m * N + un * CW + cc] = f32_to_bf16_rne(v);
    }
}

namespace {
constexpr int kDot2Depth = 4;
constexpr int kNarrowPerCu = 1;  // workgroups per CU of the narrow-unit plan

template <int M, int WAVES, int GS>
hipError_t dot2_launch_w(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                         int64_t N, int64_t K, void *ws, hipStream_t stream) {
    return launch_gemm(w4a16_dot2_kernel<M, WAVES, kDot2Depth, GS>,
                       dim3((uint32_t)(N / 16 * p.splits)), dim3(64 * WAVES), 0, stream,
                       (const uint32_t *)x, (const uint4 *)wt, (const uint16_t *)sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), (int)N, (int)K, p.splits, p.S);
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

// Narrow-unit plan: units of 4 columns, `upw` per workgroup (about `per_cu`
// workgroups per CU), `wpu` waves per unit, each wave issuing at most `lpw`
// four-tile loads, all of them up front.
struct NarrowPlan {
    int upw, wpu, lpw, waves, grid;
    size_t lds;
};

bool plan_narrow(int M, int64_t N, int64_t K, int cus, int per_cu, NarrowPlan &p) {
    if (M > 2 || cus <= 0) return false;
    const int64_t units = N / kNarrowCols, KT = K / 128, TPL = 16 / kNarrowCols, TG = (KT + TPL - 1) / TPL;
    if (N / 16 >= cus) return false;  // enough 16-column blocks: the block kernel
    if (units < cus) return false;     // too few units to fill the chip: the split-K path
    const int64_t target = (int64_t)cus * per_cu;
    const int64_t upw = (units + target - 1) / target;
    if (upw > 16) return false;
    // Few waves per unit: a workgroup of fewer waves is dispatched sooner (a
    // timeline of the N = 1024 GEMV showed workgroup starts spread over 1.3 us
    // at 10 waves each), so the most waves is not the fastest: M = 1, K = 5120,
    // N = 1024 takes 3.35 us at 4 waves (three loads each) against 3.77 at 10,
    // 3.39 at 3 and 3.8 at 2 (where each thread stages twice the x). At least
    // as many as keep each wave at eight loads and the x stage at four chunks
    // per thread.
    const int64_t lo = std::max<int64_t>((TG + 7) / 8, (M * TG * TPL * 16 + kNarrowXChunks * 64 * upw - 1) /
                                                            (kNarrowXChunks * 64 * upw));
    const int64_t wpu = std::min<int64_t>(std::min<int64_t>(16 / upw, TG), std::max<int64_t>(4, lo));
    const int64_t lpw = (TG + wpu - 1) / wpu;
    if (lpw > 8) return false;
    const int64_t waves = upw * wpu;
    if ((int64_t)M * TG * TPL * 16 > (int64_t)kNarrowXChunks * waves * 64) return false;
    p.upw = (int)upw;
    p.wpu = (int)wpu;
    p.lpw = (int)lpw;
    p.waves = (int)waves;
    p.grid = (int)((units + upw - 1) / upw);
    p.lds = (size_t)M * TG * TPL * (256 + 16) + (size_t)waves * M * kNarrowCols * 4;
    return p.lds <= 64 * 1024;
}

template <int M, int LPW, int GS>
hipError_t narrow_launch_l(const NarrowPlan &p, const void *x, const int32_t *wt, const void *sc,
                           void *out, int64_t N, int64_t K, hipStream_t stream) {
    return launch_gemm(w4a16_narrow_kernel<M, kNarrowCols, LPW, GS>, dim3((uint32_t)p.grid), dim3(64 * p.waves),
                       p.lds, stream, (const uint16_t *)x, (const uint4 *)wt, (const uint16_t *)sc,
                       (uint16_t *)out, (int)N, (int)K, p.upw, p.wpu);
}

template <int M, int GS>
hipError_t narrow_launch(const NarrowPlan &p, const void *x, const int32_t *wt, const void *sc,
                         void *out, int64_t N, int64_t K, hipStream_t stream) {
    switch (p.lpw) {
    case 1: return narrow_launch_l<M, 1, GS>(p, x, wt, sc, out, N, K, stream);
    case 2: return narrow_launch_l<M, 2, GS>(p, x, wt, sc, out, N, K, stream);
    case 3: return narrow_launch_l<M, 3, GS>(p, x, wt, sc, out, N, K, stream);
    case 4: return narrow_launch_l<M, 4, GS>(p, x, wt, sc, out, N, K, stream);
    case 5: return narrow_launch_l<M, 5, GS>(p, x, wt, sc, out, N, K, stream);
    case 6: return narrow_launch_l<M, 6, GS>(p, x, wt, sc, out, N, K, stream);
    default: return narrow_launch_l<M, 8, GS>(p, x, wt, sc, out, N, K, stream);
    }
}

template <int GS>
hipError_t dot2_by_m(const SmallPlan &p, int M, const void *x, const int32_t *wt, const void *sc,
                     void *out, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    NarrowPlan np;
    if (p.splits == 1 && plan_narrow(M, N, K, p.cus, kNarrowPerCu, np))
        return M == 1 ? narrow_launch<1, GS>(np, x, wt, sc, out, N, K, stream)
                      : narrow_launch<2, GS>(np, x, wt, sc, out, N, K, stream);
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

bool w4a16_dot2_is_narrow(const SmallPlan &plan, int M, int64_t N, int64_t K, int G) {
    (void)G;
    NarrowPlan np;
    return plan.splits == 1 && plan_narrow(M, N, K, plan.cus, kNarrowPerCu, np);
}

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
