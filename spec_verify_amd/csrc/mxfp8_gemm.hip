// MXFP8 weight-only GEMM kernels for gfx950: y = x . (e4m3(W) * 2^(e8m0(S)-127))^T.
//
// Format: MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp", opening summary
// (OCP Microscaling: 8-bit block floating point with E8M0 group scales, plain
// round-to-nearest), section "2. Precision plan" (kernel constraints N >= 128,
// K % 32 == 0) and section "8. License and attribution" (E8M0 shared scale per
// 32-element block). Elements are E4M3FN, stored [N][K]; scales [N][K/32].
//
// Dequant: v_cvt_scalef32_pk_bf16_fp8 turns two E4M3 codes into two bf16 values
// multiplied by the block's power-of-two scale; every E4M3 value times a
// power of two is exact in bf16 inside bf16's range, so the MAC operands equal
// the format's values. Unlike W4A16 no bias or per-group rescale is needed: the
// scale is applied before the products, so MFMA/dot2 accumulate straight into
// the fp32 result.
//
// Lane mapping for a 16-column x 128-row (of K) tile: lane l owns column l%16
// and the 32 consecutive K-rows 32*(l/16).. (one 32-element scale block, two
// 128-bit loads). The three kernels mirror the W4A16 ones: a VALU dot2 kernel
// with a row broadcast of x for M <= 8, a one-MFMA-tile kernel for M <= 16, and
// the persistent stream-K MFMA kernel with LDS-staged x for larger M.
#include "svq_launch.h"
#include "svq_streamk.h"
#include "dot2_asm.h"

namespace svq {

__device__ __forceinline__ uint4 cvt8_e4m3_bf16(uint32_t lo, uint32_t hi, float scale) {
    return make_uint4(e4m3_pair_scaled<false>(lo, scale), e4m3_pair_scaled<true>(lo, scale),
                      e4m3_pair_scaled<false>(hi, scale), e4m3_pair_scaled<true>(hi, scale));
}

// ---------------------------------------------------------------------------
// dot2 kernel, M <= 8
// ---------------------------------------------------------------------------
template <int M>
struct MxDot2Stage {
    uint4 w0, w1;    // 32 codes: K-rows 32*(lane/16) + 0..31 of column lane%16
    uint32_t x[M];   // bf16 pair (rows 2*lane, 2*lane+1 of the tile)
    uint32_t s;      // E8M0 code of this lane's block
};

template <int M, int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_dot2_kernel(
    const uint32_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rg = lane >> 4;
    const int nb = blockIdx.x;
    const int KT = K >> 7;
    const int col = nb * 16 + (lane & 15);
    const size_t KH = (size_t)K >> 1;
    const uint8_t *wp = w + (size_t)col * K + rg * 32;
    const uint8_t *sp = sc + (size_t)col * (K >> 5) + rg;
    const uint32_t *xp = x + lane;
    const int ntile = wave < KT ? (KT - 1 - wave) / WAVES + 1 : 0;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;

    auto load = [&](MxDot2Stage<M>(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            int i = i0 + d;
            i = i < ntile ? i : ntile - 1;
            const int kt = wave + i * WAVES;
            S[d].w0 = load_stream16(wp + (size_t)kt * 128);
            S[d].w1 = load_stream16(wp + (size_t)kt * 128 + 16);
#pragma unroll
            for (int m = 0; m < M; ++m) S[d].x[m] = xp[m * KH + (size_t)kt * 64];
            S[d].s = sp[(size_t)kt * 4];
        }
    };

    auto tile = [&](const MxDot2Stage<M> &S) {
        const float sf = e8m0_to_f32(S.s);
        const uint32_t wd[8] = {S.w0.x, S.w0.y, S.w0.z, S.w0.w, S.w1.x, S.w1.y, S.w1.z, S.w1.w};
        mxfp8_tile_dots<M>(acc, S.x, wd, sf);
    };

    auto compute = [&](const MxDot2Stage<M>(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d)
            if (i0 + d < ntile) tile(S[d]);
    };

    if (ntile > 0) {
        MxDot2Stage<M> A[D], B[D];
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
        for (int wv = 0; wv < WAVES; ++wv) s += red[wv][m][c];
        out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(s);
    }
}

// ---------------------------------------------------------------------------
// skinny MFMA kernel, M <= 16
// ---------------------------------------------------------------------------
struct MxSkinnyStage {
    uint4 w0, w1;
    uint4 a[4];
    uint32_t s;
};

template <int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_skinny_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, int M, int N, int K) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int nb = blockIdx.x;
    const int KT = K >> 7;
    const int col = nb * 16 + r;
    const uint8_t *wp = w + (size_t)col * K + g * 32;
    const uint8_t *sp = sc + (size_t)col * (K >> 5) + g;
    const bool arow = r < M;
    const uint16_t *xr = x + (size_t)(arow ? r : 0) * K + g * 32;
    const int ntile = wave < KT ? (KT - 1 - wave) / WAVES + 1 : 0;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};

    auto load = [&](MxSkinnyStage(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            int i = i0 + d;
            i = i < ntile ? i : ntile - 1;
            const int kt = wave + i * WAVES;
            S[d].w0 = load_stream16(wp + (size_t)kt * 128);
            S[d].w1 = load_stream16(wp + (size_t)kt * 128 + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                S[d].a[j] = arow ? *(const uint4 *)(xr + (size_t)kt * 128 + 8 * j) : make_uint4(0, 0, 0, 0);
            S[d].s = sp[(size_t)kt * 4];
        }
    };

    auto compute = [&](const MxSkinnyStage(&S)[D], int i0) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i0 + d >= ntile) continue;
            const float sf = e8m0_to_f32(S[d].s);
            acc = mfma16x16x32(S[d].a[0], cvt8_e4m3_bf16(S[d].w0.x, S[d].w0.y, sf), acc);
            acc = mfma16x16x32(S[d].a[1], cvt8_e4m3_bf16(S[d].w0.z, S[d].w0.w, sf), acc);
            acc = mfma16x16x32(S[d].a[2], cvt8_e4m3_bf16(S[d].w1.x, S[d].w1.y, sf), acc);
            acc = mfma16x16x32(S[d].a[3], cvt8_e4m3_bf16(S[d].w1.z, S[d].w1.w, sf), acc);
        }
    };

    if (ntile > 0) {
        MxSkinnyStage A[D], B[D];
        load(A, 0);
        for (int i0 = 0; i0 < ntile; i0 += 2 * D) {
            load(B, i0 + D);
            compute(A, i0);
            load(A, i0 + 2 * D);
            compute(B, i0 + D);
        }
    }

    __shared__ float red[WAVES][16][17];
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
    __syncthreads();
    for (int t = threadIdx.x; t < M * 16; t += 64 * WAVES) {
        const int m = t >> 4, c = t & 15;
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < WAVES; ++wv) s += red[wv][m][c];
        out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(s);
    }
}

// ---------------------------------------------------------------------------
// wide stream-K MFMA kernel, any M
// ---------------------------------------------------------------------------
template <int MBW, int WR, int WC, int CT>
__global__ __launch_bounds__(64 * WR * WC) void mxfp8_wide_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    f32x4 *__restrict__ part, int M, int N, int K, int col_tiles, int64_t units, int grid,
    int maxt) {
    constexpr int NT = 64 * WR * WC;
    constexpr int BM = 16 * MBW * WR;
    constexpr int BN = 16 * CT * WC;
    constexpr int XROW = 128 + 8;
    constexpr int UPT = BM * 16 / NT;
    constexpr int TPR = 16 / UPT;
    constexpr int NV = MBW * CT;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][XROW];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int r = lane & 15, g = lane >> 4;
    const int KT = K >> 7;
    const int NB16 = N >> 4;
    const int wg = blockIdx.x;
    const int64_t u_begin = (int64_t)wg * units / grid;
    const int64_t u_end = (int64_t)(wg + 1) * units / grid;
    const int srow = tid / TPR, sseg = tid % TPR;

    for (int64_t u = u_begin; u < u_end;) {
        const int tile = (int)(u / KT);
        const int s0 = (int)(u % KT);
        const int s1 = (int)((u_end - u) < (int64_t)(KT - s0) ? s0 + (u_end - u) : KT);
        const int rt = tile / col_tiles, cb = tile % col_tiles;
        const int row0 = rt * BM;

        const uint8_t *wp[CT];
        const uint8_t *spp[CT];
        bool ctv[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int nbg = cb * (BN / 16) + wc * CT + ct;
            ctv[ct] = nbg < NB16;
            const int colg = (ctv[ct] ? nbg : NB16 - 1) * 16 + r;
            wp[ct] = w + (size_t)colg * K + g * 32;
            spp[ct] = sc + (size_t)colg * (K >> 5) + g;
        }
        const bool srv = row0 + srow < M;
        const uint4 *xsrc = (const uint4 *)(x + (size_t)(srv ? row0 + srow : 0) * K) + sseg * UPT;

        f32x4 acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 xreg[UPT];
        uint4 wcur[CT][2], wnext[CT][2];
        uint32_t scur[CT], snext[CT];

        auto load_x = [&](int s) {
#pragma unroll
            for (int v = 0; v < UPT; ++v) xreg[v] = srv ? xsrc[(size_t)s * 16 + v] : make_uint4(0, 0, 0, 0);
        };
        auto load_w = [&](uint4(&W)[CT][2], uint32_t(&S)[CT], int s) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                W[ct][0] = load_stream16(wp[ct] + (size_t)s * 128);
                W[ct][1] = load_stream16(wp[ct] + (size_t)s * 128 + 16);
                S[ct] = spp[ct][(size_t)s * 4];
            }
        };
        auto compute = [&](int buf) {
            const int rbase = wr * MBW * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint4 A[MBW];
#pragma unroll
                for (int rb = 0; rb < MBW; ++rb) A[rb] = *(const uint4 *)&xs[buf][rbase + rb * 16 + r][32 * g + 8 * j];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const float sf = e8m0_to_f32(scur[ct]);
                    const uint4 &wv = wcur[ct][j >> 1];
                    const uint4 B = (j & 1) ? cvt8_e4m3_bf16(wv.z, wv.w, sf) : cvt8_e4m3_bf16(wv.x, wv.y, sf);
#pragma unroll
                    for (int rb = 0; rb < MBW; ++rb) acc[rb * CT + ct] = mfma16x16x32(A[rb], B, acc[rb * CT + ct]);
                }
            }
        };

        __syncthreads();
        load_x(s0);
        load_w(wcur, scur, s0);
        for (int s = s0; s < s1; ++s) {
            const int buf = (s - s0) & 1;
#pragma unroll
            for (int v = 0; v < UPT; ++v) *(uint4 *)&xs[buf][srow][(sseg * UPT + v) * 8] = xreg[v];
            __syncthreads();
            if (s + 1 < s1) {
                load_x(s + 1);
                load_w(wnext, snext, s + 1);
            }
            compute(buf);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                wcur[ct][0] = wnext[ct][0];
                wcur[ct][1] = wnext[ct][1];
                scur[ct] = snext[ct];
            }
        }

        const int rowb = row0 + wr * MBW * 16 + 4 * g;
        auto store_out = [&]() {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                if (!ctv[ct]) continue;
                const int colg = (cb * (BN / 16) + wc * CT + ct) * 16 + r;
#pragma unroll
                for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = rowb + rb * 16 + i;
                        if (row < M) out[(size_t)row * N + colg] = f32_to_bf16_rne(acc[rb * CT + ct][i]);
                    }
            }
        };
        if ((s0 == 0 && s1 == KT) || sk_fixup<NV, NT>(acc, tile, KT, units, grid, maxt, cnt, part, &s_last))
            store_out();
        u += s1 - s0;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
constexpr int kMxWaves = 8;
constexpr int kMxDot2Depth = 4;
constexpr int kMxSkinnyDepth = 2;

template <int M>
hipError_t mx_dot2_launch(const void *x, const uint8_t *w, const uint8_t *sc, void *out, int64_t N,
                          int64_t K, hipStream_t stream) {
    hipLaunchKernelGGL((mxfp8_dot2_kernel<M, kMxWaves, kMxDot2Depth>), dim3((uint32_t)(N / 16)),
                       dim3(64 * kMxWaves), 0, stream, (const uint32_t *)x, w, sc, (uint16_t *)out,
                       (int)N, (int)K);
    return hipGetLastError();
}

template <int MBW, int WR, int WC, int CT>
hipError_t mx_wide_launch(const WidePlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                          void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    const size_t cnt_bytes = ((size_t)p.row_tiles * p.col_tiles * 4 + 255) & ~(size_t)255;
    uint32_t *cnt = (uint32_t *)ws;
    f32x4 *part = ws ? (f32x4 *)((char *)ws + cnt_bytes) : nullptr;
    hipLaunchKernelGGL((mxfp8_wide_kernel<MBW, WR, WC, CT>), dim3((uint32_t)p.grid),
                       dim3(64 * WR * WC), 0, stream, (const uint16_t *)x, w, sc, (uint16_t *)out,
                       cnt, part, (int)M, (int)N, (int)K, p.col_tiles, p.units, p.grid, p.maxt);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_mxfp8_dot2(const void *x, const uint8_t *w, const uint8_t *scales, void *out,
                             int M, int64_t N, int64_t K, hipStream_t stream) {
    switch (M) {
    case 1: return mx_dot2_launch<1>(x, w, scales, out, N, K, stream);
    case 2: return mx_dot2_launch<2>(x, w, scales, out, N, K, stream);
    case 3: return mx_dot2_launch<3>(x, w, scales, out, N, K, stream);
    case 4: return mx_dot2_launch<4>(x, w, scales, out, N, K, stream);
    case 5: return mx_dot2_launch<5>(x, w, scales, out, N, K, stream);
    case 6: return mx_dot2_launch<6>(x, w, scales, out, N, K, stream);
    case 7: return mx_dot2_launch<7>(x, w, scales, out, N, K, stream);
    case 8: return mx_dot2_launch<8>(x, w, scales, out, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mxfp8_skinny(const void *x, const uint8_t *w, const uint8_t *scales, void *out,
                               int M, int64_t N, int64_t K, hipStream_t stream) {
    hipLaunchKernelGGL((mxfp8_skinny_kernel<kMxWaves, kMxSkinnyDepth>), dim3((uint32_t)(N / 16)),
                       dim3(64 * kMxWaves), 0, stream, (const uint16_t *)x, w, scales,
                       (uint16_t *)out, M, (int)N, (int)K);
    return hipGetLastError();
}

hipError_t launch_mxfp8_wide(const WidePlan &plan, const void *x, const uint8_t *w,
                             const uint8_t *scales, void *out, int64_t M, int64_t N, int64_t K,
                             void *workspace, hipStream_t stream) {
    if (plan.bm == 128) return mx_wide_launch<4, 2, 2, 4>(plan, x, w, scales, out, M, N, K, workspace, stream);
    return mx_wide_launch<4, 1, 4, 4>(plan, x, w, scales, out, M, N, K, workspace, stream);
}

}  // namespace svq
