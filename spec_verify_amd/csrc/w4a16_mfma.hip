// W4A16 MFMA kernels for gfx950: v_mfma_f32_16x16x32_bf16 on weights dequantized
// in registers from the 16-column x 128-row tile layout.
//
// What they compute: y[m][n] = sum_k x[m][k] * (q[k][n] - 8) * s[k/G][n], fp32
// accumulation, bf16 (RNE) output. Format: GPTQ INT4 card
// "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16", section "Quantization contract";
// group sizes 32/64/128 per the Eole recipe "Qwen3.8-27B and native MTP
// speculative decoding", section "Compressed-tensors INT4 layout". The batched
// verify shape (32 streams x (1 + 3) tokens) comes from the autobench page
// "Qwen3.8-27B · vLLM · FP8 + MTP" (concurrency 32, three speculative tokens).
//
// Operand mapping (16x16x32 bf16): lane l supplies row/column l%16 and 8 K-values
// of K-group l/16 for both A (x) and B (weights); C holds rows 4*(l/16)+i of
// column l%16. A tile word j of lane l covers rows 32*(l/16) + 8j + (0..7), so
// for G = 128 MFMA step j simply takes word j, with x read at the same rows; for
// G = 32/64 the four words and the four 16-lane rows are first transposed
// (permlane swaps) so that step j covers the contiguous rows 32j.. of one group.
//
// Weights enter the MFMA as the exact bf16 values 128 + q; the bias is removed
// per group by starting the group's accumulator at -136 * (sum of x over the
// group), then the fp16 scale multiplies the group result into fp32 accumulators.
#include <algorithm>

#include "svq_launch.h"
#include "svq_streamk.h"

namespace svq {

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16, one 16-row MFMA tile (MFMA rows >= M repeat row M-1
// and their results are dropped). A workgroup owns one 16-column block and a
// range of S K-tiles; its waves take the tiles round-robin. The workgroup's
// x rows (M x 128*S bf16) are staged once in LDS, so the A operands come from
// LDS and the vector-memory path carries only weights and scales, which each
// wave prefetches 2*D tiles deep behind the staging loads. Memory-bound; the
// MFMA pipe is mostly idle, so the -136 * sum(x) term is also computed on it,
// by an MFMA against a constant -136 operand.
// ---------------------------------------------------------------------------
template <int WAVES, int D, int GSHIFT>
__global__ __launch_bounds__(64 * WAVES) void w4a16_skinny_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int M, int N, int K, int splits, int S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NG = 128 >> GSHIFT;
    constexpr int SPG = 4 / NG;
    constexpr bool kTrans = GSHIFT < 7;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int nb = lb / splits, sp = lb % splits;
    const int KT = K >> 7;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt + (size_t)nb * KT * 64, (uint32_t)KT * 1024);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + nb * 16, (uint32_t)(((size_t)(K >> GSHIFT) * N - nb * 16) * 2));
    const uint32_t w_vo = lane * 16;
    // the aligned dword holding this lane's fp16 scale; s_sh selects the half
    const uint32_t s_vo = (r & 14) * 2;
    const int s_sh = (r & 1) * 16;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = wave < kcnt ? (kcnt - 1 - wave) / WAVES + 1 : 0;
    const uint4 bneg = make_uint4(kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair);

    uint4 wA[D], wB[D];
    uint32_t sA[D][NG], sB[D][NG];
#define SVQ_LOAD(W, SS, I0)                                                          \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wave + ((I0) + d) * WAVES;                             \
        W[d] = bload16(wr, w_vo, kt * 1024);                                         \
        _Pragma("unroll") for (int q = 0; q < NG; ++q) SS[d][q] = bload4(sr, s_vo, (kt * NG + q) * N * 2); \
    }
    // stage x[0..M)[128*kbeg, 128*(kbeg+kcnt)) in LDS by DMA (one 64-chunk
    // segment of a row per instruction); rows padded by 16 bytes so that the
    // 16-byte A reads of different rows fall in different banks. The weight
    // prefetch is issued behind it, and only the x loads are waited for.
    const int xs_stride = kcnt * 256 + 16;
    {
        const int row_chunks = kcnt * 16;
        const int nseg = (row_chunks + 63) >> 6;
        for (int i = wave; i < M * nseg; i += WAVES) {
            const int m = i / nseg, c = ((i - m * nseg) << 6) + lane;
            if (c < row_chunks)
                dma16(x + (size_t)m * K + (size_t)kbeg * 128 + c * 8, smem + m * xs_stride + ((c - lane) << 4));
        }
    }
    // two stages of D tiles (weights and scales) in flight behind the x loads
    if (ntile > 0) SVQ_LOAD(wA, sA, 0)
    if (ntile > D) SVQ_LOAD(wB, sB, D)
    {
        const int na = ntile < D ? ntile : D;
        const int nb2 = ntile - D < 0 ? 0 : (ntile - D < D ? ntile - D : D);
        wait_vmcnt_at_most<2 * D * (1 + NG)>((na + nb2) * (1 + NG));
    }
    // a bare barrier: __syncthreads() would also wait for the weight prefetch
    __builtin_amdgcn_s_barrier();

    // A operand of MFMA step j for tile i of the range: row min(r, M-1), 8 bf16
    // at K offset 32j + 8g (transposed words) or 32g + 8j
    const int arow = r < M ? r : M - 1;
    const uint8_t *abase = smem + arow * xs_stride + (kTrans ? 16 * g : 64 * g);
    constexpr int kXStep = kTrans ? 64 : 16;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#define SVQ_COMPUTE(W, SS, I0)                                                       \
    {                                                                                \
        uint32_t wj[D][4];                                                           \
        _Pragma("unroll") for (int d = 0; d < D; ++d) {                              \
            wj[d][0] = W[d].x; wj[d][1] = W[d].y; wj[d][2] = W[d].z; wj[d][3] = W[d].w; \
            if constexpr (kTrans) transpose_rows_words(wj[d][0], wj[d][1], wj[d][2], wj[d][3]); \
        }                                                                            \
        _Pragma("unroll") for (int d = 0; d < D; ++d) {                              \
            if ((I0) + d < ntile) {                                                  \
                const uint8_t *ap = abase + (wave + ((I0) + d) * WAVES) * 256;       \
                _Pragma("unroll") for (int q = 0; q < NG; ++q) {                     \
                    f32x4 P = {0.f, 0.f, 0.f, 0.f};                                  \
                    _Pragma("unroll") for (int jj = 0; jj < SPG; ++jj) {             \
                        const int j = q * SPG + jj;                                  \
                        const uint4 A = *(const uint4 *)(ap + j * kXStep);           \
                        P = mfma16x16x32(A, bneg, P);                                \
                        P = mfma16x16x32(A, word_to_bf16x8(wj[d][j]), P);            \
                    }                                                                \
                    const float sf = fp16_bits_to_f32((uint16_t)(SS[d][q] >> s_sh));           \
                    _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sf, P[i], acc[i]); \
                }                                                                    \
            }                                                                        \
        }                                                                            \
    }

    if (ntile > 0) {
        for (int i0 = 0;; i0 += 2 * D) {
            SVQ_COMPUTE(wA, sA, i0)
            if (i0 + D >= ntile) break;
            SVQ_LOAD(wA, sA, i0 + 2 * D)
            SVQ_COMPUTE(wB, sB, i0 + D)
            if (i0 + 2 * D >= ntile) break;
            SVQ_LOAD(wB, sB, i0 + 3 * D)
        }
    }
#undef SVQ_LOAD
#undef SVQ_COMPUTE

    // cross-wave sum of the valid rows through LDS (the x stage is dead now)
    __syncthreads();
    float *red = (float *)smem;  // [WAVES][M][16]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        if (row < M) red[(wave * M + row) * 16 + r] = acc[i];
    }
    __syncthreads();
    __shared__ int s_flag;
    float v = 0.f;
    if (threadIdx.x < 16 * M) {
        for (int w = 0; w < WAVES; ++w) v += red[w * M * 16 + threadIdx.x];
    }
    smallm_finish(v, M, N, nb, sp, splits, out, cnt, part, &s_flag);
}

// ---------------------------------------------------------------------------
// Wide kernel: any M (tuned for M = 128). Persistent stream-K: the grid has one
// workgroup per compute unit and each takes an equal contiguous share of the
// (output tile, 128-row K step) units. A tile computed by several workgroups is
// finished by the last to arrive, which adds the fp32 partials in workgroup
// order (fixed order: deterministic) and clears the tile's arrival counter.
//
// Per step, the workgroup stages the x tile (BM rows x 128, bf16) in LDS with
// -136 * (group sums of x) and the step's scales; each wave owns MBW 16-row
// blocks x CT 16-column weight tiles, streams its weight tiles with 128-bit
// loads one step ahead, and runs MBW*CT MFMA chains per group.
// ---------------------------------------------------------------------------
template <int MBW, int WR, int WC, int CT, int GSHIFT>
struct WideCfg {
    static constexpr int NT = 64 * WR * WC;
    static constexpr int BM = 16 * MBW * WR;
    static constexpr int BN = 16 * CT * WC;
    static constexpr int NG = 128 >> GSHIFT;
    static constexpr int SPG = 4 / NG;
    static constexpr bool kTrans = GSHIFT < 7;
    static constexpr int XROW = 128 + 8;        // bf16 per LDS row (16-byte pad)
    static constexpr int UPT = BM * 16 / NT;    // 16-byte x chunks staged per thread
    static constexpr int TPR = 16 / UPT;        // staging threads per x row
    static constexpr int SPT = (NG * BN + NT - 1) / NT;  // scales staged per thread
    static constexpr int NV = MBW * CT;         // f32x4 accumulators per lane
    static_assert(UPT == 4 || UPT == 8, "staging assumes 1 or 2 32-row blocks per thread");
};

template <int MBW, int WR, int WC, int CT, int GSHIFT>
__global__ __launch_bounds__(64 * WR * WC) void w4a16_wide_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    f32x4 *__restrict__ part, int M, int N, int K, int col_tiles, int64_t units, int grid,
    int maxt) {
    using C = WideCfg<MBW, WR, WC, CT, GSHIFT>;
    constexpr int NT = C::NT, BM = C::BM, BN = C::BN, NG = C::NG, SPG = C::SPG;
    constexpr int XROW = C::XROW, UPT = C::UPT, TPR = C::TPR, SPT = C::SPT, NV = C::NV;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][XROW];
    __shared__ __attribute__((aligned(16))) float xneg[2][NG][BM];
    __shared__ uint16_t sl[2][NG][BN];
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

        // this wave's weight tiles (clamped to a valid tile past the last column)
        const uint4 *tp[CT];
        bool ctv[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int nbg = cb * (BN / 16) + wc * CT + ct;
            ctv[ct] = nbg < NB16;
            tp[ct] = wt + (size_t)(ctv[ct] ? nbg : NB16 - 1) * KT * 64 + lane;
        }
        const bool srv = row0 + srow < M;
        const uint4 *xsrc = (const uint4 *)(x + (size_t)(srv ? row0 + srow : 0) * K) + sseg * UPT;

        f32x4 acc[NV];  // [rb * CT + ct]
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 xreg[UPT];
        uint16_t sreg[SPT];
        uint4 wcur[CT], wnext[CT];

        auto load_x = [&](int s) {
#pragma unroll
            for (int v = 0; v < UPT; ++v) xreg[v] = srv ? xsrc[(size_t)s * 16 + v] : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < SPT; ++v) {
                const int i = tid + v * NT;
                const int q = i / BN, c = i % BN;
                int colg = cb * BN + c;
                colg = colg < N ? colg : N - 1;
                sreg[v] = (i < NG * BN) ? sc[(size_t)(s * NG + q) * N + colg] : (uint16_t)0;
            }
        };
        auto load_w = [&](uint4(&W)[CT], int s) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) W[ct] = load_stream16(tp[ct] + (size_t)s * 64);
        };
        auto store_stage = [&](int buf) {
#pragma unroll
            for (int v = 0; v < UPT; ++v) *(uint4 *)&xs[buf][srow][(sseg * UPT + v) * 8] = xreg[v];
            float bsum[UPT / 4];
#pragma unroll
            for (int b = 0; b < UPT / 4; ++b) {
                float t = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 q4 = xreg[4 * b + v];
                    t = dot2_bf16(q4.x, kBf16OnePair, t);
                    t = dot2_bf16(q4.y, kBf16OnePair, t);
                    t = dot2_bf16(q4.z, kBf16OnePair, t);
                    t = dot2_bf16(q4.w, kBf16OnePair, t);
                }
                bsum[b] = t;
            }
            if constexpr (NG == 4) {  // G = 32: one group per 32-row block
#pragma unroll
                for (int b = 0; b < UPT / 4; ++b) xneg[buf][sseg * (UPT / 4) + b][srow] = -136.f * bsum[b];
            } else if constexpr (NG == 2) {  // G = 64
                if constexpr (UPT == 8) {
                    xneg[buf][sseg][srow] = -136.f * (bsum[0] + bsum[1]);
                } else {
                    const float v = bsum[0] + __shfl_xor(bsum[0], 1);
                    if ((sseg & 1) == 0) xneg[buf][sseg >> 1][srow] = -136.f * v;
                }
            } else {  // G = 128
                float v = bsum[0];
                if constexpr (UPT == 8) v += bsum[1];
                v += __shfl_xor(v, 1);
                if constexpr (TPR == 4) v += __shfl_xor(v, 2);
                if (sseg == 0) xneg[buf][0][srow] = -136.f * v;
            }
#pragma unroll
            for (int v = 0; v < SPT; ++v) {
                const int i = tid + v * NT;
                if (i < NG * BN) sl[buf][i / BN][i % BN] = sreg[v];
            }
        };
        auto compute = [&](int buf, const uint4(&W)[CT]) {
            uint32_t wj[CT][4];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                wj[ct][0] = W[ct].x;
                wj[ct][1] = W[ct].y;
                wj[ct][2] = W[ct].z;
                wj[ct][3] = W[ct].w;
                if constexpr (C::kTrans) transpose_rows_words(wj[ct][0], wj[ct][1], wj[ct][2], wj[ct][3]);
            }
            const int rbase = wr * MBW * 16;
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                f32x4 P[MBW][CT];
#pragma unroll
                for (int rb = 0; rb < MBW; ++rb) {
                    const f32x4 c = *(const f32x4 *)&xneg[buf][q][rbase + rb * 16 + 4 * g];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) P[rb][ct] = c;
                }
#pragma unroll
                for (int jj = 0; jj < SPG; ++jj) {
                    const int j = q * SPG + jj;
                    const int koff = C::kTrans ? (32 * j + 8 * g) : (32 * g + 8 * j);
                    uint4 A[MBW];
#pragma unroll
                    for (int rb = 0; rb < MBW; ++rb) A[rb] = *(const uint4 *)&xs[buf][rbase + rb * 16 + r][koff];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const uint4 B = word_to_bf16x8(wj[ct][j]);
#pragma unroll
                        for (int rb = 0; rb < MBW; ++rb) P[rb][ct] = mfma16x16x32(A[rb], B, P[rb][ct]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const float sf = fp16_bits_to_f32(sl[buf][q][wc * CT * 16 + ct * 16 + r]);
#pragma unroll
                    for (int rb = 0; rb < MBW; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[rb * CT + ct][i] = __builtin_fmaf(sf, P[rb][ct][i], acc[rb * CT + ct][i]);
                }
            }
        };

        __syncthreads();  // LDS of a previous segment is no longer read
        load_x(s0);
        load_w(wcur, s0);
        for (int s = s0; s < s1; ++s) {
            const int buf = (s - s0) & 1;
            store_stage(buf);
            __syncthreads();
            if (s + 1 < s1) {
                load_x(s + 1);
                load_w(wnext, s + 1);
            }
            compute(buf, wcur);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) wcur[ct] = wnext[ct];
        }

        // ---- epilogue ----
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
constexpr int kSkinnyDepth = 2;

template <int WAVES, int GS>
hipError_t skinny_launch_w(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                           int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    hipLaunchKernelGGL((w4a16_skinny_kernel<WAVES, kSkinnyDepth, GS>),
                       dim3((uint32_t)(N / 16 * p.splits)), dim3(64 * WAVES),
                       skinny_lds_bytes(M, p.S, WAVES), stream,
                       (const uint16_t *)x, (const uint4 *)wt, (const uint16_t *)sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), M, (int)N, (int)K, p.splits, p.S);
    return hipGetLastError();
}

template <int GS>
hipError_t skinny_launch(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                         int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    static const int r16 = resident_blocks(w4a16_skinny_kernel<16, kSkinnyDepth, GS>, 1024);
    static const int r8 = resident_blocks(w4a16_skinny_kernel<8, kSkinnyDepth, GS>, 512);
    const int by_lds = (int)(kLdsPerCu / skinny_lds_bytes(M, p.S, 16));
    switch (pick_waves(N / 16 * p.splits, p.cus, std::min(r16, by_lds), std::min(r8, by_lds))) {
    case 16: return skinny_launch_w<16, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    case 8: return skinny_launch_w<8, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    default: return skinny_launch_w<4, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    }
}

template <int MBW, int WR, int WC, int CT, int GS>
hipError_t wide_launch(const WidePlan &p, const void *x, const int32_t *wt, const void *sc,
                       void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    uint32_t *cnt = ws_counters(ws);
    f32x4 *part = (f32x4 *)ws_partials(ws);
    hipLaunchKernelGGL((w4a16_wide_kernel<MBW, WR, WC, CT, GS>), dim3((uint32_t)p.grid),
                       dim3(64 * WR * WC), 0, stream, (const uint16_t *)x, (const uint4 *)wt,
                       (const uint16_t *)sc, (uint16_t *)out, cnt, part, (int)M, (int)N, (int)K,
                       p.col_tiles, p.units, p.grid, p.maxt);
    return hipGetLastError();
}

template <int GS>
hipError_t wide_by_shape(const WidePlan &p, const void *x, const int32_t *wt, const void *sc,
                         void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    if (p.bm == 128) return wide_launch<4, 2, 2, 4, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    return wide_launch<4, 1, 4, 4, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
}
}  // namespace

hipError_t launch_w4a16_skinny(const SmallPlan &plan, const void *x, const int32_t *wt,
                               const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                               void *workspace, hipStream_t stream) {
    switch (G) {
    case 32: return skinny_launch<5>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    case 64: return skinny_launch<6>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    case 128: return skinny_launch<7>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_w4a16_wide(const WidePlan &plan, const void *x, const int32_t *wt,
                             const void *scales, void *out, int64_t M, int64_t N, int64_t K,
                             int G, void *workspace, hipStream_t stream) {
    switch (G) {
    case 32: return wide_by_shape<5>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    case 64: return wide_by_shape<6>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    case 128: return wide_by_shape<7>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace svq
