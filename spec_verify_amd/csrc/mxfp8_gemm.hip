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
template <int M, int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_dot2_kernel(
    const uint32_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int N, int K, int splits, int S) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int r = lane & 15, rg = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int nb = lb / splits, sp = lb % splits;
    const int KT = K >> 7;
    // this block's 16 weight rows ([N][K] layout) and their scale rows
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + (size_t)nb * 16 * K, (uint32_t)16 * K);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * K * 2);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + (size_t)nb * 16 * (K >> 5), (uint32_t)16 * (K >> 5));
    const uint32_t w_vo = r * K + rg * 32;
    const uint32_t x_vo = lane * 4;
    // the dword holding the tile's four block scales; s_sh selects this lane's
    const uint32_t s_vo = r * (K >> 5);
    const int s_sh = rg * 8;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = wave < kcnt ? (kcnt - 1 - wave) / WAVES + 1 : 0;

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = 0.f;
    uint4 vA[D][2], vB[D][2];
    uint32_t xA[D][M], xB[D][M], sA[D], sB[D];

#define SVQ_LOAD(V, X, S, I0)                                                        \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wave + ((I0) + d) * WAVES;                                    \
        V[d][0] = bload16(wr, w_vo, kt * 128);                                       \
        V[d][1] = bload16(wr, w_vo + 16, kt * 128);                                  \
        _Pragma("unroll") for (int m = 0; m < M; ++m) X[d][m] = bload4(xr, x_vo, m * K * 2 + kt * 256); \
        S[d] = bload4(sr, s_vo, kt * 4);                                             \
    }
#define SVQ_COMPUTE(V, X, S, I0)                                                     \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const float sf = e8m0_to_f32((uint8_t)(S[d] >> s_sh));                                          \
        const uint32_t wd[8] = {V[d][0].x, V[d][0].y, V[d][0].z, V[d][0].w,          \
                                V[d][1].x, V[d][1].y, V[d][1].z, V[d][1].w};         \
        mxfp8_tile_dots<M>(acc, X[d], wd, sf);                                       \
    }

    if (ntile > 0) {
        SVQ_LOAD(vA, xA, sA, 0)
        for (int i0 = 0;; i0 += 2 * D) {
            SVQ_LOAD(vB, xB, sB, i0 + D)
            SVQ_COMPUTE(vA, xA, sA, i0)
            if (i0 + D >= ntile) break;
            SVQ_LOAD(vA, xA, sA, i0 + 2 * D)
            SVQ_COMPUTE(vB, xB, sB, i0 + D)
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
        for (int wv = 0; wv < WAVES; ++wv) v += red[wv][threadIdx.x >> 4][threadIdx.x & 15];
    }
    smallm_finish(v, M, N, nb, sp, splits, out, cnt, part, &s_flag);
}

// ---------------------------------------------------------------------------
// skinny MFMA kernel, M <= 16: a workgroup owns one 16-column block and a
// range of S K-tiles; its x rows are staged once in LDS (so the vector-memory
// path carries only weights and scales: staging cut M = 5, K = N = 5120 from
// 13.6 to 11.5 us against x loaded per tile from L2), and each tile is four
// MFMAs on weights converted with the block scale applied.
// ---------------------------------------------------------------------------
template <int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void mxfp8_skinny_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int M, int N, int K, int splits, int S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int nb = lb / splits, sp = lb % splits;
    const int KT = K >> 7;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + (size_t)nb * 16 * K, (uint32_t)16 * K);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + (size_t)nb * 16 * (K >> 5), (uint32_t)16 * (K >> 5));
    const uint32_t w_vo = r * K + g * 32;
    // the dword holding the tile's four block scales; s_sh selects this lane's
    const uint32_t s_vo = r * (K >> 5);
    const int s_sh = g * 8;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = wave < kcnt ? (kcnt - 1 - wave) / WAVES + 1 : 0;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    uint4 vA[D][2], vB[D][2];
    uint32_t sA[D], sB[D];

#define SVQ_LOAD(V, S, I0)                                                           \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wave + ((I0) + d) * WAVES;                             \
        V[d][0] = bload16(wr, w_vo, kt * 128);                                       \
        V[d][1] = bload16(wr, w_vo + 16, kt * 128);                                  \
        S[d] = bload4(sr, s_vo, kt * 4);                                             \
    }
    // stage x[0..M)[128*kbeg, 128*(kbeg+kcnt)) in LDS by DMA (one 64-chunk
    // segment of a row per instruction), rows padded by 16 bytes so that the
    // 16-byte A reads of different rows fall in different banks; the weight
    // prefetch is issued behind it and only the x loads are waited for
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
    if (ntile > 0) SVQ_LOAD(vA, sA, 0)
    if (ntile > D) SVQ_LOAD(vB, sB, D)
    {
        const int na = ntile < D ? ntile : D;
        const int nb2 = ntile - D < 0 ? 0 : (ntile - D < D ? ntile - D : D);
        wait_vmcnt_at_most<6 * D>((na + nb2) * 3);
    }
    // a bare barrier: __syncthreads() would also wait for the weight prefetch
    __builtin_amdgcn_s_barrier();
    // A operand of step j of tile i: row min(r, M-1) (rows past M repeat the
    // last row; their products are never stored), K-rows 32g + 8j..
    const int arow = r < M ? r : M - 1;
    const uint8_t *abase = smem + arow * xs_stride + 64 * g;

#define SVQ_COMPUTE(V, S, I0)                                                        \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const uint8_t *ap = abase + (wave + ((I0) + d) * WAVES) * 256;               \
        const float sf = e8m0_to_f32((uint8_t)(S[d] >> s_sh));                      \
        acc = mfma16x16x32(*(const uint4 *)(ap), cvt8_e4m3_bf16(V[d][0].x, V[d][0].y, sf), acc);      \
        acc = mfma16x16x32(*(const uint4 *)(ap + 16), cvt8_e4m3_bf16(V[d][0].z, V[d][0].w, sf), acc); \
        acc = mfma16x16x32(*(const uint4 *)(ap + 32), cvt8_e4m3_bf16(V[d][1].x, V[d][1].y, sf), acc); \
        acc = mfma16x16x32(*(const uint4 *)(ap + 48), cvt8_e4m3_bf16(V[d][1].z, V[d][1].w, sf), acc); \
    }

    if (ntile > 0) {
        for (int i0 = 0;; i0 += 2 * D) {
            SVQ_COMPUTE(vA, sA, i0)
            if (i0 + D >= ntile) break;
            SVQ_LOAD(vA, sA, i0 + 2 * D)
            SVQ_COMPUTE(vB, sB, i0 + D)
            if (i0 + 2 * D >= ntile) break;
            SVQ_LOAD(vB, sB, i0 + 3 * D)
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
        for (int wv = 0; wv < WAVES; ++wv) v += red[wv * M * 16 + threadIdx.x];
    }
    smallm_finish(v, M, N, nb, sp, splits, out, cnt, part, &s_flag);
}

// ---------------------------------------------------------------------------
// wide stream-K MFMA kernel, any M
// ---------------------------------------------------------------------------
template <int MBW, int WR, int WC, int CT>
__global__ __launch_bounds__(64 * WR * WC) void mxfp8_wide_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    f32x4 *__restrict__ part, int M, int N, int K, int col_tiles, int64_t units, int grid,
    int maxt, SkWait skw) {
    constexpr int NT = 64 * WR * WC;
    constexpr int BM = 16 * MBW * WR;
    constexpr int BN = 16 * CT * WC;
    constexpr int XROW = 128 + 8;
    // x stage: 16 lanes per row (16 chunks of 16 bytes = one step of a row),
    // NT / 16 rows per pass, UPT passes
    constexpr int RPP = NT / 16;
    constexpr int UPT = BM / RPP;
    static_assert(UPT * RPP == BM, "x stage split over the threads");
    constexpr int NV = MBW * CT;
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM][XROW];
    __shared__ int s_sk[3];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC;
    const int r = lane & 15, g = lane >> 4;
    const int KT = K >> 7;
    const int NB16 = N >> 4;
    const int wg = blockIdx.x;
    const int64_t u_begin = (int64_t)wg * units / grid;
    const int64_t u_end = (int64_t)(wg + 1) * units / grid;
    const int srow = tid >> 4, schunk = tid & 15;

    // Buffer views: a per-lane offset past the end reads zeros without touching
    // memory, which turns rows >= M and the prefetch after a segment's last step
    // into loads that need no branch (a conditional load would make the
    // compiler wait for every load in flight before the next compute).
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
    const __amdgpu_buffer_rsrc_t wrs = make_rsrc(w, (uint32_t)((size_t)N * K));
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(sc, (uint32_t)((size_t)N * (K >> 5)));
    constexpr uint32_t kOob = 0x80000000u;

    for (int64_t u = u_begin; u < u_end;) {
        const int tile = (int)(u / KT);
        const int s0 = (int)(u % KT);
        const int s1 = (int)((u_end - u) < (int64_t)(KT - s0) ? s0 + (u_end - u) : KT);
        const int rt = tile / col_tiles, cb = tile % col_tiles;
        const int row0 = rt * BM;

        // lane (r, g) of column tile ct: column colg, K-rows 32g.. of each step
        // (one 32-element scale block); the step's four block scales of the
        // column are one aligned dword, byte g is this lane's
        uint32_t wvo[CT], svo[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int nbg = cb * (BN / 16) + wc * CT + ct;
            const int colg = (nbg < NB16 ? nbg : NB16 - 1) * 16 + r;
            wvo[ct] = (uint32_t)colg * (uint32_t)K + g * 32;
            svo[ct] = (uint32_t)colg * (uint32_t)(K >> 5);
        }
        // rows past M read row M - 1 (their products are never stored)
        uint32_t xvo[UPT];
#pragma unroll
        for (int v = 0; v < UPT; ++v) {
            const int row = row0 + srow + RPP * v;
            xvo[v] = (uint32_t)(row < M ? row : M - 1) * (uint32_t)K * 2u + schunk * 16;
        }
        // kOob for a step past the segment (operands stay below 2^31 bytes)
        auto past = [&](int s) { return (uint32_t)(s1 - 1 - s) & kOob; };

        f32x4 acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

        uint4 xreg[UPT];
        uint4 wcur[CT][2], wnext[CT][2];
        uint32_t scur[CT], snext[CT];

        // loads of K step s (s >= s1: out of range, zeros, no traffic)
        // (the out-of-range bit is formed arithmetically: a select on the
        // wave-uniform condition would become a branch around the loads)
        // A step's loads are issued in one fixed order, x then weights and
        // scales, fenced from the surrounding code: the s_waitcnt counts then
        // agree on every path into the loop. The empty asm with a memory
        // clobber keeps the optimizer from sinking the loads below the next
        // compute phase (it emits no instruction and no wait).
        auto load_step = [&](uint4(&W)[CT][2], uint32_t(&S)[CT], int s) {
            const uint32_t o = past(s);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < UPT; ++v) xreg[v] = bload16(xr, (xvo[v] + (uint32_t)s * 256u) | o, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const uint32_t vo = (wvo[ct] + (uint32_t)s * 128u) | o;
                W[ct][0] = bload16(wrs, vo, 0);
                W[ct][1] = bload16(wrs, vo + 16, 0);
                S[ct] = bload4(srs, (svo[ct] + (uint32_t)s * 4u) | o, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
        };
        auto compute = [&](int buf, const uint4 (&W)[CT][2], const uint32_t (&S)[CT]) {
            const int rbase = wr * MBW * 16;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint4 A[MBW];
#pragma unroll
                for (int rb = 0; rb < MBW; ++rb) A[rb] = *(const uint4 *)&xs[buf][rbase + rb * 16 + r][32 * g + 8 * j];
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const float sf = e8m0_to_f32((S[ct] >> (8 * g)) & 0xFFu);
                    const uint4 &wv = W[ct][j >> 1];
                    const uint4 B = (j & 1) ? cvt8_e4m3_bf16(wv.z, wv.w, sf) : cvt8_e4m3_bf16(wv.x, wv.y, sf);
#pragma unroll
                    for (int rb = 0; rb < MBW; ++rb) acc[rb * CT + ct] = mfma16x16x32(A[rb], B, acc[rb * CT + ct]);
                }
            }
        };
        auto stage_x = [&](int buf) {
#pragma unroll
            for (int v = 0; v < UPT; ++v) *(uint4 *)&xs[buf][srow + RPP * v][schunk * 8] = xreg[v];
        };

        // Two register sets for the weights and scales, used alternately, so
        // that the compute of a step never reads registers that the next
        // step's loads are still filling (a copy between the sets would make
        // every step wait for the next step's loads).
        // Steps go in pairs; every half issues its prefetch (past the segment
        // it reads zeros), and only the compute of a missing second step is
        // skipped, so no load sits behind a branch.
        __syncthreads();
        load_step(wcur, scur, s0);
        for (int s = s0; s < s1; s += 2) {
            stage_x(0);
            __syncthreads();
            load_step(wnext, snext, s + 1);
            compute(0, wcur, scur);
            stage_x(1);
            __syncthreads();
            load_step(wcur, scur, s + 2);
            if (s + 1 < s1) compute(1, wnext, snext);
        }

        const int rowb = row0 + wr * MBW * 16 + 4 * g;
        // accumulator v = (row block v / CT, column tile v % CT) of this thread
        auto store_v = [&](int v, const f32x4 &val) {
            const int rb = v / CT, ct = v % CT;
            const int nbg = cb * (BN / 16) + wc * CT + ct;
            if (nbg >= NB16) return;
            const int colg = nbg * 16 + r;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = rowb + rb * 16 + i;
                if (row < M) out[(size_t)row * N + colg] = f32_to_bf16_rne(val[i]);
            }
        };
        if (s0 == 0 && s1 == KT) {
#pragma unroll
            for (int v = 0; v < NV; ++v) store_v(v, acc[v]);
        } else {
            sk_reduce<NV, NT>(acc, tile, KT, units, grid, maxt, cnt, part, s_sk, skw, store_v);
        }
        u += s1 - s0;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
// two tiles per prefetch stage: the registers then allow two 16-wave
// workgroups per CU (four tiles per stage: one), measured faster at M = 1
// (10.5 against 10.8 us, K = N = 5120) and M = 5 (13.0 against 14.5 us)
constexpr int kMxDot2Depth = 2;
constexpr int kMxSkinnyDepth = 2;

template <int M, int WAVES>
hipError_t mx_dot2_launch_w(const SmallPlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                            void *out, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    return launch_gemm(mxfp8_dot2_kernel<M, WAVES, kMxDot2Depth>, dim3((uint32_t)(N / 16 * p.splits)),
                       dim3(64 * WAVES), 0, stream, (const uint32_t *)x, w, sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), (int)N, (int)K, p.splits, p.S);
}

template <int M>
hipError_t mx_dot2_launch(const SmallPlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                          void *out, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    static const int r16 = resident_blocks(mxfp8_dot2_kernel<M, 16, kMxDot2Depth>, 1024);
    static const int r8 = resident_blocks(mxfp8_dot2_kernel<M, 8, kMxDot2Depth>, 512);
    switch (pick_waves(N / 16 * p.splits, p.cus, r16, r8)) {
    case 16: return mx_dot2_launch_w<M, 16>(p, x, w, sc, out, N, K, ws, stream);
    case 8: return mx_dot2_launch_w<M, 8>(p, x, w, sc, out, N, K, ws, stream);
    default: return mx_dot2_launch_w<M, 4>(p, x, w, sc, out, N, K, ws, stream);
    }
}

template <int WAVES>
hipError_t mx_skinny_launch_w(const SmallPlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                              void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    return launch_gemm(mxfp8_skinny_kernel<WAVES, kMxSkinnyDepth>, dim3((uint32_t)(N / 16 * p.splits)),
                       dim3(64 * WAVES), skinny_lds_bytes(M, p.S, WAVES), stream, (const uint16_t *)x, w, sc,
                       (uint16_t *)out, ws_counters(ws), (float *)ws_partials(ws), M, (int)N,
                       (int)K, p.splits, p.S);
}

template <int MBW, int WR, int WC, int CT>
hipError_t mx_wide_launch(const WidePlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                          void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    uint32_t *cnt = ws_counters(ws);
    f32x4 *part = (f32x4 *)ws_partials(ws);
    return launch_gemm(mxfp8_wide_kernel<MBW, WR, WC, CT>, dim3((uint32_t)p.grid),
                       dim3(64 * WR * WC), 0, stream, (const uint16_t *)x, w, sc, (uint16_t *)out,
                       cnt, part, (int)M, (int)N, (int)K, p.col_tiles, p.units, p.grid, p.maxt, SkWait{p.wait_arrive, p.wait_range});
}
}  // namespace

hipError_t launch_mxfp8_dot2(const SmallPlan &plan, const void *x, const uint8_t *w,
                             const uint8_t *scales, void *out, int M, int64_t N, int64_t K,
                             void *ws, hipStream_t stream) {
    switch (M) {
    case 1: return mx_dot2_launch<1>(plan, x, w, scales, out, N, K, ws, stream);
    case 2: return mx_dot2_launch<2>(plan, x, w, scales, out, N, K, ws, stream);
    case 3: return mx_dot2_launch<3>(plan, x, w, scales, out, N, K, ws, stream);
    case 4: return mx_dot2_launch<4>(plan, x, w, scales, out, N, K, ws, stream);
    case 5: return mx_dot2_launch<5>(plan, x, w, scales, out, N, K, ws, stream);
    case 6: return mx_dot2_launch<6>(plan, x, w, scales, out, N, K, ws, stream);
    case 7: return mx_dot2_launch<7>(plan, x, w, scales, out, N, K, ws, stream);
    case 8: return mx_dot2_launch<8>(plan, x, w, scales, out, N, K, ws, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mxfp8_skinny(const SmallPlan &plan, const void *x, const uint8_t *w,
                               const uint8_t *scales, void *out, int M, int64_t N, int64_t K,
                               void *ws, hipStream_t stream) {
    static const int r16 = resident_blocks(mxfp8_skinny_kernel<16, kMxSkinnyDepth>, 1024);
    static const int r8 = resident_blocks(mxfp8_skinny_kernel<8, kMxSkinnyDepth>, 512);
    const int by_lds = (int)(kLdsPerCu / skinny_lds_bytes(M, plan.S, 16));
    switch (pick_waves(N / 16 * plan.splits, plan.cus, std::min(r16, by_lds), std::min(r8, by_lds))) {
    case 16: return mx_skinny_launch_w<16>(plan, x, w, scales, out, M, N, K, ws, stream);
    case 8: return mx_skinny_launch_w<8>(plan, x, w, scales, out, M, N, K, ws, stream);
    default: return mx_skinny_launch_w<4>(plan, x, w, scales, out, M, N, K, ws, stream);
    }
}

hipError_t launch_mxfp8_wide(const WidePlan &plan, const void *x, const uint8_t *w,
                             const uint8_t *scales, void *out, int64_t M, int64_t N, int64_t K,
                             void *workspace, hipStream_t stream) {
    // 128 x 128 tiles: four waves side by side (each all 128 rows x 32 columns),
    // so every weight byte is loaded and converted by one wave only
    if (plan.bm == 128) return mx_wide_launch<8, 1, 4, 2>(plan, x, w, scales, out, M, N, K, workspace, stream);
    return mx_wide_launch<4, 1, 4, 4>(plan, x, w, scales, out, M, N, K, workspace, stream);
}

}  // namespace svq
