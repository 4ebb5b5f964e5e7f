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
// Weights are read from the device tile layout written once at setup by
// mxfp8_tile_kernel: tiles of 16 columns x 128 K-elements (2 KiB), column-block-
// major with the K-tiles of a block consecutive, byte 1024*h + 16*l + b of a
// tile holding column 16*nb + l%16, K-element 128*kt + 32*(l/16) + 16*h + b. So
// lane l of a wave owns column l%16 and the 32 consecutive K-rows 32*(l/16)..
// (one 32-element scale block) and reads them with two 128-bit loads, each of
// which is a contiguous 1 KiB for the wave (the untouched [N][K] rows put each
// lane's bytes K apart: a plain stream in that pattern measured 7.42 us against
// 6.41 us for the same 26 MB in tiles, at N = K = 5120 in the M = 1 launch shape).
// The three kernels mirror the W4A16 ones: a VALU dot2 kernel
// with a row broadcast of x for M <= 8, a one-MFMA-tile kernel for M <= 16, and
// the split-K MFMA kernel with LDS-staged x for larger M (shared tiles'
// partials summed by a second launch).
#include "svq_dma.h"
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
    // this block's tiles (2 KiB per K-tile, consecutive) and its 16 scale rows
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + (size_t)nb * 16 * K, (uint32_t)16 * K);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)M * K * 2);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + (size_t)nb * 16 * (K >> 5), (uint32_t)16 * (K >> 5));
    const uint32_t w_vo = lane * 16;
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
        V[d][0] = bload16(wr, w_vo, kt * 2048);                                      \
        V[d][1] = bload16(wr, w_vo + 1024, kt * 2048);                               \
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
    const uint32_t w_vo = lane * 16;
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
        V[d][0] = bload16(wr, w_vo, kt * 2048);                                      \
        V[d][1] = bload16(wr, w_vo + 1024, kt * 2048);                               \
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
// wide MFMA kernel, M > 16 (any M). Output tiles of BM x 128 (BM = 32, 64 or
// 128 by M); with fewer tiles than CUs each tile's K range is split evenly over
// floor(CUs / tiles) workgroups, otherwise the (tile, K step) units are split
// evenly over one workgroup per CU (stream-K). A tile computed whole by one
// workgroup is written as bf16 directly; a shared tile's fp32 partials are
// written with plain stores to the workspace and summed, in contributor order,
// by a second launch (wide_sum_kernel): the launch boundary orders the
// partials' stores before their loads, so no workgroup waits for another, and
// no coherent (cache-bypassing) memory traffic is needed. Measured on the
// MI355X at M = 128, K = N = 5120 (40 tiles x 6 K ranges): 27.2 us with the
// partials reduced inside the kernel through coherent stores, arrival counters
// and bounded waits (about 14 us of it after the K loop), 20.8 us with the
// second launch.
//
// Workgroup: 8 waves as 2 row halves x 4 column quarters; a wave owns MBW
// 16-row blocks x 2 16-column tiles (16x16x32 bf16 MFMA). Every K step of 128
// is staged in one slot of a three-slot LDS ring by LDS-DMA (buffer loads that
// write LDS directly; rows past M and columns past N read as zero): x (BM rows,
// 16-byte chunks XOR-swizzled by row so that the A reads are bank-conflict
// free), the E4M3 codes of the tile's 128 columns (eight 2 KiB weight tiles)
// and their E8M0 scales. The
// ring runs two steps ahead of the MFMAs; one barrier per step frees the slot
// the next DMAs go to. Lane (r, g) of a column tile converts the 32 codes of
// its column at K 32g.. (one E8M0 block) with the block scale applied in the
// conversion, and MFMA step j takes bytes 8j.. of them against x at the same K.
// ---------------------------------------------------------------------------
template <int MBW>
struct MxWideCfg {
    static constexpr int WR = 2, WC = 4, WAVES = WR * WC, NT = 64 * WAVES, CT = 2;
    static constexpr int BM = 16 * MBW * WR;
    static constexpr int BN = 16 * CT * WC;       // 128 columns
    static constexpr int NV = MBW * CT;           // f32x4 accumulators per lane
    static constexpr int XB = BM * 256;           // x: BM rows x 128 K, bf16
    static constexpr int WB = BN * 128;           // E4M3 codes: BN columns x 128 K
    static constexpr int SB = BN * 4;             // E8M0: BN columns x 4 blocks
    static constexpr int OFF_W = XB, OFF_S = XB + WB, SLOT = XB + WB + SB;
    static constexpr int XI = XB / 1024 / WAVES;  // x DMAs (1 KiB each) per wave per step
    static constexpr int WI = WB / 1024 / WAVES;  // code DMAs per wave per step
    static constexpr int SI = SB / 256;           // scale DMAs per step (waves 0 .. SI-1)
    static constexpr int MAXPS = XI + WI + 1;     // most DMAs one wave issues per step
    static_assert(XI >= 1 && XI * 1024 * WAVES == XB, "x stage split over the waves");
    static_assert(WI * 1024 * WAVES == WB && SI <= WAVES, "code and scale stages split over the waves");
    static_assert(SLOT % 16 == 0 && 3 * SLOT <= 160 * 1024, "three slots fit the LDS");
};

template <int MBW>
__global__ __launch_bounds__(512) void mxfp8_wide_kernel(
    const uint16_t *__restrict__ x, const uint8_t *__restrict__ w,
    const uint8_t *__restrict__ sc, uint16_t *__restrict__ out, f32x4 *__restrict__ part,
    int M, int N, int K, int col_tiles, int64_t units, int grid, int maxt) {
    using C = MxWideCfg<MBW>;
    constexpr int BM = C::BM, BN = C::BN, NV = C::NV, CT = C::CT;
    __shared__ __attribute__((aligned(16))) uint8_t ring[3 * C::SLOT];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wr = wave / C::WC, wc = wave % C::WC;
    const int r = lane & 15, g = lane >> 4;
    const int KT = K >> 7;
    const int NB16 = N >> 4;
    const int wg = blockIdx.x;
    const int64_t u_begin = (int64_t)wg * units / grid;
    const int64_t u_end = (int64_t)(wg + 1) * units / grid;
    const uint32_t ring_lds = lds_addr(ring);
    // buffer views: reads past the end return zero (rows >= M, columns >= N)
    const BufDesc xr = buf_desc(x, (uint32_t)((size_t)M * K * 2));
    const BufDesc wrs = buf_desc(w, (uint32_t)((size_t)N * K));
    const BufDesc srs = buf_desc(sc, (uint32_t)((size_t)N * (K >> 5)));

    // per-lane LDS offsets within a slot
    uint32_t offA[4];  // A of MFMA step j: row r of the wave's first row block, K 32g + 8j..
#pragma unroll
    for (int j = 0; j < 4; ++j) offA[j] = wr * MBW * 4096 + r * 256 + (((4 * g + j) ^ r) << 4);
    // codes of column (wc*CT + ct)*16 + r at K 32g.. (the two halves of a
    // staged tile, lane 16g + r of each), and its scale dword
    uint32_t offB[CT], offS[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int cb16 = wc * CT + ct;
        offB[ct] = C::OFF_W + cb16 * 2048 + (16 * g + r) * 16;
        offS[ct] = C::OFF_S + (cb16 * 16 + r) * 4;
    }
    const int per_step = C::XI + C::WI + (wave < C::SI ? 1 : 0);  // this wave's DMAs per stage

    struct Seg {
        int tile, s0, n, rt, cb;
    };
    auto seg_at = [&](int64_t u) {
        Seg sg;
        sg.tile = (int)(u / KT);
        sg.s0 = (int)(u % KT);
        sg.n = (int)((u_end - u) < (int64_t)(KT - sg.s0) ? (u_end - u) : (KT - sg.s0));
        sg.rt = sg.tile / col_tiles;
        sg.cb = sg.tile % col_tiles;
        return sg;
    };
    // DMA of K step kt of segment sg into slot st: x (1 KiB = 4 rows per
    // instruction), codes (one 1 KiB half-tile per instruction), scales (64
    // columns x 4 blocks per instruction)
    auto issue = [&](const Seg &sg, int st, int kt) {
        const uint32_t base = ring_lds + st * C::SLOT;
#pragma unroll
        for (int v = 0; v < C::XI; ++v) {
            const int q = wave * C::XI + v;
            const int rl = 4 * q + (lane >> 4);
            const uint32_t vx = (uint32_t)(sg.rt * BM + rl) * (uint32_t)K * 2u + (uint32_t)(((lane & 15) ^ (rl & 15)) * 16);
            dma_b128(xr, base + q * 1024, vx, (uint32_t)kt * 256u);
        }
#pragma unroll
        for (int v = 0; v < C::WI; ++v) {
            const int t = wave * C::WI + v;  // column block t/2 of the tile, half t%2
            const uint32_t blk = (uint32_t)(sg.cb * (BN / 16) + (t >> 1));  // blocks past N read as zero
            dma_b128(wrs, base + C::OFF_W + t * 1024, (blk * (uint32_t)KT * 2048u) + (uint32_t)((t & 1) * 1024 + lane * 16),
                     (uint32_t)kt * 2048u);
        }
        if (wave < C::SI) {
            const uint32_t col = (uint32_t)(sg.cb * BN + wave * 64 + lane);
            dma_b32(srs, base + C::OFF_S + wave * 256, col * (uint32_t)(K >> 5), (uint32_t)kt * 4u);
        }
    };
    auto compute = [&](int st, f32x4 (&acc)[NV]) {
        const lds_u8 *b = lds_opaque(ring_lds + st * C::SLOT);
        uint4 wv[CT][2];
        float sf[CT];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            wv[ct][0] = lds_ld16(b + offB[ct]);
            wv[ct][1] = lds_ld16(b + offB[ct] + 1024);
            sf[ct] = e8m0_to_f32((lds_ld<uint32_t>(b + offS[ct]) >> (8 * g)) & 0xFFu);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 A[MBW];
#pragma unroll
            for (int rb = 0; rb < MBW; ++rb) A[rb] = lds_ld16(b + offA[j] + rb * 4096);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const uint4 &q = wv[ct][j >> 1];
                const uint4 B = (j & 1) ? cvt8_e4m3_bf16(q.z, q.w, sf[ct]) : cvt8_e4m3_bf16(q.x, q.y, sf[ct]);
#pragma unroll
                for (int rb = 0; rb < MBW; ++rb) acc[rb * CT + ct] = mfma16x16x32(A[rb], B, acc[rb * CT + ct]);
            }
        }
    };

    // Segments (runs of K steps of one tile) one after another; each runs the
    // ring from its start: two stages issued, then per step a wait for this
    // wave's stage, a barrier, the DMA of the stage two steps ahead and the
    // step's MFMAs. (With fewer tiles than CUs every workgroup has one segment.)
    for (int64_t u = u_begin; u < u_end;) {
        const Seg sg = seg_at(u);
        const int n = sg.n;
        f32x4 acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
        lds_barrier();  // the previous segment is done with every slot
        issue(sg, 0, sg.s0);
        if (n > 1) issue(sg, 1, sg.s0 + 1);
        for (int i = 0; i < n; ++i) {
            // this wave's stage of step i has landed (only step i+1's may be outstanding)
            if (i + 1 < n) wait_vmcnt_at_most<C::MAXPS>(per_step);
            else wait_vmcnt<0>();
            lds_barrier();  // every wave's stage of step i is in; every wave is done with step i-1
            if (i + 2 < n) issue(sg, (i + 2) % 3, sg.s0 + i + 2);
            compute(i % 3, acc);
        }
        if (sg.s0 == 0 && n == KT) {
            // the whole tile: bf16 straight to y
            const int rowb = sg.rt * BM + wr * MBW * 16 + 4 * g;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int rb = v / CT, ct = v % CT;
                const int nbg = sg.cb * (BN / 16) + wc * CT + ct;
                if (nbg >= NB16) continue;
                const int colg = nbg * 16 + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = rowb + rb * 16 + i;
                    if (row < M) out[(size_t)row * N + colg] = f32_to_bf16_rne(acc[v][i]);
                }
            }
        } else {
            // a K range of a shared tile: the fp32 partial, summed by wide_sum_kernel
            f32x4 *mp = wide_partial<NV, C::NT>(part, wg, maxt, sg.tile - sk_first_tile(wg, units, grid, KT));
#pragma unroll
            for (int v = 0; v < NV; ++v) mp[v * C::NT + threadIdx.x] = acc[v];
        }
        u += n;
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

template <int MBW>
hipError_t mx_wide_launch(const WidePlan &p, const void *x, const uint8_t *w, const uint8_t *sc,
                          void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    using C = MxWideCfg<MBW>;
    f32x4 *part = (f32x4 *)ws_partials(ws);
    hipError_t e = launch_gemm(mxfp8_wide_kernel<MBW>, dim3((uint32_t)p.grid), dim3(C::NT), 0, stream,
                               (const uint16_t *)x, w, sc, (uint16_t *)out, part, (int)M, (int)N, (int)K,
                               p.col_tiles, p.units, p.grid, p.maxt);
    if (e != hipSuccess || !p.workspace_bytes) return e;
    // shared tiles: the partials' sum, one workgroup per (tile, accumulator pair)
    return launch_gemm(wide_sum_kernel<MBW, C::WR, C::WC, C::CT, C::BM, C::BN>,
                       dim3((uint32_t)((int64_t)p.row_tiles * p.col_tiles * C::NV / 2)), dim3(C::NT), 0, stream,
                       (const f32x4 *)part, (uint16_t *)out, (int)M, (int)N, (int)K, p.col_tiles, p.units,
                       p.grid, p.maxt);
}
}  // namespace

// Setup: [N][K] codes -> the tile layout above. Thread t writes the t-th
// 16-byte chunk of the tiled array, so a wave writes 1 KiB contiguously; it
// reads the 16 codes of its column at K-elements 128*kt + 32*(l/16) + 16*h, and
// the two halves of each 128-byte run of a row are read by adjacent waves.
// (Moving source chunks in row order instead scattered 16-byte stores over
// the tile, each 256-byte lane run assembled by 16 workgroups: 53 MB written
// for 26 MB of tiles and 29.6 us at N = K = 5120.)
__global__ __launch_bounds__(256) void mxfp8_tile_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         int64_t N, int64_t K) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t k16 = K >> 4, KT = K >> 7;
    if (t >= N * k16) return;
    const int64_t tile = t >> 7, h = (t >> 6) & 1, lane = t & 63;   // 128 chunks per 2 KiB tile
    const int64_t nb = tile / KT, kt = tile - nb * KT;
    const int64_t col = nb * 16 + (lane & 15), q = lane >> 4;
    dst[t] = src[col * k16 + 8 * kt + 2 * q + h];
}

hipError_t launch_mxfp8_tile(const uint8_t *src, uint8_t *dst, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t chunks = N * K / 16;
    hipLaunchKernelGGL(mxfp8_tile_kernel, dim3((uint32_t)((chunks + 255) / 256)), dim3(256), 0, stream,
                       (const uint4 *)src, (uint4 *)dst, N, K);
    return hipGetLastError();
}

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
    // row tiles of 32, 64 or 128 (MBW = 1, 2, 4 row blocks per wave), 128 columns
    switch (plan.bm) {
    case 32: return mx_wide_launch<1>(plan, x, w, scales, out, M, N, K, workspace, stream);
    case 64: return mx_wide_launch<2>(plan, x, w, scales, out, M, N, K, workspace, stream);
    default: return mx_wide_launch<4>(plan, x, w, scales, out, M, N, K, workspace, stream);
    }
}

}  // namespace svq
