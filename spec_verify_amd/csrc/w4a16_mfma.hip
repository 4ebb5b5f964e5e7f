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
#include <type_traits>

#include "svq_launch.h"
#include "svq_streamk.h"

namespace svq {

// ---------------------------------------------------------------------------
// Skinny kernel: M <= 16, one 16-row MFMA tile (MFMA rows >= M repeat row M-1
// and their results are dropped). A workgroup owns BPW consecutive 16-column
// blocks and one range of S K-tiles of each; WAVES / BPW waves per block take
// its tiles round-robin. The workgroup's x rows (M x 128*S bf16) are staged
// once in LDS and shared by its blocks, so the A operands come from LDS and the
// vector-memory path carries only weights and scales, which each wave
// prefetches 2*D tiles deep behind the staging loads. Several blocks per
// workgroup keep every workgroup resident at once where one x stage per block
// would not fit the chip's LDS (the launcher picks BPW). Memory-bound; the
// MFMA pipe is mostly idle, so the -136 * sum(x) term is also computed on it,
// by an MFMA against a constant -136 operand.
// ---------------------------------------------------------------------------
template <int WAVES, int BPW, int D, int GSHIFT>
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
    const int sp = lb % splits;
    static_assert(WAVES % BPW == 0, "whole waves per block");
    constexpr int wpb = WAVES / BPW;                   // waves per block
    const int nb0 = (lb / splits) * BPW;               // first block of the workgroup
    const int nblk = min(BPW, (N >> 4) - nb0);         // blocks it owns (last one: fewer)
    const int bw = wave / wpb, wsub = wave - bw * wpb;   // this wave's block and rank in it
    const int nb = nb0 + min(bw, nblk - 1);            // clamped: a wave past the last block idles
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
    const int ntile = (bw < nblk && wsub < kcnt) ? (kcnt - 1 - wsub) / wpb + 1 : 0;
    const uint4 bneg = make_uint4(kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair);

    uint4 wA[D], wB[D];
    uint32_t sA[D][NG], sB[D][NG];
#define SVQ_LOAD(W, SS, I0)                                                          \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wsub + ((I0) + d) * wpb;                               \
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
                const uint8_t *ap = abase + (wsub + ((I0) + d) * wpb) * 256;         \
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
    __shared__ int s_flags[16];
    float v = 0.f;
    if (threadIdx.x < nblk * 16 * M) {
        const int b = threadIdx.x / (16 * M), t = threadIdx.x - b * 16 * M;
        for (int w = 0; w < wpb; ++w) v += red[((b * wpb + w) * M) * 16 + t];
    }
    multiblock_finish(v, M, N, nb0, nblk, sp, splits, out, cnt, part, s_flags);
}

// ---------------------------------------------------------------------------
// Wide kernel: any M (built for M = 128). Persistent stream-K: one workgroup
// per compute unit, each taking an equal contiguous share of the (output tile,
// 128-row K step) units. A tile computed by several workgroups is reduced by
// the ones that finish it together (sk_reduce): fp32 partials added in
// workgroup order, so the result is deterministic.
//
// Workgroup: WR x WC waves (two per SIMD, so one wave's MFMAs cover the other's
// VALU work), output tile BM x BN; a wave owns MBW 16-row blocks x CT 16-column
// tiles. With MBW = 8 every converted weight operand feeds eight MFMAs, which
// keeps the dequant VALU work under the MFMA issue budget.
//
// Pipeline: a ring of three LDS stages, each one K step: x (BM rows x 128,
// 16-byte chunks XOR-swizzled by row so that the MFMA A reads are
// bank-conflict free), the BN/16 weight tiles, the fp16 scales, and
// -136 * (group sums of x). Stages are filled by LDS-DMA (buffer loads that
// write LDS directly; rows past M and columns past N read as zero), two steps
// ahead; the group sums of step i+1 are computed during step i. Each slot is
// its own LDS object, so the compiler can tell a DMA into one slot from reads
// of another and does not wait for in-flight DMAs before every LDS read.
//
// MFMA step j of a K step covers rows 32j..32j+31; lane (r, g) supplies
// K-rows 32j+8g.. of x row r and of column r, and its weight word is word g of
// lane 16j+r of the repacked tile (a transposed read from LDS), so every
// group size uses the same mapping.
// ---------------------------------------------------------------------------
template <int MBW, int WR, int WC, int CT, int GSHIFT>
struct WideCfg {
    static constexpr int WAVES = WR * WC;
    static constexpr int NT = 64 * WAVES;
    static constexpr int BM = 16 * MBW * WR;
    static constexpr int BN = 16 * CT * WC;
    static constexpr int NG = 128 >> GSHIFT;
    static constexpr int SPG = 4 / NG;
    static constexpr int NV = MBW * CT;          // f32x4 accumulators per lane
    // one LDS stage (slot): x, weight tiles, fp16 scales [NG][BN], -136 *
    // group sums of x [NG][BM]
    static constexpr int XB = BM * 256;
    static constexpr int WB = (BN / 16) * 1024;
    static constexpr int SB = NG * BN * 2;
    static constexpr int OFF_W = XB, OFF_S = XB + WB, OFF_N = XB + WB + SB;
    static constexpr int SLOT = OFF_N + NG * BM * 4;
    static constexpr int XI = BM / 4 / WAVES;    // x DMAs per wave per stage (1 KiB = 4 rows each)
    static constexpr int WI = BN / 16 / WAVES;   // weight DMAs per wave per stage (one tile each)
    static constexpr int SI = NG * BN / 128;     // scale DMAs per stage (128 fp16 each), waves 0..SI-1
    static_assert(XI * 4 * WAVES == BM && WI * 16 * WAVES == BN, "stage split over the waves");
    static_assert(SI <= WAVES, "one scale DMA per wave at most");
    static_assert(BM == 16 * WAVES, "each wave sums x over 16 rows");
    static_assert(SLOT % 16 == 0 && SLOT < 65536, "slot offsets fit a ds immediate");
    static_assert(MBW % 2 == 0, "row blocks go in pairs");
};

// LDS-DMA loads (buffer_load ... lds: lane l's bytes land at M0 + size*l, and
// offsets past num_records read as zero). Written in asm so that the compiler
// does not track them: it cannot tell the ring's slots apart and would wait
// for every DMA in flight before each LDS read. The asm has no output
// registers; every wait for these loads is an explicit s_waitcnt vmcnt, and
// the "memory" clobber keeps LDS accesses in order with them. s_nop 0 covers
// the wait state between writing M0 and the DMA reading it.
struct BufDesc {
    u32x4 v;
};
__device__ __forceinline__ BufDesc buf_desc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return BufDesc{u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u}};
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ void dma_b128(const BufDesc &d, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(d.v), "s"(lds), "s"(soff)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const BufDesc &d, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, %3 offen lds"
                 :
                 : "v"(voff), "s"(d.v), "s"(lds), "s"(soff)
                 : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); }

typedef __attribute__((address_space(3))) uint8_t lds_u8;
// An LDS address the compiler must treat as unknown at this point: every
// address derived from it is then base + per-lane offset + immediate, instead
// of dozens of precomputed addresses held in registers across the loop.
__device__ __forceinline__ const lds_u8 *lds_opaque(uint32_t a) {
    asm volatile("" : "+v"(a));
    return (const lds_u8 *)(uintptr_t)a;
}
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_u8 *p) { return *(const __attribute__((address_space(3))) T *)p; }
__device__ __forceinline__ uint4 lds_ld16(const lds_u8 *p) {
    const u32x4 v = lds_ld<u32x4>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int MBW, int WR, int WC, int CT, int GSHIFT>
__global__ __launch_bounds__(64 * WR * WC) void w4a16_wide_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    f32x4 *__restrict__ part, int M, int N, int K, int col_tiles, int64_t units, int grid,
    int maxt) {
    using C = WideCfg<MBW, WR, WC, CT, GSHIFT>;
    constexpr int BM = C::BM, BN = C::BN, NG = C::NG, SPG = C::SPG, NV = C::NV;
    __shared__ __attribute__((aligned(16))) uint8_t ring[3 * C::SLOT];
    __shared__ int s_sk[3];

    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int wr = wave / WC, wc = wave % WC;
    const int r = lane & 15, g = lane >> 4;
    const int KT = K >> 7;
    const int NB16 = N >> 4;
    const int wg = blockIdx.x;
    const int64_t u_begin = (int64_t)wg * units / grid;
    const int64_t u_end = (int64_t)(wg + 1) * units / grid;
    const uint32_t ring_lds = lds_addr(ring);
    // buffer views: reads past the end return zero (rows >= M, columns >= N)
    const BufDesc xr = buf_desc(x, (uint32_t)((size_t)M * K * 2));
    const BufDesc wrs = buf_desc(wt, (uint32_t)((size_t)N * K / 2));
    const BufDesc sr = buf_desc(sc, (uint32_t)((size_t)(K >> GSHIFT) * N * 2));

    // per-lane LDS offsets within a slot (constant for the whole kernel)
    uint32_t offA[4];  // A operand of MFMA step j: row r of the block, K-rows 32j+8g..
#pragma unroll
    for (int j = 0; j < 4; ++j) offA[j] = r * 256 + (((4 * j + g) ^ r) << 4);
    const uint32_t offW = C::OFF_W + wc * CT * 1024 + (r << 4) + (g << 2);  // word g of lane 16j+r
    const uint32_t offS = C::OFF_S + (wc * CT * 16 + r) * 2;
    const uint32_t offN = C::OFF_N + 16 * g;
    const int srow = 16 * wave + (lane >> 2), q4 = lane & 3;  // group-sum rows of this wave
    uint32_t offX[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) offX[c] = srow * 256 + (((4 * q4 + c) ^ (srow & 15)) << 4);
    const uint32_t offNw = C::OFF_N + srow * 4;

    // A segment is a run of K steps of one tile. Its stages use consecutive
    // ring slots; the next segment's first two stages are issued during the
    // last step of the current one, so their latency hides behind that step
    // and the epilogue.
    struct Seg {
        int tile, s0, n, rt, cb;
    };
    auto seg_at = [&](int64_t u) {
        Seg g;
        g.tile = (int)(u / KT);
        g.s0 = (int)(u % KT);
        g.n = (int)((u_end - u) < (int64_t)(KT - g.s0) ? (u_end - u) : (KT - g.s0));
        g.rt = g.tile / col_tiles;
        g.cb = g.tile % col_tiles;
        return g;
    };
    // DMA of K step kt of segment g into slot st: x, then scales, then
    // weights (the order the waits below rely on)
    auto issue = [&](const Seg &sg, int st, int kt) {
        const uint32_t base = ring_lds + st * C::SLOT;
#pragma unroll
        for (int v = 0; v < C::XI; ++v) {
            const int rl = 4 * (wave * C::XI + v) + (lane >> 4);
            const uint32_t vx = (uint32_t)(sg.rt * BM + rl) * (uint32_t)K * 2u + (uint32_t)(((lane & 15) ^ (rl & 15)) * 16);
            dma_b128(xr, base + (wave * C::XI + v) * 1024, vx, (uint32_t)kt * 256u);
        }
        if (wave < C::SI) {
            const int q = wave / (BN / 128), prt = wave % (BN / 128);
            dma_b32(sr, base + C::OFF_S + (q * BN + prt * 128) * 2, lane * 4,
                    ((uint32_t)(kt * NG + q) * (uint32_t)N + (uint32_t)(sg.cb * BN + prt * 128)) * 2u);
        }
#pragma unroll
        for (int v = 0; v < C::WI; ++v) {
            const int t = wave * C::WI + v;
            dma_b128(wrs, base + C::OFF_W + t * 1024, lane * 16,
                     ((uint32_t)(sg.cb * (BN / 16) + t) * (uint32_t)KT + (uint32_t)kt) * 1024u);
        }
    };
    int slot0 = 0;         // ring slot of the segment's first stage
    bool issued = false;   // the segment's first stages were issued ahead
    for (int64_t u = u_begin; u < u_end;) {
        const Seg sg = seg_at(u);
        const int tile = sg.tile, s0 = sg.s0, n = sg.n, rt = sg.rt, cb = sg.cb;
        const int s1 = s0 + n;
        // -136 * (sum of x over each group) for rows 16*wave.. of slot st
        auto sums = [&](int st) {
            const lds_u8 *b = lds_opaque(ring_lds + st * C::SLOT);
            float t = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 v = lds_ld16(b + offX[c]);
                t = dot2_bf16(v.x, kBf16OnePair, t);
                t = dot2_bf16(v.y, kBf16OnePair, t);
                t = dot2_bf16(v.z, kBf16OnePair, t);
                t = dot2_bf16(v.w, kBf16OnePair, t);
            }
            __attribute__((address_space(3))) float *xn =
                (__attribute__((address_space(3))) float *)(b + offNw);
            // the four K quarters of a row sit in adjacent lanes: quad DPP sums
            if constexpr (NG == 4) {
                xn[q4 * BM] = -136.f * t;
            } else if constexpr (NG == 2) {
                t += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(t), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
                if ((q4 & 1) == 0) xn[(q4 >> 1) * BM] = -136.f * t;
            } else {
                t += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(t), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
                t += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(t), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
                if (q4 == 0) xn[0] = -136.f * t;
            }
        };

        f32x4 acc[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

        // The MFMA work of a step, in two halves of the (group, row-block pair)
        // items, so that the step's DMA issue and group sums can sit between
        // them and overlap MFMAs.
        // dequantized weight operands and scales of a step: converted once
        // and shared by both halves of the MFMA work
        uint4 B[4][CT];
        float sfa[NG][CT];
        auto prep = [&](int st) {
            const lds_u8 *b = lds_opaque(ring_lds + st * C::SLOT);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
                for (int q = 0; q < NG; ++q) sfa[q][ct] = fp16_bits_to_f32(lds_ld<uint16_t>(b + offS + (q * BN + ct * 16) * 2));
#pragma unroll
                for (int j = 0; j < 4; ++j) B[j][ct] = word_to_bf16x8(lds_ld<uint32_t>(b + offW + ct * 1024 + j * 256));
            }
        };
        auto compute = [&](int st, auto H) {
            constexpr int half = decltype(H)::value;
            constexpr int NP = MBW / 2;
            constexpr int NI = NG * NP;
            const lds_u8 *b = lds_opaque(ring_lds + st * C::SLOT);
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const int i0 = q * NP;  // first item of group q
                if ((i0 + NP <= half * NI / 2) || (i0 >= (half + 1) * NI / 2)) continue;
                const int pa = (i0 < half * NI / 2 ? half * NI / 2 - i0 : 0);
                const int pe = (i0 + NP > (half + 1) * NI / 2 ? (half + 1) * NI / 2 - i0 : NP);
                const float (&sf)[CT] = sfa[q];
                // Row blocks go in pairs (2*CT independent MFMA chains); the
                // next pair's A operands are read while this pair's MFMAs run,
                // and a pair's scale FMAs wait until the next pair's MFMAs are
                // issued, so that neither an MFMA nor an FMA waits on its input.
                uint4 A[2][2][SPG];
                f32x4 I[2][2];
                f32x4 P[2][2][CT];
                auto load_pair = [&](int p, uint4 (&Ap)[2][SPG], f32x4 (&Ip)[2]) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int rb = 2 * p + h;
#pragma unroll
                        for (int jj = 0; jj < SPG; ++jj)
                            Ap[h][jj] = lds_ld16(b + offA[q * SPG + jj] + (wr * MBW + rb) * 4096);
                        Ip[h] = lds_ld<f32x4>(b + offN + (q * BM + (wr * MBW + rb) * 16) * 4);
                    }
                };
                auto fma_pair = [&](int p, const f32x4 (&Pp)[2][CT]) {
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                acc[(2 * p + h) * CT + ct][i] =
                                    __builtin_fmaf(sf[ct], Pp[h][ct][i], acc[(2 * p + h) * CT + ct][i]);
                };
                load_pair(pa, A[pa & 1], I[pa & 1]);
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    if (p < pa || p >= pe) continue;
                    if (p + 1 < pe) load_pair(p + 1, A[(p + 1) & 1], I[(p + 1) & 1]);
                    uint4 (&Ac)[2][SPG] = A[p & 1];
                    f32x4 (&Pc)[2][CT] = P[p & 1];
#pragma unroll
                    for (int jj = 0; jj < SPG; ++jj)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int ct = 0; ct < CT; ++ct)
                                Pc[h][ct] = mfma16x16x32(Ac[h][jj], B[q * SPG + jj][ct], jj == 0 ? I[p & 1][h] : Pc[h][ct]);
                    if (p > pa) fma_pair(p - 1, P[(p - 1) & 1]);
                }
                fma_pair(pe - 1, P[(pe - 1) & 1]);
            }
        };

        const int slot1 = slot0 == 2 ? 0 : slot0 + 1;
        if (!issued) {
            lds_barrier();  // the previous segment is done with every slot
            issue(sg, slot0, s0);
            if (n > 1) issue(sg, slot1, s0 + 1);
        }
        // stage 0 has landed (at most stage 1's DMAs are outstanding)
        if (n > 1) wait_vmcnt_at_most<C::XI + 1 + C::WI>(C::XI + (wave < C::SI ? 1 : 0) + C::WI);
        else wait_vmcnt<0>();
        lds_barrier();
        sums(slot0);
        int st = slot0;
        for (int i = 0; i < n; ++i, st = (st == 2 ? 0 : st + 1)) {
            // this wave's DMAs: all but the weights of step i+1 have landed
            if (i + 1 < n) wait_vmcnt<C::WI>();
            else wait_vmcnt<0>();
            lds_barrier();  // every wave's slot st and x of slot st+1 are in; slot st+2 is free
            const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
            prep(st);
            compute(st, std::integral_constant<int, 0>{});
            if (i + 2 < n) issue(sg, st2, s0 + i + 2);
            if (i + 1 < n) sums(st1);
            if (i + 1 == n && u + n < u_end) {
                // the next segment's first two stages go into the two slots
                // this step does not use
                const Seg nx = seg_at(u + n);
                issue(nx, st1, nx.s0);
                if (nx.n > 1) issue(nx, st2, nx.s0 + 1);
            }
            compute(st, std::integral_constant<int, 1>{});
        }
        slot0 = st;  // one past the last stage's slot
        issued = true;

        // ---- epilogue ----
        // accumulator v = (row block v / CT, column tile v % CT) of this thread
        auto store_v = [&](int v, const f32x4 &val) {
            const int rb = v / CT, ct = v % CT;
            const int nbg = cb * (BN / 16) + wc * CT + ct;
            if (nbg >= NB16) return;
            const int row0 = rt * BM + (wr * MBW + rb) * 16 + 4 * g;
            uint16_t *o = out + (size_t)row0 * N + nbg * 16 + r;
            if (row0 + 4 <= M) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o[(size_t)i * N] = f32_to_bf16_rne(val[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < M) o[(size_t)i * N] = f32_to_bf16_rne(val[i]);
            }
        };
        if (s0 == 0 && s1 == KT) {
#pragma unroll
            for (int v = 0; v < NV; ++v) store_v(v, acc[v]);
        } else {
            sk_reduce<NV, C::NT>(acc, tile, KT, units, grid, maxt, cnt, part, s_sk, store_v);
        }
        u += n;
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
constexpr int kSkinnyDepth = 2;

template <int WAVES, int BPW, int GS>
hipError_t skinny_launch_b(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc,
                           void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    const int64_t groups = (N / 16 + BPW - 1) / BPW;
    hipLaunchKernelGGL((w4a16_skinny_kernel<WAVES, BPW, kSkinnyDepth, GS>),
                       dim3((uint32_t)(groups * p.splits)), dim3(64 * WAVES),
                       skinny_lds_bytes(M, p.S, WAVES), stream,
                       (const uint16_t *)x, (const uint4 *)wt, (const uint16_t *)sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), M, (int)N, (int)K, p.splits, p.S);
    return hipGetLastError();
}

template <int WAVES, int GS>
hipError_t skinny_launch_w(const SmallPlan &p, int bpw, const void *x, const int32_t *wt, const void *sc,
                           void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    switch (bpw) {
    case 1: return skinny_launch_b<WAVES, 1, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    case 2: return skinny_launch_b<WAVES, 2, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    default: return skinny_launch_b<WAVES, 4, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
    }
}

// Workgroup shape: WAVES waves and bpw column blocks per workgroup (WAVES/bpw
// waves per block), chosen so that the whole grid is resident at once
// (registers, waves and LDS per CU), with as many waves per block as
// possible and then as few blocks per workgroup as possible. One x stage per workgroup is shared by its blocks, so more blocks
// per workgroup means fewer stages in LDS. If nothing fits, 4 waves and one
// block per workgroup.
struct SkinnyShape {
    int waves, bpw;
};

template <int GS>
SkinnyShape skinny_shape(const SmallPlan &p, int M, int64_t N) {
    // register-limited residency (the BPW = 2 and 4 instances use as many registers)
    static const int r16 = resident_blocks(w4a16_skinny_kernel<16, 1, kSkinnyDepth, GS>, 1024);
    static const int r8 = resident_blocks(w4a16_skinny_kernel<8, 1, kSkinnyDepth, GS>, 512);
    static const int r4 = resident_blocks(w4a16_skinny_kernel<4, 1, kSkinnyDepth, GS>, 256);
    const int64_t blocks = N / 16;
    SkinnyShape best{4, 1};
    int best_wpb = 0;
    for (const int waves : {16, 8, 4}) {
        const int r_occ = waves == 16 ? r16 : waves == 8 ? r8 : r4;
        const int r = std::min(r_occ, (int)(kLdsPerCu / skinny_lds_bytes(M, p.S, waves)));
        // bpw * 16 * M outputs are summed by one thread each: bpw * M <= 4 * waves
        for (int bpw = 1; bpw <= 4 && bpw * M <= 4 * waves; bpw *= 2) {
            if ((blocks + bpw - 1) / bpw * p.splits <= (int64_t)r * p.cus) {
                // most waves per block; on a tie, fewer blocks per workgroup
                // (measured: 640 workgroups of 8 waves beat 320 of 16 waves)
                if (waves / bpw > best_wpb || (waves / bpw == best_wpb && bpw < best.bpw)) {
                    best = SkinnyShape{waves, bpw};
                    best_wpb = waves / bpw;
                }
                break;
            }
        }
    }
    return best;
}

template <int GS>
hipError_t skinny_launch(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                         int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    const SkinnyShape sh = skinny_shape<GS>(p, M, N);
    switch (sh.waves) {
    case 16: return skinny_launch_w<16, GS>(p, sh.bpw, x, wt, sc, out, M, N, K, ws, stream);
    case 8: return skinny_launch_w<8, GS>(p, sh.bpw, x, wt, sc, out, M, N, K, ws, stream);
    default: return skinny_launch_w<4, GS>(p, sh.bpw, x, wt, sc, out, M, N, K, ws, stream);
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
    // 8 waves of 128 rows x 32 columns: a 128 x 256 tile
    return wide_launch<8, 1, 8, 2, GS>(p, x, wt, sc, out, M, N, K, ws, stream);
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
