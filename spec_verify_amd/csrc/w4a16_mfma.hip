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

#include "svq_dma.h"
#include "svq_launch.h"
#include "svq_streamk.h"

namespace svq {

// Scale words of the NG groups of one K tile (G = 128 / NG): v is, in lane row
// g, the word of group g (rows past NG repeat groups); on return o[q] holds in
// every row the word of row q. Two permlane swaps for NG = 2, three for NG = 4.
template <int NG>
__device__ __forceinline__ void group_scale_words(uint32_t v, uint32_t (&o)[NG]) {
    if constexpr (NG == 1) {
        o[0] = v;
    } else {
        // rows (0, 1, 0, 1) and (2, 3, 2, 3)
        const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        // row 0 and row 1 in every row
        const auto c = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
        o[0] = c[0];
        o[1] = c[1];
        if constexpr (NG == 4) {
            const auto e = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
            o[2] = e[0];
            o[3] = e[1];
        }
    }
}

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
//
// G = 32 / 64 with few rows (PACK > 0): the 16 A-operand rows are split into
// slots of RS rows, one slot per group, and a lane supplies x row r % RS of its
// slot's group or zeros, so one MFMA chain leaves several groups' partial sums
// in different output rows, and a single scale FMA per output element applies
// the right group's scale (unpacked, every group needs its own chain and one
// FMA per element). The groups' rows are summed across lane rows once, after
// the loop. PACK 1 (G = 32: 4 slots of 4 rows, M <= 4; G = 64: 2 slots of 8
// rows, M <= 8): the words stay as repacked, so in MFMA step j lane row g
// supplies K-rows 32g + 8j.., of group g (G = 32) or g / 2 (G = 64): lane
// (r, g) reads x when slot r / RS is that group; one chain per tile. PACK 2
// (G = 32, M <= 8): transposed words (step j is group j), 2 slots of 8 rows:
// steps 0 and 1 feed one chain with x in slot j, steps 2 and 3 a second chain
// likewise. PACK 0: transposed words, one chain per group (any M).
// ---------------------------------------------------------------------------
template <int WAVES, int WPB, int D, int GSHIFT, int PACK>
__global__ __launch_bounds__(64 * WAVES) void w4a16_skinny_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int M, int N, int K, int splits, int S, int groups) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NG = 128 >> GSHIFT;
    constexpr int SPG = 4 / NG;
    static_assert(PACK == 0 || (GSHIFT == 5 && (PACK == 1 || PACK == 2)) || (GSHIFT == 6 && PACK == 1),
                  "packed rows: G = 32 (one or two chains) or G = 64 (one chain)");
    constexpr bool kTrans = GSHIFT < 7 && PACK != 1;
    constexpr int RS = (GSHIFT == 5 && PACK == 1) ? 4 : 8;  // rows per slot when packed
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int sp = lb % splits;
    // the column blocks are dealt evenly to `groups` workgroups per K range
    // (floor or ceil of blocks / groups each, at most WAVES / WPB); WPB waves
    // per block, waves past the workgroup's last block idle
    constexpr int wpb = WPB;
    const uint32_t grp = (uint32_t)(lb / splits), nblocks = (uint32_t)(N >> 4);
    const int nb0 = (int)(grp * nblocks / (uint32_t)groups);                   // first block of the workgroup
    const int nblk = (int)((grp + 1) * nblocks / (uint32_t)groups) - nb0;      // blocks it owns
    const int bw = wave / wpb, wsub = wave - bw * wpb;   // this wave's block and rank in it
    const int nb = nb0 + min(bw, nblk - 1);            // clamped: a wave past the last block idles
    const int KT = K >> 7;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wt + (size_t)nb * KT * 64, (uint32_t)KT * 1024);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + nb * 16, (uint32_t)(((size_t)(K >> GSHIFT) * N - nb * 16) * 2));
    const uint32_t w_vo = lane * 16;
    // the aligned dword holding this lane's fp16 scale; s_sh selects the half.
    // Unpacked, one load per tile brings the scales of all NG groups: lane row g
    // loads group g mod NG, and group_scale_words hands every row all of them.
    // Packed, lane row g's output rows belong to one group per chain: g (PACK 1,
    // G = 32), g / 2 (PACK 1, G = 64, and PACK 2's first chain; its second
    // chain's group is 2 + g / 2, read by a second load)
    const uint32_t s_grp = PACK == 0 ? (uint32_t)(g & (NG - 1)) : (RS == 4 ? (uint32_t)g : (uint32_t)(g >> 1));
    const uint32_t s_vo = (r & 14) * 2 + s_grp * (uint32_t)N * 2u;
    const int s_sh = (r & 1) * 16;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = (bw < nblk && wsub < kcnt) ? (kcnt - 1 - wsub) / wpb + 1 : 0;
    const uint4 bneg = make_uint4(kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair, kBf16Neg136Pair);

    uint4 wA[D], wB[D];
    uint32_t sA[D], sB[D], sA2[D], sB2[D];
#define SVQ_LOAD(W, SS, SS2, I0)                                                     \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wsub + ((I0) + d) * wpb;                               \
        W[d] = bload16(wr, w_vo, kt * 1024);                                         \
        SS[d] = bload4(sr, s_vo, kt * NG * N * 2);                                   \
        if constexpr (PACK == 2) SS2[d] = bload4(sr, s_vo + 4u * (uint32_t)N, kt * NG * N * 2); \
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
    if (ntile > 0) SVQ_LOAD(wA, sA, sA2, 0)
    if (ntile > D) SVQ_LOAD(wB, sB, sB2, D)
    // packed rows: 256 zero bytes after the x stage, read by the lanes whose
    // slot does not hold the group of the step
    const int zoff = M * xs_stride;
    if constexpr (PACK > 0) {
        if (threadIdx.x < 16) *(uint4 *)(smem + zoff + 16 * threadIdx.x) = make_uint4(0, 0, 0, 0);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    {
        constexpr int LPT = PACK == 2 ? 3 : 2;  // loads per prefetched tile
        const int na = ntile < D ? ntile : D;
        const int nb2 = ntile - D < 0 ? 0 : (ntile - D < D ? ntile - D : D);
        wait_vmcnt_at_most<LPT * 2 * D>((na + nb2) * LPT);
    }
    // a bare barrier: __syncthreads() would also wait for the weight prefetch
    __builtin_amdgcn_s_barrier();

    // A operand of MFMA step j for tile i of the range: row min(r, M-1), 8 bf16
    // at K offset 32j + 8g (transposed words) or 32g + 8j
    const int arow = PACK > 0 ? (r % RS < M ? r % RS : M - 1) : (r < M ? r : M - 1);
    const uint8_t *abase = smem + arow * xs_stride + (kTrans ? 16 * g : 64 * g);
    constexpr int kXStep = kTrans ? 64 : 16;
    // packed rows: whether this lane reads x (rows past M of a slot read zeros):
    // PACK 1 when its slot holds its lane row's group; PACK 2 in even steps
    // for slot 0, in odd steps for slot 1
    const int slot = r / RS;
    const bool act0 = PACK == 0 || ((r % RS) < M && (PACK == 1 ? slot == (RS == 4 ? g : g >> 1) : slot == 0));
    const bool act1 = PACK == 2 && (r % RS) < M && slot == 1;
    const uint8_t *zrow = smem + zoff;

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#define SVQ_COMPUTE(W, SS, SS2, I0)                                                  \
    {                                                                                \
        uint32_t wj[D][4];                                                           \
        _Pragma("unroll") for (int d = 0; d < D; ++d) {                              \
            wj[d][0] = W[d].x; wj[d][1] = W[d].y; wj[d][2] = W[d].z; wj[d][3] = W[d].w; \
            if constexpr (kTrans) transpose_rows_words(wj[d][0], wj[d][1], wj[d][2], wj[d][3]); \
        }                                                                            \
        _Pragma("unroll") for (int d = 0; d < D; ++d) {                              \
            if ((I0) + d < ntile) {                                                  \
                const uint8_t *ap = abase + (wsub + ((I0) + d) * wpb) * 256;         \
                if constexpr (PACK == 0) {                                           \
                    uint32_t sw[NG];                                                 \
                    group_scale_words<NG>(SS[d], sw);                                \
                    _Pragma("unroll") for (int q = 0; q < NG; ++q) {                 \
                        f32x4 P = {0.f, 0.f, 0.f, 0.f};                              \
                        _Pragma("unroll") for (int jj = 0; jj < SPG; ++jj) {         \
                            const int j = q * SPG + jj;                              \
                            const uint4 A = *(const uint4 *)(ap + j * kXStep);       \
                            P = mfma16x16x32(A, bneg, P);                            \
                            P = mfma16x16x32(A, word_to_bf16x8(wj[d][j]), P);        \
                        }                                                            \
                        const float sf = fp16_bits_to_f32((uint16_t)(sw[q] >> s_sh));          \
                        _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sf, P[i], acc[i]); \
                    }                                                                \
                } else {                                                             \
                    const uint8_t *a0 = act0 ? ap : zrow, *a1 = act1 ? ap : zrow;    \
                    f32x4 P = {0.f, 0.f, 0.f, 0.f}, P2 = {0.f, 0.f, 0.f, 0.f};       \
                    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                  \
                        const uint4 B = word_to_bf16x8(wj[d][j]);                    \
                        if constexpr (PACK == 1) {                                   \
                            const uint4 A = *(const uint4 *)(a0 + j * kXStep);       \
                            P = mfma16x16x32(A, bneg, P);                            \
                            P = mfma16x16x32(A, B, P);                               \
                        } else {                                                     \
                            const uint4 A = *(const uint4 *)(((j & 1) ? a1 : a0) + j * kXStep); \
                            f32x4 &Q = j < 2 ? P : P2;                               \
                            Q = mfma16x16x32(A, bneg, Q);                            \
                            Q = mfma16x16x32(A, B, Q);                               \
                        }                                                            \
                    }                                                                \
                    const float sf = fp16_bits_to_f32((uint16_t)(SS[d] >> s_sh));    \
                    _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sf, P[i], acc[i]); \
                    if constexpr (PACK == 2) {                                       \
                        const float sf2 = fp16_bits_to_f32((uint16_t)(SS2[d] >> s_sh)); \
                        _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sf2, P2[i], acc[i]); \
                    }                                                                \
                }                                                                    \
            }                                                                        \
        }                                                                            \
    }

    if (ntile > 0) {
        for (int i0 = 0;; i0 += 2 * D) {
            SVQ_COMPUTE(wA, sA, sA2, i0)
            if (i0 + D >= ntile) break;
            SVQ_LOAD(wA, sA, sA2, i0 + 2 * D)
            SVQ_COMPUTE(wB, sB, sB2, i0 + D)
            if (i0 + 2 * D >= ntile) break;
            SVQ_LOAD(wB, sB, sB2, i0 + 3 * D)
        }
    }
#undef SVQ_LOAD
#undef SVQ_COMPUTE

    if constexpr (PACK > 0) {
        // each group's rows sit in another lane row: sum lane rows g and g ^ 2
        // (and then g ^ 1 when the slots are 4 rows), which leaves output row
        // 4g + i of the usual layout in lane row g for every valid row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const auto a = __builtin_amdgcn_permlane32_swap(f32_bits(acc[i]), f32_bits(acc[i]), false, false);
            acc[i] = bits_f32(a[0]) + bits_f32(a[1]);
            if constexpr (RS == 4) {
                const auto c = __builtin_amdgcn_permlane16_swap(f32_bits(acc[i]), f32_bits(acc[i]), false, false);
                acc[i] = bits_f32(c[0]) + bits_f32(c[1]);
            }
        }
    }

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
// Wide kernel: any M (built for M = 128). Stream-K: the (output tile, 128-row
// K step) units are split evenly over the workgroups (tile-aligned K ranges when
// there are fewer tiles than CUs). A tile computed whole by one workgroup is
// written as bf16; a shared tile's fp32 partials are plain-stored and summed in
// workgroup order by a second launch (wide_sum_kernel), so the result is
// deterministic and no workgroup waits for another. Measured on the MI355X at
// M = 128 (K = 5120, N = 17408 / K = 17408, N = 5120): 45.0 / 46.0 us with the
// partials reduced inside the kernel through coherent stores, arrival counters
// and bounded waits, 41.5 / 39.6 us with the second launch.
//
// Workgroup: WR x WC waves (two per SIMD, so one wave's MFMAs cover the other's
// VALU work), output tile BM x BN; a wave owns MBW 16-row blocks x CT 16-column
// tiles. With MBW = 8 every converted weight operand feeds eight MFMAs, which
// keeps the dequant VALU work under the MFMA issue budget.
//
// Pipeline: a ring of three LDS stages, each one K step: x (BM rows x 128,
// 16-byte chunks XOR-swizzled by row so that the MFMA A reads are
// bank-conflict free), the BN/16 weight tiles, the fp16 scales, and (G = 128)
// -136 * (group sums of x). Stages are filled by LDS-DMA (buffer loads that
// write LDS directly; rows past M and columns past N read as zero), two steps
// ahead.
//
// Two ways to apply the scales, by group size. G = 128: the weight operand is
// the exact bf16 of 128 + q, each group's MFMA chain starts from -136 * (sum of
// x over the group), computed for step i+1 during step i from the staged x,
// and the chain's result is scaled by one fp32 FMA per output: about one FMA
// per MFMA. G = 32 and 64: that costs 2 or 4 FMAs per MFMA (one per output per
// group), which the dequantization then has to fit beside; instead the weight
// operand itself is (q - 8) * s, formed in fp32 (q * s - 8 s, one rounding) and
// rounded to bf16, so the MFMAs accumulate straight across groups, with no
// group sums and no FMAs (23 VALU ops per weight word, shared by the MBW row
// blocks). The bf16 rounding of each dequantized weight (relative 2^-9, random
// in sign) stays far inside the accuracy gate. The DMAs are
// issued from inline asm and waited for explicitly (s_waitcnt vmcnt), because
// the compiler cannot tell a DMA into one slot from reads of another and would
// wait for every DMA in flight before each LDS read.
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
    static constexpr bool PS = GSHIFT < 7;       // scales applied in the dequantization
    // one LDS stage (slot): x, weight tiles, fp16 scales [NG][BN], and for
    // G = 128 -136 * group sums of x [BM]
    static constexpr int XB = BM * 256;
    static constexpr int WB = (BN / 16) * 1024;
    static constexpr int SB = NG * BN * 2;
    static constexpr int OFF_W = XB, OFF_S = XB + WB, OFF_N = XB + WB + SB;
    static constexpr int SLOT = OFF_N + (PS ? 0 : BM * 4);
    static constexpr int XI = BM / 4 / WAVES;    // x DMAs per wave per stage (1 KiB = 4 rows each)
    static constexpr int WI = BN / 16 / WAVES;   // weight DMAs per wave per stage (one tile each)
    static constexpr int SI = NG * BN / 128;     // scale DMAs per stage (128 fp16 each), waves 0..SI-1
    static constexpr int MAXPS = XI + WI + 1;    // most DMAs one wave issues per stage
    static_assert(XI * 4 * WAVES == BM && WI * 16 * WAVES == BN, "stage split over the waves");
    static_assert(SI <= WAVES, "one scale DMA per wave at most");
    static_assert(PS || BM == 16 * WAVES, "each wave sums x over 16 rows");
    static_assert(SLOT % 16 == 0 && SLOT < 65536, "slot offsets fit a ds immediate");
    static_assert(MBW % 2 == 0, "row blocks go in pairs");
};

template <int MBW, int WR, int WC, int CT, int GSHIFT>
__global__ __launch_bounds__(64 * WR * WC) void w4a16_wide_kernel(
    const uint16_t *__restrict__ x, const uint4 *__restrict__ wt,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, f32x4 *__restrict__ part, int M,
    int N, int K, int col_tiles, int64_t units, int grid, int maxt) {
    using C = WideCfg<MBW, WR, WC, CT, GSHIFT>;
    constexpr int BM = C::BM, BN = C::BN, NG = C::NG, SPG = C::SPG, NV = C::NV;
    __shared__ __attribute__((aligned(16))) uint8_t ring[3 * C::SLOT];

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
    // this wave's DMAs per stage: x, a scale row, weights
    const int per_step = C::XI + (wave < C::SI ? 1 : 0) + C::WI;
    // group sums (G = 128): rows and K quarters of this wave, and their LDS offsets
    const int srow = 16 * wave + (lane >> 2), q4 = lane & 3;
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
    // weights (the order the G = 128 waits below rely on)
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
        // G = 128: -136 * (sum of x over the group) for rows 16*wave.. of slot st
        auto sums = [&](int st) {
            static_assert(C::PS || NG == 1, "the sums cover one group per step");
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
            // the four K quarters of a row sit in adjacent lanes: quad DPP sums
            t += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(t), 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
            t += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(t), 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
            __attribute__((address_space(3))) float *xn =
                (__attribute__((address_space(3))) float *)(b + offNw);
            if (q4 == 0) xn[0] = -136.f * t;
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
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = lds_ld<uint32_t>(b + offW + ct * 1024 + j * 256);
                    if constexpr (C::PS) {
                        const float s = sfa[j / SPG][ct];
                        B[j][ct] = word_to_bf16x8_scaled(w, s, -8.f * s);
                    } else {
                        B[j][ct] = word_to_bf16x8(w);
                    }
                }
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
                if constexpr (C::PS) {
                    // scaled weights: the MFMAs accumulate into acc directly
                    uint4 A[2][2][SPG];
                    auto load_a = [&](int p, uint4 (&Ap)[2][SPG]) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int jj = 0; jj < SPG; ++jj)
                                Ap[h][jj] = lds_ld16(b + offA[q * SPG + jj] + (wr * MBW + 2 * p + h) * 4096);
                    };
                    load_a(pa, A[pa & 1]);
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        if (p < pa || p >= pe) continue;
                        if (p + 1 < pe) load_a(p + 1, A[(p + 1) & 1]);
#pragma unroll
                        for (int jj = 0; jj < SPG; ++jj)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int ct = 0; ct < CT; ++ct)
                                    acc[(2 * p + h) * CT + ct] = mfma16x16x32(A[p & 1][h][jj], B[q * SPG + jj][ct],
                                                                              acc[(2 * p + h) * CT + ct]);
                    }
                    continue;
                }
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
        if constexpr (!C::PS) {
            // stage 0 has landed (at most stage 1's DMAs are outstanding)
            if (n > 1) wait_vmcnt_at_most<C::MAXPS>(per_step);
            else wait_vmcnt<0>();
            lds_barrier();
            sums(slot0);
        }
        int st = slot0;
        for (int i = 0; i < n; ++i, st = (st == 2 ? 0 : st + 1)) {
            if constexpr (C::PS) {
                // this wave's stage of step i has landed (only step i+1's may be outstanding)
                if (i + 1 < n) wait_vmcnt_at_most<C::MAXPS>(per_step);
                else wait_vmcnt<0>();
            } else {
                // all but the weights of step i+1 have landed: its x is summed below
                if (i + 1 < n) wait_vmcnt<C::WI>();
                else wait_vmcnt<0>();
            }
            lds_barrier();  // every wave's slot st (and x of slot st+1) is in; slot st+2 is free
            const int st1 = st == 2 ? 0 : st + 1, st2 = st1 == 2 ? 0 : st1 + 1;
            prep(st);
            compute(st, std::integral_constant<int, 0>{});
            if (i + 2 < n) issue(sg, st2, s0 + i + 2);
            if constexpr (!C::PS)
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
            // a K range of a shared tile: the fp32 partial, summed by wide_sum_kernel
            f32x4 *mp = wide_partial<NV, C::NT>(part, wg, maxt, tile - sk_first_tile(wg, units, grid, KT));
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
constexpr int kSkinnyDepth = 2;

// Workgroup shape: WAVES waves, WPB of them per column block, and `groups`
// workgroups per K range over which the column blocks are dealt evenly (each
// takes floor or ceil of blocks / groups). One x stage per workgroup is shared
// by its blocks. First choice: 16 waves and one workgroup per CU and K range,
// so that every CU streams the same number of blocks give or take one (with
// 1088 blocks, 4 or 5 per CU, against 4 or 6 when 544 two-block workgroups land
// 2 or 3 to a CU) and stages x once (measured: verify M = 5 up 14.9 -> 13.1 us,
// M = 3 up 13.8 -> 12.7 us, M = 3 down 14.8 -> 14.0 us). When that does not
// fit (more than 8 blocks per workgroup, or more outputs than threads), the
// most waves per block, then the fewest blocks per workgroup, at 16, 8 or 4
// waves and 1, 2 or 4 blocks, with the whole grid resident at once
// (registers, waves and LDS per CU).
struct SkinnyShape {
    int waves, wpb, groups;
};

// Packed rows for G = 32 / 64 (see the kernel): 1 = one chain, 2 = two chains,
// 0 = transposed words (G = 128 and larger M).
inline int skinny_pack(int GS, int M) {
    if (GS == 5) return M <= 4 ? 1 : M <= 8 ? 2 : 0;
    if (GS == 6) return M <= 8 ? 1 : 0;
    return 0;
}
// the packed kernels keep 256 zero bytes after the x stage
inline size_t skinny_lds(int M, int S, int waves, int pack) {
    return skinny_lds_bytes(M, S, waves) + (pack ? 256 : 0);
}

template <int GS, int PACK>
SkinnyShape skinny_shape(const SmallPlan &p, int M, int64_t N) {
    static const int r16 = resident_blocks(w4a16_skinny_kernel<16, 4, kSkinnyDepth, GS, PACK>, 1024);
    static const int r8 = resident_blocks(w4a16_skinny_kernel<8, 4, kSkinnyDepth, GS, PACK>, 512);
    static const int r4 = resident_blocks(w4a16_skinny_kernel<4, 4, kSkinnyDepth, GS, PACK>, 256);
    const int64_t blocks = N / 16;
    {
        const int r = std::min(r16, (int)(kLdsPerCu / skinny_lds(M, p.S, 16, PACK)));
        const int64_t groups = std::min<int64_t>(blocks, (int64_t)p.cus / p.splits);
        const int64_t maxblk = groups > 0 ? (blocks + groups - 1) / groups : 0;
        if (r >= 1 && groups >= 1 && maxblk <= 8 && maxblk * M <= 64) {
            const int wpb = (int)(16 / maxblk);
            return SkinnyShape{16, wpb >= 16 ? 16 : wpb >= 8 ? 8 : wpb, (int)groups};
        }
    }
    SkinnyShape best{4, 4, (int)blocks};
    int best_wpb = 0, best_bpw = 1;
    for (const int waves : {16, 8, 4}) {
        const int r_occ = waves == 16 ? r16 : waves == 8 ? r8 : r4;
        const int r = std::min(r_occ, (int)(kLdsPerCu / skinny_lds(M, p.S, waves, PACK)));
        // bpw * 16 * M outputs are summed by one thread each: bpw * M <= 4 * waves
        for (int bpw = 1; bpw <= 4 && bpw * M <= 4 * waves; bpw *= 2) {
            if ((blocks + bpw - 1) / bpw * p.splits <= (int64_t)r * p.cus) {
                // most waves per block; on a tie, fewer blocks per workgroup
                // (measured: 640 workgroups of 8 waves beat 320 of 16 waves)
                if (waves / bpw > best_wpb || (waves / bpw == best_wpb && bpw < best_bpw)) {
                    best = SkinnyShape{waves, waves / bpw, (int)((blocks + bpw - 1) / bpw)};
                    best_wpb = waves / bpw;
                    best_bpw = bpw;
                }
                break;
            }
        }
    }
    return best;
}

template <int WAVES, int WPB, int GS, int PACK>
hipError_t skinny_launch_g(const SmallPlan &p, int groups, const void *x, const int32_t *wt, const void *sc,
                           void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    return launch_gemm(w4a16_skinny_kernel<WAVES, WPB, kSkinnyDepth, GS, PACK>,
                       dim3((uint32_t)((int64_t)groups * p.splits)), dim3(64 * WAVES),
                       skinny_lds(M, p.S, WAVES, PACK), stream,
                       (const uint16_t *)x, (const uint4 *)wt, (const uint16_t *)sc, (uint16_t *)out,
                       ws_counters(ws), (float *)ws_partials(ws), M, (int)N, (int)K, p.splits, p.S, groups);
}

template <int GS, int PACK>
hipError_t skinny_launch(const SmallPlan &p, const void *x, const int32_t *wt, const void *sc, void *out,
                         int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    const SkinnyShape sh = skinny_shape<GS, PACK>(p, M, N);
    const int g = sh.groups;
#define SVQ_SKINNY(W, P) return skinny_launch_g<W, P, GS, PACK>(p, g, x, wt, sc, out, M, N, K, ws, stream)
    if (sh.waves == 16) {
        switch (sh.wpb) {
        case 16: SVQ_SKINNY(16, 16);
        case 8: SVQ_SKINNY(16, 8);
        case 5: SVQ_SKINNY(16, 5);
        case 4: SVQ_SKINNY(16, 4);
        case 3: SVQ_SKINNY(16, 3);
        default: SVQ_SKINNY(16, 2);
        }
    }
    if (sh.waves == 8) {
        switch (sh.wpb) {
        case 8: SVQ_SKINNY(8, 8);
        case 4: SVQ_SKINNY(8, 4);
        default: SVQ_SKINNY(8, 2);
        }
    }
    switch (sh.wpb) {
    case 4: SVQ_SKINNY(4, 4);
    case 2: SVQ_SKINNY(4, 2);
    default: SVQ_SKINNY(4, 1);
    }
#undef SVQ_SKINNY
}

template <int MBW, int WR, int WC, int CT, int GS>
hipError_t wide_launch(const WidePlan &p, const void *x, const int32_t *wt, const void *sc,
                       void *out, int64_t M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    using C = WideCfg<MBW, WR, WC, CT, GS>;
    f32x4 *part = (f32x4 *)ws_partials(ws);
    hipError_t e = launch_gemm(w4a16_wide_kernel<MBW, WR, WC, CT, GS>, dim3((uint32_t)p.grid),
                               dim3(C::NT), 0, stream, (const uint16_t *)x, (const uint4 *)wt,
                               (const uint16_t *)sc, (uint16_t *)out, part, (int)M, (int)N, (int)K,
                               p.col_tiles, p.units, p.grid, p.maxt);
    if (e != hipSuccess || !p.workspace_bytes) return e;
    // shared tiles: the partials' sum, one workgroup per (tile, accumulator pair)
    return launch_gemm(wide_sum_kernel<MBW, WR, WC, CT, C::BM, C::BN>,
                       dim3((uint32_t)((int64_t)p.row_tiles * p.col_tiles * C::NV / 2)), dim3(C::NT), 0, stream,
                       (const f32x4 *)part, (uint16_t *)out, (int)M, (int)N, (int)K, p.col_tiles, p.units,
                       p.grid, p.maxt);
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
    case 32:
        switch (skinny_pack(5, M)) {
        case 1: return skinny_launch<5, 1>(plan, x, wt, scales, out, M, N, K, workspace, stream);
        case 2: return skinny_launch<5, 2>(plan, x, wt, scales, out, M, N, K, workspace, stream);
        default: return skinny_launch<5, 0>(plan, x, wt, scales, out, M, N, K, workspace, stream);
        }
    case 64:
        return skinny_pack(6, M) ? skinny_launch<6, 1>(plan, x, wt, scales, out, M, N, K, workspace, stream)
                                 : skinny_launch<6, 0>(plan, x, wt, scales, out, M, N, K, workspace, stream);
    case 128: return skinny_launch<7, 0>(plan, x, wt, scales, out, M, N, K, workspace, stream);
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
