// Quantized vocabulary head for gfx950: the W8A16 GEMM for small M and the
// load-time round-to-nearest quantizer that produces its weights (and the INT4
// weights of the W4A16 path).
//
// Format: Eole recipe "Qwen3.8-27B and native MTP speculative decoding",
// section "Optional vocabulary-head quantization": the dense vocabulary
// projection is quantized when the model loads, to int8 or int4, symmetric,
// group-wise (32, 64 or 128 elements along K), round to nearest. Stored here as
//   int8:  codes q [N][K] row-major (two's complement), fp16 scales [K/G][N]
//   int4:  GPTQ words [K/8][N] holding q + 8 (the W4A16 format), fp16 scales [K/G][N]
// with w[n][k] = q[n][k] * s[k/G][n].
//
// W8A16 kernel (M <= 16): the W4A16 skinny design on one byte per weight. A
// workgroup owns one 16-column block; its waves take the 16 x 128 K-tiles
// round-robin. Lane l owns column l%16 and K-rows 32*(l/16).. of a tile: two
// 128-bit loads of its row of W. x comes straight from L2 per tile (rows >= M
// read past the buffer's end as zeros). MFMA 16x16x32 bf16; the MFMA pipe is
// idle enough that the offset of the byte decode is also removed on it.
//
// Byte decode: b ^ 0x80 is q + 128 as an unsigned byte, which v_cvt_f32_ubyte
// turns into an exact float; its upper half is the exact bf16 (integers below
// 256 need 8 significant bits). The -128 comes back per 32-row step as an MFMA
// of x against a constant -128 operand, and the fp16 group scale multiplies
// each group's fp32 MFMA result into the accumulator, as in W4A16.
#include <hip/hip_fp16.h>

#include "svq_launch.h"
#include "svq_streamk.h"

namespace svq {

constexpr uint32_t kBf16Neg128Pair = 0xC300C300u;

// Two bf16 values (q + 128 of bytes 2p, 2p+1 of a flipped dword) in one dword.
__device__ __forceinline__ uint32_t u8pair_bf16(uint32_t u, int p) {
    const float a = (float)((u >> (16 * p)) & 0xffu);
    const float b = (float)((u >> (16 * p + 8)) & 0xffu);
    // upper halves of the two floats: bytes 2,3 of a then bytes 2,3 of b
    return __builtin_amdgcn_perm(f32_bits(b), f32_bits(a), 0x07060302u);
}

// Eight codes (dwords lo, hi: K-rows e = 0..7) -> the bf16x8 B operand of q + 128.
__device__ __forceinline__ uint4 i8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
    return make_uint4(u8pair_bf16(a, 0), u8pair_bf16(a, 1), u8pair_bf16(b, 0), u8pair_bf16(b, 1));
}

// ---------------------------------------------------------------------------
// W8A16 skinny MFMA kernel, M <= 16: one 16-column block and a range of S
// K-tiles per workgroup, x of the range staged once in LDS (the vocabulary
// head, M = 1, K = 5120, N = 248320: 243 -> 218 us against x loaded per tile),
// waves take the tiles round-robin, 8 MFMAs per tile (4 bias, 4 weight).
// ---------------------------------------------------------------------------
template <int WAVES, int D, int GSHIFT>
__global__ __launch_bounds__(64 * WAVES) void w8a16_skinny_kernel(
    const uint16_t *__restrict__ x, const int8_t *__restrict__ w,
    const uint16_t *__restrict__ sc, uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
    float *__restrict__ part, int M, int N, int K, int splits, int S) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NG = 128 >> GSHIFT;  // groups per 128-row tile
    constexpr int SPG = 4 / NG;        // MFMA steps per group
    constexpr bool kTrans = GSHIFT < 7;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int r = lane & 15, g = lane >> 4;
    const int lb = xcd_contiguous(blockIdx.x, gridDim.x);
    const int nb = lb / splits, sp = lb % splits;
    const int KT = K >> 7;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(w + (size_t)nb * 16 * K, (uint32_t)16 * K);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sc + nb * 16, (uint32_t)(((size_t)(K >> GSHIFT) * N - nb * 16) * 2));
    const uint32_t w_vo = r * K + g * 32;
    constexpr int kXStep = kTrans ? 64 : 16;
    // the aligned dword holding this lane's fp16 scale; s_sh selects the half
    const uint32_t s_vo = (r & 14) * 2;
    const int s_sh = (r & 1) * 16;
    // this workgroup's K range: tiles [kbeg, kbeg + kcnt) of the column block
    const int kbeg = sp * S;
    const int kcnt = KT - kbeg < S ? KT - kbeg : S;
    const int ntile = wave < kcnt ? (kcnt - 1 - wave) / WAVES + 1 : 0;
    const uint4 bneg = make_uint4(kBf16Neg128Pair, kBf16Neg128Pair, kBf16Neg128Pair, kBf16Neg128Pair);

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    uint4 vA[D][2], vB[D][2];
    uint32_t sA[D][NG], sB[D][NG];

#define SVQ_LOAD(V, SS, I0)                                                          \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const int kt = kbeg + wave + ((I0) + d) * WAVES;                             \
        V[d][0] = bload16(wr, w_vo, kt * 128);                                       \
        V[d][1] = bload16(wr, w_vo + 16, kt * 128);                                  \
        _Pragma("unroll") for (int q = 0; q < NG; ++q) SS[d][q] = bload4(sr, s_vo, (kt * NG + q) * N * 2); \
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
        wait_vmcnt_at_most<2 * D * (2 + NG)>((na + nb2) * (2 + NG));
    }
    // a bare barrier: __syncthreads() would also wait for the weight prefetch
    __builtin_amdgcn_s_barrier();
    // A operand of MFMA step j: x row min(r, M-1) (rows past M repeat the last
    // row; their products are never stored), K-rows 32j + 8g.. for every group
    // size below 128 (the weight words are transposed to match) or 32g + 8j..
    const int arow = r < M ? r : M - 1;
    const uint8_t *abase = smem + arow * xs_stride + (kTrans ? 16 * g : 64 * g);

#define SVQ_COMPUTE(V, SS, I0)                                                       \
    _Pragma("unroll") for (int d = 0; d < D; ++d) if ((I0) + d < ntile) {            \
        const uint8_t *ap = abase + (wave + ((I0) + d) * WAVES) * 256;               \
        uint32_t lo[4] = {V[d][0].x, V[d][0].z, V[d][1].x, V[d][1].z};               \
        uint32_t hi[4] = {V[d][0].y, V[d][0].w, V[d][1].y, V[d][1].w};               \
        if constexpr (kTrans) {                                                      \
            transpose_rows_words(lo[0], lo[1], lo[2], lo[3]);                        \
            transpose_rows_words(hi[0], hi[1], hi[2], hi[3]);                        \
        }                                                                            \
        _Pragma("unroll") for (int q = 0; q < NG; ++q) {                             \
            f32x4 P = {0.f, 0.f, 0.f, 0.f};                                          \
            _Pragma("unroll") for (int jj = 0; jj < SPG; ++jj) {                     \
                const int j = q * SPG + jj;                                          \
                const uint4 A = *(const uint4 *)(ap + j * kXStep);                   \
                P = mfma16x16x32(A, bneg, P);                                        \
                P = mfma16x16x32(A, i8x8_to_bf16(lo[j], hi[j]), P);                  \
            }                                                                        \
            const float sf = fp16_bits_to_f32((uint16_t)(SS[d][q] >> s_sh));         \
            _Pragma("unroll") for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sf, P[i], acc[i]); \
        }                                                                            \
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

    // cross-wave sum of the valid rows through LDS, in wave order (the x
    // stage is dead now)
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
// Load-time quantizer: dense bf16 W [N][K] -> codes + fp16 scales [K/G][N].
// A workgroup quantizes four groups of 64 consecutive rows: G/8 lanes per row,
// each lane 8 consecutive weights (one 16-byte load; a row's group is one
// contiguous run of 2G bytes, read by consecutive lanes). The group maximum is
// reduced over the row's lanes with DPP and each lane quantizes its 8 weights.
// int8 codes go straight to [N][K] (8 contiguous bytes per lane); GPTQ words
// ([K/8][N]) and scales ([K/G][N]) are transposed through LDS, so that one
// wave stores 64 consecutive columns at once. Per group, in fp32 with IEEE
// division:
//   amax = max |w|, s = fp16_rne(amax / qmax), q = clamp(rint(w / s), -qmax-1, qmax)
// with s used as stored; a group whose stored scale is zero gets q = 0.
// ---------------------------------------------------------------------------
constexpr int kRtnGroupsPerWg = 4;  // groups one workgroup quantizes (loads issued together)

template <int BITS, int GSHIFT>
__global__ __launch_bounds__(8 << GSHIFT) void rtn_quantize_kernel(const uint16_t *__restrict__ w,
                                                                 void *__restrict__ codes,
                                                                 uint16_t *__restrict__ scales, int N,
                                                                 int K) {
    constexpr int G = 1 << GSHIFT;
    constexpr int L = G / 8;  // lanes per row (4, 8 or 16: within one 16-lane DPP row)
    constexpr int GP = kRtnGroupsPerWg;
    constexpr float kQmax = (float)((1 << (BITS - 1)) - 1);
    __shared__ uint32_t words[BITS == 4 ? GP : 1][BITS == 4 ? L : 1][65];
    __shared__ uint16_t sc_lds[GP][64];
    const int t = threadIdx.x;
    const int r = t / L, l = t % L;  // row within the workgroup, lane within the row
    const int n0 = blockIdx.x * 64;
    const int n = n0 + r;
    const int ngroups = K >> GSHIFT;
    const int g0 = blockIdx.y * GP;
    uint4 v[GP];
#pragma unroll
    for (int gi = 0; gi < GP; ++gi) {
        v[gi] = make_uint4(0u, 0u, 0u, 0u);
        if (n < N && g0 + gi < ngroups) v[gi] = *(const uint4 *)(w + (size_t)n * K + (size_t)(g0 + gi) * G + 8 * l);
    }
#pragma unroll
    for (int gi = 0; gi < GP; ++gi) {
        const int grp = g0 + gi;
        const uint32_t wd[4] = {v[gi].x, v[gi].y, v[gi].z, v[gi].w};
        float e[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // bf16 -> fp32, exact
            e[2 * i] = bits_f32(wd[i] << 16);
            e[2 * i + 1] = bits_f32(wd[i] & 0xffff0000u);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(e[i]));
        // maximum over the row's L lanes: quads, then pairs of quads, then halves
        amax = fmaxf(amax, bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(amax), 0xB1, 0xF, 0xF, true)));  // quad_perm [1,0,3,2]
        amax = fmaxf(amax, bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(amax), 0x4E, 0xF, 0xF, true)));  // quad_perm [2,3,0,1]
        if constexpr (L >= 8)
            amax = fmaxf(amax, bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(amax), 0x141, 0xF, 0xF, true)));  // row_half_mirror
        if constexpr (L >= 16)
            amax = fmaxf(amax, bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(amax), 0x140, 0xF, 0xF, true)));  // row_mirror
        const __half s16 = __float2half_rn(__fdiv_rn(amax, kQmax));
        const float s = __half2float(s16);
        if (l == 0) sc_lds[gi][r] = __half_as_ushort(s16);
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            q[i] = 0;
            if (s > 0.f) {
                const float tq = rintf(__fdiv_rn(e[i], s));
                q[i] = (int)fminf(fmaxf(tq, -kQmax - 1.f), kQmax);
            }
        }
        if constexpr (BITS == 8) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                lo |= ((uint32_t)q[b] & 0xffu) << (8 * b);
                hi |= ((uint32_t)q[4 + b] & 0xffu) << (8 * b);
            }
            if (n < N && grp < ngroups)
                *(uint2 *)((int8_t *)codes + (size_t)n * K + (size_t)grp * G + 8 * l) = make_uint2(lo, hi);
        } else {
            // GPTQ word grp*L + l of column n: nibble b is row 8 * (grp*L + l) + b
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) word |= (uint32_t)(q[b] + 8) << (4 * b);
            words[gi][l][r] = word;
        }
    }
    __syncthreads();
    if (t < 64 && n0 + t < N) {
#pragma unroll
        for (int gi = 0; gi < GP; ++gi)
            if (g0 + gi < ngroups) scales[(size_t)(g0 + gi) * N + n0 + t] = sc_lds[gi][t];
    }
    if constexpr (BITS == 4) {
        // thread t stores word row grp*L + t/64, column n0 + t%64 (blockDim = 64 * L)
        const int kw = t >> 6, c = t & 63;
#pragma unroll
        for (int gi = 0; gi < GP; ++gi)
            if (n0 + c < N && g0 + gi < ngroups)
                ((int32_t *)codes)[((size_t)(g0 + gi) * L + kw) * N + n0 + c] = (int32_t)words[gi][kw][c];
    }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
namespace {
// four tiles per prefetch stage: the vocabulary head (many rounds of small
// workgroups) streams faster with more bytes in flight per wave (M = 1,
// N = 248320: 220 -> 213 us against two tiles)
constexpr int kW8SkinnyDepth = 4;

template <int WAVES, int GS>
hipError_t w8_skinny_launch_w(const SmallPlan &p, const void *x, const int8_t *w, const void *sc,
                              void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    return launch_gemm(w8a16_skinny_kernel<WAVES, kW8SkinnyDepth, GS>, dim3((uint32_t)(N / 16 * p.splits)),
                       dim3(64 * WAVES), skinny_lds_bytes(M, p.S, WAVES), stream, (const uint16_t *)x, w, (const uint16_t *)sc,
                       (uint16_t *)out, ws_counters(ws), (float *)ws_partials(ws), M, (int)N, (int)K,
                       p.splits, p.S);
}

template <int GS>
hipError_t w8_skinny_launch(const SmallPlan &p, const void *x, const int8_t *w, const void *sc,
                            void *out, int M, int64_t N, int64_t K, void *ws, hipStream_t stream) {
    static const int r16 = resident_blocks(w8a16_skinny_kernel<16, kW8SkinnyDepth, GS>, 1024);
    static const int r8 = resident_blocks(w8a16_skinny_kernel<8, kW8SkinnyDepth, GS>, 512);
    const int by_lds = (int)(kLdsPerCu / skinny_lds_bytes(M, p.S, 16));
    switch (pick_waves(N / 16 * p.splits, p.cus, std::min(r16, by_lds), std::min(r8, by_lds))) {
    case 16: return w8_skinny_launch_w<16, GS>(p, x, w, sc, out, M, N, K, ws, stream);
    case 8: return w8_skinny_launch_w<8, GS>(p, x, w, sc, out, M, N, K, ws, stream);
    default: return w8_skinny_launch_w<4, GS>(p, x, w, sc, out, M, N, K, ws, stream);
    }
}

template <int BITS, int GS>
hipError_t rtn_launch(const void *w, void *codes, void *scales, int64_t N, int64_t K, hipStream_t stream) {
    // one workgroup per (64 rows, kRtnGroupsPerWg groups): G/8 lanes per row
    const dim3 grid((uint32_t)((N + 63) / 64), (uint32_t)(((K >> GS) + kRtnGroupsPerWg - 1) / kRtnGroupsPerWg));
    hipLaunchKernelGGL((rtn_quantize_kernel<BITS, GS>), grid, dim3(8 << GS), 0, stream,
                       (const uint16_t *)w, codes, (uint16_t *)scales, (int)N, (int)K);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_w8a16_skinny(const SmallPlan &plan, const void *x, const int8_t *w,
                               const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                               void *workspace, hipStream_t stream) {
    switch (G) {
    case 32: return w8_skinny_launch<5>(plan, x, w, scales, out, M, N, K, workspace, stream);
    case 64: return w8_skinny_launch<6>(plan, x, w, scales, out, M, N, K, workspace, stream);
    case 128: return w8_skinny_launch<7>(plan, x, w, scales, out, M, N, K, workspace, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rtn_quantize(const void *w, int bits, int G, void *codes, void *scales, int64_t N,
                               int64_t K, hipStream_t stream) {
    if (bits == 8) {
        switch (G) {
        case 32: return rtn_launch<8, 5>(w, codes, scales, N, K, stream);
        case 64: return rtn_launch<8, 6>(w, codes, scales, N, K, stream);
        case 128: return rtn_launch<8, 7>(w, codes, scales, N, K, stream);
        default: return hipErrorInvalidValue;
        }
    }
    switch (G) {
    case 32: return rtn_launch<4, 5>(w, codes, scales, N, K, stream);
    case 64: return rtn_launch<4, 6>(w, codes, scales, N, K, stream);
    case 128: return rtn_launch<4, 7>(w, codes, scales, N, K, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace svq
