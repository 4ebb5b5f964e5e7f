/*
 * CPU oracle for the weight-only quantized linear layer  y = x . deq(W)^T.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library. The product path
 * (spec_verify_amd) never links, imports or calls it, and this file shares no
 * code, header, table or constant with the HIP kernels.
 *
 * Everything here is the plain definition written out, with k ascending and no
 * blocking, fusion or reordering:
 *
 *   W4A16 (GPTQ INT4 card "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16", section
 *   "Quantization contract": symmetric INT4, group 128, desc_act off, packed
 *   int32; Eole recipe "Qwen3.8-27B and native MTP speculative decoding",
 *   section "Compressed-tensors INT4 layout": symmetric groups of 32/64/128,
 *   no reordered groups):
 *       q[k][n] = (qweight[k/8][n] >> 4*(k%8)) & 15
 *       w[k][n] = (q[k][n] - 8) * fp16(scales[k/G][n])           (exact in fp32)
 *       y[m][n] = sum_k bf16(x[m][k]) * w[k][n]
 *
 *   MXFP8 (MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp", opening summary,
 *   section "2. Precision plan" and "8. License and attribution": OCP MX,
 *   8-bit elements with an E8M0 scale per 32-element block; K % 32 == 0):
 *       w[n][k] = e4m3(W8[n][k]) * 2^(S8[n][k/32] - 127)         (exact)
 *       y[m][n] = sum_k bf16(x[m][k]) * w[n][k]
 *
 * Two sums are produced for every output: y64, carried in fp64 (every product
 * is exact, so y64 is the exact result up to fp64 rounding of the running sum),
 * and y32, carried in fp32 with k ascending and no fused multiply-add (this
 * file is built with -ffp-contract=off).
 *
 * The repack functions define the device layout of packed INT4 weights used by
 * the GPU path (a tile of 16 columns x 128 K-rows per 1 KiB). They are plain
 * index arithmetic, written here independently of the GPU repack kernel.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- scalar format decoders, from the format definitions ------------------- */

/* bf16 is the upper half of an IEEE binary32 pattern. */
double oracle_bf16_to_f64(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double oracle_fp16_to_f64(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; exponent 0 = subnormal
 * m/8 * 2^-6; S.1111.111 is NaN; no infinities; max 448. */
double oracle_e4m3_to_f64(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* OCP E8M0: unsigned exponent, value 2^(b-127); 255 is NaN. */
double oracle_e8m0_to_f64(uint8_t b) {
    if (b == 255)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays NaN. */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void oracle_bf16_rne_array(const float *in, uint16_t *out, int64_t n) {
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(in[i]);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- W4A16 ------------------------------------------------------------------ */

static int gptq_nibble(const int32_t *qweight, int64_t N, int64_t k, int64_t n) {
    uint32_t word = (uint32_t)qweight[(k >> 3) * N + n];
    return (int)((word >> (4 * (k & 7))) & 15u);
}

/* q[K][N] codes from GPTQ words [K/8][N]. */
void oracle_q4_unpack(const int32_t *qweight, uint8_t *q, int64_t N, int64_t K) {
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            q[k * N + n] = (uint8_t)gptq_nibble(qweight, N, k, n);
}

/* Dequantised column n into wcol[K] (fp64, exact). */
static void w4a16_column(const int32_t *qweight, const uint16_t *scales, int64_t N,
                         int64_t K, int G, int64_t n, double *wcol) {
    for (int64_t k = 0; k < K; ++k) {
        int q = gptq_nibble(qweight, N, k, n);
        double s = oracle_fp16_to_f64(scales[(k / G) * N + n]);
        wcol[k] = (double)(q - 8) * s;
    }
}

static void dot_column(const uint16_t *x, int64_t m, int64_t K, const double *wcol,
                       double *y64, float *y32) {
    double acc = 0.0;
    float acc32 = 0.0f;
    const uint16_t *xr = x + m * K;
    for (int64_t k = 0; k < K; ++k) {
        double a = oracle_bf16_to_f64(xr[k]);
        acc += a * wcol[k];
        /* exact for W4A16 (8 x 14 significant bits) and MXFP8; rounded to
           fp32 for W8A16, whose weights carry up to 19 */
        float p = (float)a * (float)wcol[k];
        acc32 = acc32 + p;
    }
    *y64 = acc;
    *y32 = acc32;
}

/* Full output: y64[M][N], y32[M][N]. Returns 0, or -1 on bad arguments. */
int oracle_w4a16(const uint16_t *x, const int32_t *qweight, const uint16_t *scales,
                 int64_t M, int64_t N, int64_t K, int G, double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || G <= 0 || K % G || K % 8)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                w4a16_column(qweight, scales, N, K, G, n, wcol);
                for (int64_t m = 0; m < M; ++m)
                    dot_column(x, m, K, wcol, &y64[m * N + n], &y32[m * N + n]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

/* Selected outputs (rows[i], cols[i]) only, for large shapes. */
int oracle_w4a16_points(const uint16_t *x, const int32_t *qweight,
                        const uint16_t *scales, int64_t M, int64_t N, int64_t K, int G,
                        const int64_t *rows, const int64_t *cols, int64_t npts,
                        double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || G <= 0 || K % G || K % 8)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < npts; ++i) {
                if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                w4a16_column(qweight, scales, N, K, G, cols[i], wcol);
                dot_column(x, rows[i], K, wcol, &y64[i], &y32[i]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

/* ---- MXFP8 ------------------------------------------------------------------ */

static void mxfp8_column(const uint8_t *w, const uint8_t *scales, int64_t K, int64_t n,
                         double *wcol) {
    for (int64_t k = 0; k < K; ++k)
        wcol[k] = oracle_e4m3_to_f64(w[n * K + k]) *
                  oracle_e8m0_to_f64(scales[n * (K / 32) + k / 32]);
}

int oracle_mxfp8(const uint16_t *x, const uint8_t *w, const uint8_t *scales, int64_t M,
                 int64_t N, int64_t K, double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || K % 32)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                mxfp8_column(w, scales, K, n, wcol);
                for (int64_t m = 0; m < M; ++m)
                    dot_column(x, m, K, wcol, &y64[m * N + n], &y32[m * N + n]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

int oracle_mxfp8_points(const uint16_t *x, const uint8_t *w, const uint8_t *scales,
                        int64_t M, int64_t N, int64_t K, const int64_t *rows,
                        const int64_t *cols, int64_t npts, double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || K % 32)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < npts; ++i) {
                if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                mxfp8_column(w, scales, K, cols[i], wcol);
                dot_column(x, rows[i], K, wcol, &y64[i], &y32[i]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

/* ---- W8A16 (quantized vocabulary head) ------------------------------------- */
/*
 * Eole recipe "Qwen3.8-27B and native MTP speculative decoding", section
 * "Optional vocabulary-head quantization": the dense vocabulary projection is
 * quantized at load time to int8 (or int4) by symmetric group-wise
 * round-to-nearest, groups of 32, 64 or 128 along K. Stored for the GPU path as
 * int8 two's-complement codes [N][K] row-major and fp16 scales [K/G][N]:
 *     w[n][k] = q[n][k] * fp16(scales[k/G][n])      (exact: 8 + 11 significant bits)
 *     y[m][n] = sum_k bf16(x[m][k]) * w[n][k]
 * y64 is exact up to the fp64 running sum; y32 also rounds each product to fp32
 * (a product can carry 8 + 19 significant bits).
 */
static void w8a16_column(const int8_t *w, const uint16_t *scales, int64_t N, int64_t K,
                         int G, int64_t n, double *wcol) {
    for (int64_t k = 0; k < K; ++k)
        wcol[k] = (double)w[n * K + k] * oracle_fp16_to_f64(scales[(k / G) * N + n]);
}

int oracle_w8a16(const uint16_t *x, const int8_t *w, const uint16_t *scales, int64_t M,
                 int64_t N, int64_t K, int G, double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || G <= 0 || K % G)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t n = 0; n < N; ++n) {
                w8a16_column(w, scales, N, K, G, n, wcol);
                for (int64_t m = 0; m < M; ++m)
                    dot_column(x, m, K, wcol, &y64[m * N + n], &y32[m * N + n]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

int oracle_w8a16_points(const uint16_t *x, const int8_t *w, const uint16_t *scales,
                        int64_t M, int64_t N, int64_t K, int G, const int64_t *rows,
                        const int64_t *cols, int64_t npts, double *y64, float *y32) {
    if (M < 0 || N < 0 || K < 0 || G <= 0 || K % G)
        return -1;
    int bad = 0;
#pragma omp parallel
    {
        double *wcol = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wcol) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < npts; ++i) {
                if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                w8a16_column(w, scales, N, K, G, cols[i], wcol);
                dot_column(x, rows[i], K, wcol, &y64[i], &y32[i]);
            }
            free(wcol);
        }
    }
    return bad ? -1 : 0;
}

/* ---- device layout of packed INT4 weights ----------------------------------- */
/*
 * Tiles of 16 columns x 128 K-rows, 1 KiB each, stored column-block-major with
 * the K-tiles of one column block consecutive:
 *     tile (nb, kt) starts at word 256 * (nb * (K/128) + kt).
 * Inside a tile, lane l in 0..63 owns 4 consecutive words (16 bytes):
 *     column   n = 16*nb + (l % 16)
 *     word j (0..3) holds the 8 rows k = 128*kt + 32*(l/16) + 8*j + e, e = 0..7,
 *     with element e stored in nibble slot p where e = (0,2,4,6,1,3,5,7)[p],
 * so that (word >> 4*s) & 0x000F000F puts rows (2s, 2s+1) of the 8 in the two
 * 16-bit halves.
 */
static const int kSlotElem[8] = {0, 2, 4, 6, 1, 3, 5, 7};

static int64_t tiled_word_index(int64_t N, int64_t K, int64_t nb, int64_t kt, int lane,
                                int j) {
    (void)N;
    return ((nb * (K / 128) + kt) * 64 + lane) * 4 + j;
}

int oracle_q4_repack(const int32_t *qweight, int32_t *tiled, int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || N % 16 || K % 128)
        return -1;
    for (int64_t nb = 0; nb < N / 16; ++nb)
        for (int64_t kt = 0; kt < K / 128; ++kt)
            for (int lane = 0; lane < 64; ++lane)
                for (int j = 0; j < 4; ++j) {
                    int64_t n = 16 * nb + lane % 16;
                    uint32_t word = 0;
                    for (int p = 0; p < 8; ++p) {
                        int64_t k = 128 * kt + 32 * (lane / 16) + 8 * j + kSlotElem[p];
                        word |= (uint32_t)gptq_nibble(qweight, N, k, n) << (4 * p);
                    }
                    tiled[tiled_word_index(N, K, nb, kt, lane, j)] = (int32_t)word;
                }
    return 0;
}

int oracle_q4_unrepack(const int32_t *tiled, int32_t *qweight, int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || N % 16 || K % 128)
        return -1;
    memset(qweight, 0, sizeof(int32_t) * (size_t)(K / 8) * (size_t)N);
    for (int64_t nb = 0; nb < N / 16; ++nb)
        for (int64_t kt = 0; kt < K / 128; ++kt)
            for (int lane = 0; lane < 64; ++lane)
                for (int j = 0; j < 4; ++j) {
                    int64_t n = 16 * nb + lane % 16;
                    uint32_t word = (uint32_t)tiled[tiled_word_index(N, K, nb, kt, lane, j)];
                    for (int p = 0; p < 8; ++p) {
                        int64_t k = 128 * kt + 32 * (lane / 16) + 8 * j + kSlotElem[p];
                        uint32_t q = (word >> (4 * p)) & 15u;
                        uint32_t *dst = (uint32_t *)&qweight[(k >> 3) * N + n];
                        *dst |= q << (4 * (k & 7));
                    }
                }
    return 0;
}
