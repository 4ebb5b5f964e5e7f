/*
 * svq.h -- C ABI of the weight-only quantized linear layer for decode and
 * speculative-verify shapes on AMD Instinct MI355X (gfx950).
 *
 *   y[M][N] = x[M][K] . deq(W)^T     (bf16 x, fp32 accumulation, bf16 y)
 *
 * Two weight formats:
 *  - W4A16: symmetric INT4 with zero point 8, one fp16 scale per group of G
 *    K-rows (G = 32, 64 or 128), GPTQ words packed 8 per int32 along K, no
 *    group reordering. GPTQ INT4 card "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16",
 *    section "Quantization contract"; Eole recipe "Qwen3.8-27B and native MTP
 *    speculative decoding", section "Compressed-tensors INT4 layout".
 *  - MXFP8: OCP E4M3FN elements with one E8M0 scale per 32 K-elements. MXFP8
 *    card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp", opening summary, sections
 *    "2. Precision plan" (N >= 128, K % 32 == 0) and "8. License and
 *    attribution" (OCP MX, E8M0 scale per 32-element block).
 *  - W8A16, the quantized vocabulary head: symmetric int8 codes with one fp16
 *    scale per group of G K-rows, produced at load time from the dense bf16
 *    projection by svq_rtn_quantize (which also produces W4A16 weights). Eole
 *    recipe, section "Optional vocabulary-head quantization".
 *
 * M is the number of tokens verified per call: streams x (1 + draft tokens)
 * (Eole recipe, opening paragraph: the main model verifies a chunk of drafted
 * tokens). Packed INT4 weights are repacked once at setup, as the Eole recipe's
 * section "Pack inference projections" does before its own GEMM kernel runs.
 *
 * Conventions for every entry point:
 *  - All buffer pointers are DEVICE pointers to memory the caller owns. The
 *    library keeps no pointer after returning and allocates, frees and
 *    synchronizes nothing.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *    is enqueued asynchronously on it; buffers must stay alive until it runs.
 *  - Every argument is checked on the host BEFORE anything is enqueued. On any
 *    error nothing is launched and outputs are left untouched. Unsupported
 *    formats (asymmetric weights, zero points, group reordering, activation
 *    quantization) cannot be expressed: there are no such parameters.
 *  - Row-major everywhere; bf16 and fp16 values are passed as their 16-bit
 *    patterns.
 *  - GEMM operands stay below 2 GiB each (M*K*2, N*K, M*N*2 < 2^31 bytes;
 *    the kernels use 32-bit buffer offsets); larger shapes return
 *    SVQ_ERR_DIM.
 *  - Results are deterministic: repeated calls with equal inputs give equal
 *    bits (all reductions run in a fixed order).
 */
#ifndef SVQ_H
#define SVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVQ_ABI_VERSION 1

typedef enum svq_status {
    SVQ_OK = 0,
    SVQ_ERR_NULL = 1,          /* a required pointer is NULL */
    SVQ_ERR_DIM = 2,           /* M, N or K out of range (<= 0 or too large) */
    SVQ_ERR_GROUP = 3,         /* group size not supported for this format */
    SVQ_ERR_DIVISIBILITY = 4,  /* N % 16 != 0, K % 128 != 0 or K % G != 0 */
    SVQ_ERR_MXFP8_SHAPE = 5,   /* MXFP8 needs N >= 128 and K % 32 == 0 */
    SVQ_ERR_ALIGN = 6,         /* a pointer is not suitably aligned */
    SVQ_ERR_OVERLAP = 7,       /* output overlaps an input */
    SVQ_ERR_WORKSPACE = 8,     /* workspace missing, too small or misaligned */
    SVQ_ERR_HIP = 9,           /* the HIP runtime refused the launch */
    SVQ_ERR_UNSUPPORTED = 10   /* the requested kernel cannot run this shape */
} svq_status;

/* Kernel selectors for the *_with entry points (diagnostics and benchmarks).
 * SVQ_KERNEL_AUTO is what svq_w4a16_gemm / svq_mxfp8_gemm use. */
typedef enum svq_kernel {
    SVQ_KERNEL_AUTO = 0,
    SVQ_KERNEL_DOT2 = 1,        /* VALU bf16 dot2, M <= 8: 16-column blocks with row
                                   broadcast of x; for M <= 2 and fewer 16-column
                                   blocks than CUs, 4-column units with x in LDS */
    SVQ_KERNEL_MFMA_SKINNY = 2, /* one 16-row MFMA tile, waves split K, M <= 16 */
    SVQ_KERNEL_MFMA_WIDE = 3    /* LDS-staged x, 64/128-row MFMA tiles, split-K, any M */
} svq_kernel;

/* Operations, for the format-generic queries svq_workspace_bytes and
 * svq_kernel_name. */
typedef enum svq_op {
    SVQ_OP_W4A16 = 1,  /* svq_w4a16_gemm */
    SVQ_OP_MXFP8 = 2,  /* svq_mxfp8_gemm (group_size must be 32) */
    SVQ_OP_W8A16 = 3   /* svq_w8a16_gemm */
} svq_op;

int svq_abi_version(void);

/* Static text for a status code; never NULL. */
const char *svq_status_string(int status);

/* ---- W4A16 ------------------------------------------------------------------ */

/* Bytes of the repacked weight buffer: K*N/2 (the same as the GPTQ input). */
size_t svq_q4_repacked_bytes(int64_t N, int64_t K);

/*
 * One-time repack of GPTQ INT4 words into the device tile layout read by the
 * W4A16 kernels (a pure bit permutation; reads and writes K*N/2 bytes once).
 *   qweight_gptq  int32 [K/8][N]; nibble i (bits 4i..4i+3) of word [j][n] is
 *                 the code of row 8j+i, column n. 16-byte aligned.
 *   qweight_tiled int32, svq_q4_repacked_bytes(N, K) bytes, 16-byte aligned,
 *                 must not overlap qweight_gptq. Layout: tiles of 16 columns x
 *                 128 rows (1 KiB), column-block-major with the K-tiles of a
 *                 column block consecutive; lane l of a tile owns 16 bytes:
 *                 column 16*nb + l%16, word j = rows 128*kt + 32*(l/16) + 8*j
 *                 + e (e = 0..7) with row e in nibble slot p, e = (0,2,4,6,
 *                 1,3,5,7)[p].
 * Requires N % 16 == 0, K % 128 == 0.
 */
int svq_q4_repack(const int32_t *qweight_gptq, int32_t *qweight_tiled, int64_t N,
                  int64_t K, void *stream);

/* Most projections svq_fuse_projections takes in one call. */
#define SVQ_MAX_FUSED_PARTS 16

/*
 * Setup-time projection fusion: `parts` quantized projections that read the
 * same x (same K, same format, same group size) become one projection whose
 * output columns are the parts' columns in the order given, so a single GEMM
 * call replaces `parts` calls and y_fused = [y_0 | y_1 | ...] (Eole recipe
 * "Qwen3.8-27B and native MTP speculative decoding", section "Pack inference
 * projections": K/V/Q and gate/up are packed at setup, before the repack, with
 * no requantization; projections that do not fit stay separate -- here the
 * call returns an error and changes nothing, and the caller keeps them).
 *   bits 4: weights[p]   GPTQ int32 words [K/8][widths[p]], 4-byte aligned;
 *           weight_fused the REPACKED fused weight (the svq_q4_repack layout of
 *                        the concatenated words), K*N/2 bytes, 16-byte aligned,
 *                        ready for svq_w4a16_gemm with N = sum of widths
 *   bits 8: weights[p]   int8 codes [widths[p]][K], 16-byte aligned;
 *           weight_fused int8 [N][K], 16-byte aligned (svq_w8a16_gemm input)
 *   scales[p]     fp16 [K/G][widths[p]], 2-byte aligned
 *   scales_fused  fp16 [K/G][N]; 4-byte aligned if it feeds a GEMM
 *   weights, scales, widths: host arrays of `parts` entries (device pointers
 *   and column counts), 1 <= parts <= SVQ_MAX_FUSED_PARTS, read during the
 *   call only. Requires every width % 16 == 0, K % 128 == 0, G in {32, 64,
 *   128}, K % G == 0. The outputs must not overlap any input or each other
 *   (inputs may overlap one another). Reads and writes every byte once, in one
 *   launch.
 */
int svq_fuse_projections(int32_t bits, const void *const *weights, const void *const *scales,
                         const int64_t *widths, int32_t parts, int64_t K, int32_t group_size,
                         void *weight_fused, void *scales_fused, void *stream);

/*
 * Compressed-tensors W4A16 ingest: words [N][K/8] and scales [N][K/G] become
 * the GPTQ layout [K/8][N] and [K/G][N] by transposition, every word and scale
 * unchanged (Eole recipe, section "Compressed-tensors INT4 layout": the
 * converter transposes packed words and scales and does not requantize). The
 * nibble order is the GPTQ one: nibble i of word [n][j] is the code of row
 * 8j + i of column n.
 *   weight_packed int32 [N][K/8], 4-byte aligned
 *   weight_scale  fp16 [N][K/G], 2-byte aligned
 *   qweight       int32 [K/8][N], 4-byte aligned (the svq_q4_repack input)
 *   scales        fp16 [K/G][N], 2-byte aligned
 *   group_size    G in {32, 64, 128}; K % G == 0 (any N >= 1)
 * Outputs must not overlap the inputs or each other. Words and scales are
 * transposed in one launch.
 */
int svq_ct_to_gptq(const int32_t *weight_packed, const void *weight_scale, int32_t *qweight,
                   void *scales, int64_t N, int64_t K, int32_t group_size, void *stream);

/* Workspace bytes needed by svq_w4a16_gemm (kernel = SVQ_KERNEL_AUTO) or by
 * svq_w4a16_gemm_with for the given kernel; 0 if none. (size_t)-1 if the
 * arguments are invalid or the kernel cannot run the shape. */
size_t svq_w4a16_workspace_bytes(int kernel, int64_t M, int64_t N, int64_t K,
                                 int32_t group_size);

/*
 * y = x . ((q - 8) * s)^T, the W4A16 linear layer: symmetric INT4 with zero
 * point 8, one fp16 scale per group of G K-rows, no group reordering (GPTQ
 * INT4 card "Qwen3.8-27B-GPTQ-Int4-sym-G128-MTP-BF16", section "Quantization
 * contract": INT4, symmetric, group 128, desc_act off, packed int32; Eole
 * recipe, section "Compressed-tensors INT4 layout": groups of 32, 64 or 128).
 * Products are accumulated in fp32 and y is rounded to bf16 (nearest even).
 *   x             bf16 [M][K], 16-byte aligned
 *   qweight_tiled output of svq_q4_repack, 16-byte aligned
 *   scales        fp16 [K/G][N], 4-byte aligned (read as aligned 32-bit words)
 *   out           bf16 [M][N], 4-byte aligned, fully overwritten, must not
 *                 overlap any input or the workspace
 *   group_size    G in {32, 64, 128}; K % 128 == 0, N % 16 == 0
 *   workspace     device buffer of at least svq_w4a16_workspace_bytes(...)
 *                 bytes, 256-byte aligned, ZERO-FILLED before its first use;
 *                 the kernels leave it zero-filled again where it matters
 *                 (split-K arrival counters). NULL/0 when 0 bytes are needed.
 *                 Calls that share a workspace must be stream-ordered.
 */
int svq_w4a16_gemm(const void *x, const int32_t *qweight_tiled, const void *scales,
                   void *out, int64_t M, int64_t N, int64_t K, int32_t group_size,
                   void *workspace, size_t workspace_bytes, void *stream);

/* Same, with an explicit kernel choice; SVQ_ERR_UNSUPPORTED if that kernel
 * cannot run M (SVQ_KERNEL_DOT2: M <= 8; SVQ_KERNEL_MFMA_SKINNY: M <= 16). */
int svq_w4a16_gemm_with(int kernel, const void *x, const int32_t *qweight_tiled,
                        const void *scales, void *out, int64_t M, int64_t N, int64_t K,
                        int32_t group_size, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Name of the kernel the call would launch (static text), or NULL if invalid. */
const char *svq_w4a16_kernel_name(int kernel, int64_t M, int64_t N, int64_t K,
                                  int32_t group_size);

/* Size of the device scratch array svq_w4a16_gemm_noalloc uses on each device:
 * the 256 KiB counter region plus 32 MiB of fp32 partials. */
#define SVQ_NOALLOC_SCRATCH_BYTES ((size_t)(32u << 20) + (size_t)(256u << 10))

/*
 * svq_w4a16_gemm without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments, results and errors as
 * svq_w4a16_gemm with the automatic kernel choice (identical bits: the same
 * kernels run); the cross-workgroup reductions use a file-scope device array
 * of SVQ_NOALLOC_SCRATCH_BYTES that each device holds until the process ends.
 * It allocates nothing (no hipMalloc, hipFree or allocating library call).
 * Shapes whose workspace (svq_w4a16_workspace_bytes) exceeds the array return
 * SVQ_ERR_WORKSPACE before anything is enqueued. The first call on a device
 * looks the array up and enqueues one small fill kernel on `stream` that
 * clears its counter region. All calls on one device share the array and each
 * call leaves it as the last call wrote it: calls that overlap in time on one
 * device race and must be ordered by the caller (one stream, or events).
 */
int svq_w4a16_gemm_noalloc(const void *x, const int32_t *qweight_tiled, const void *scales,
                           void *out, int64_t M, int64_t N, int64_t K, int32_t group_size,
                           void *stream);

/* ---- MXFP8 ------------------------------------------------------------------ */

/*
 * One-time repack of E4M3 codes into the device tile layout read by the MXFP8
 * GEMM kernels (a byte permutation; reads and writes N*K bytes once; the
 * pages repack weights once at setup, Eole recipe "Qwen3.8-27B and native MTP
 * speculative decoding", section "Pack inference projections").
 *   w        E4M3FN codes [N][K] (row n holds the K elements of output column
 *            n), 16-byte aligned
 *   w_tiled  N*K bytes, 16-byte aligned, must not overlap w. Layout: tiles of
 *            16 columns x 128 K-elements (2 KiB), column-block-major with the
 *            K-tiles of a block consecutive (tile (nb, kt) at byte
 *            2048*(nb*K/128 + kt)); byte 1024*h + 16*l + b of a tile holds
 *            column 16*nb + l%16, K-element 128*kt + 32*(l/16) + 16*h + b.
 * Requires N % 16 == 0, K % 128 == 0. The E8M0 scales keep their [N][K/32]
 * layout.
 */
int svq_mxfp8_repack(const uint8_t *w, uint8_t *w_tiled, int64_t N, int64_t K, void *stream);

size_t svq_mxfp8_workspace_bytes(int kernel, int64_t M, int64_t N, int64_t K);

/*
 * y = x . (e4m3(w) * 2^(e8m0(s) - 127))^T, the MXFP8 linear layer: OCP E4M3FN
 * elements with one E8M0 power-of-two scale per 32 consecutive K-elements
 * (MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp", opening summary and
 * section "8. License and attribution"); the kernel constraints N >= 128 and
 * K % 32 == 0 of its section "2. Precision plan" are checked and reported as
 * SVQ_ERR_MXFP8_SHAPE (its section "7. Known issues and caveats" records a
 * crash at N = 96). fp32 accumulation, bf16 (nearest even) output.
 *   x       bf16 [M][K], 16-byte aligned
 *   w       E4M3FN codes in the svq_mxfp8_repack tile layout (N*K bytes),
 *           16-byte aligned
 *   scales  E8M0 codes [N][K/32], one per 32 consecutive K-elements of a row,
 *           4-byte aligned (read as aligned 32-bit words)
 *   out     bf16 [M][N], 4-byte aligned, fully overwritten, no overlap
 *   group_size must be 32. Requires N >= 128, N % 16 == 0, K % 128 == 0.
 *   workspace as for svq_w4a16_gemm.
 * Element code 0x7F/0xFF (NaN) and scale code 255 (NaN) are not supported
 * inputs: the result for them is unspecified.
 */
int svq_mxfp8_gemm(const void *x, const uint8_t *w, const uint8_t *scales, void *out,
                   int64_t M, int64_t N, int64_t K, int32_t group_size, void *workspace,
                   size_t workspace_bytes, void *stream);

int svq_mxfp8_gemm_with(int kernel, const void *x, const uint8_t *w, const uint8_t *scales,
                        void *out, int64_t M, int64_t N, int64_t K, int32_t group_size,
                        void *workspace, size_t workspace_bytes, void *stream);

const char *svq_mxfp8_kernel_name(int kernel, int64_t M, int64_t N, int64_t K);

/*
 * MXFP8 quantization of a dense bf16 projection into the svq_mxfp8_gemm input,
 * as a model is quantized (MXFP8 card "Qwen3.8-27B-MXFP8-CT-AutoRound-mtp":
 * plain round-to-nearest, opening summary; the optimized round-to-nearest of
 * its notes on the quantizer, which evaluates the baseline block scale with
 * the scales twice and half as large and keeps the best). Per block of 32
 * consecutive K-elements of row n:
 *   baseline  X0 = floor(log2 amax) - 8, b0 = clamp(X0 + 127, 0, 254); an
 *             all-zero block takes b0 = 127
 *   candidate b: codes E4M3_RNE(|v| / 2^(b-127)) with the sign of v (-0 and
 *             negatives that round to zero give 0x80), saturating at 448;
 *             score = sum over the block, in ascending order, of fp32
 *             (v - decoded)^2 with round-to-nearest subtract, multiply, add
 *   optimized = 1: candidates b0, b0 + 1, b0 - 1 (those in 0..254); a later
 *             one is kept only with a strictly smaller score. optimized = 0:
 *             b0 (plain round-to-nearest).
 *   w       bf16 [N][K] (row n = output column n), 16-byte aligned, finite
 *   codes   E4M3FN [N][K], 16-byte aligned
 *   scales  E8M0 [N][K/32]
 * Requires K % 32 == 0 (svq_mxfp8_gemm further needs N >= 128, K % 128 == 0).
 * Outputs must not overlap w or each other. optimized outside {0, 1} returns
 * SVQ_ERR_UNSUPPORTED.
 */
int svq_mxfp8_quantize(const void *w, int32_t optimized, uint8_t *codes, uint8_t *scales, int64_t N,
                       int64_t K, void *stream);

/* ---- quantized vocabulary head (W8A16) and the load-time quantizer --------- */

/*
 * Symmetric group-wise round-to-nearest quantization of a dense projection,
 * done once when the model loads (Eole recipe, section "Optional
 * vocabulary-head quantization": int8 or int4, groups of 32, 64 or 128 along
 * K, symmetric, round to nearest). Per group of G consecutive K-elements of
 * row n, in fp32 with IEEE division:
 *     amax = max |w|,  s = fp16_rne(amax / qmax),  qmax = 127 (int8) or 7 (int4)
 *     q    = clamp(rint(w / s), -qmax - 1, qmax)   (rint: nearest, ties to even)
 * with s used as stored; a group whose stored s is 0 gets q = 0.
 *   w           bf16 [N][K] (row n = output column n), 16-byte aligned; finite values
 *   bits        8: codes = int8 [N][K] (two's complement), 16-byte aligned
 *               4: codes = GPTQ int32 words [K/8][N] holding q + 8, the W4A16
 *                  input of svq_q4_repack; 4-byte aligned
 *   scales      fp16 [K/G][N], 2-byte aligned
 *   group_size  G in {32, 64, 128}; K % G == 0
 * codes and scales must not overlap w or each other. Errors as for the GEMMs.
 */
int svq_rtn_quantize(const void *w, int32_t bits, int32_t group_size, void *codes, void *scales,
                     int64_t N, int64_t K, void *stream);

/* Workspace bytes needed by svq_w8a16_gemm; 0 if none, (size_t)-1 if invalid. */
size_t svq_w8a16_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t group_size);

/*
 * y = x . (q * s)^T for the int8 codes of svq_rtn_quantize, M <= 16
 * (SVQ_ERR_UNSUPPORTED above): the quantized vocabulary head (Eole recipe,
 * section "Optional vocabulary-head quantization"; the AWQ card
 * "Qwen3.8-27B-AWQ-INT4-MTP-LowLatency" measures the decode-latency gain of
 * a quantized head in its head-precision section). fp32 accumulation, bf16
 * (nearest even) output.
 *   x       bf16 [M][K], 16-byte aligned
 *   w       int8 codes [N][K], 16-byte aligned
 *   scales  fp16 [K/G][N], 4-byte aligned (read as aligned 32-bit words)
 *   out     bf16 [M][N], 4-byte aligned, fully overwritten, no overlap
 *   group_size G in {32, 64, 128}; K % 128 == 0, N % 16 == 0
 *   workspace as for svq_w4a16_gemm.
 */
int svq_w8a16_gemm(const void *x, const int8_t *w, const void *scales, void *out, int64_t M,
                   int64_t N, int64_t K, int32_t group_size, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Name of the kernel svq_w8a16_gemm would launch (static text), or NULL. */
const char *svq_w8a16_kernel_name(int64_t M, int64_t N, int64_t K, int32_t group_size);

/* ---- format-generic queries ---------------------------------------------------- */

/* Workspace bytes the GEMM of `op` (an svq_op) needs with its automatic kernel
 * choice: svq_w4a16_workspace_bytes(SVQ_KERNEL_AUTO, ...),
 * svq_mxfp8_workspace_bytes(SVQ_KERNEL_AUTO, ...) (group_size must be 32) or
 * svq_w8a16_workspace_bytes(...). (size_t)-1 for an unknown op or invalid
 * arguments. */
size_t svq_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int32_t group_size);

/* Name of the kernel the GEMM of `op` would launch for this shape (static
 * text), or NULL for an unknown op or invalid arguments. */
const char *svq_kernel_name(int op, int64_t M, int64_t N, int64_t K, int32_t group_size);

/* ---- measurement ---------------------------------------------------------------- */

/*
 * Launch shape of a GEMM call: the grid (workgroups), workgroup size (threads)
 * and dynamic LDS bytes the call would launch with, for op (an svq_op) and
 * kernel (an svq_kernel; SVQ_KERNEL_AUTO only for SVQ_OP_W8A16). Nothing is
 * launched. Returns the status the call would return for valid buffers.
 */
int svq_launch_geometry(int op, int kernel, int64_t M, int64_t N, int64_t K, int32_t group_size,
                        uint64_t *grid, uint32_t *threads, size_t *lds_bytes);

/*
 * Streaming probe: reads `bytes` (a non-zero multiple of 16) from src (16-byte
 * aligned) in `grid` workgroups of `threads` threads (a multiple of 64, at most
 * 1024), each workgroup one contiguous share, and does nothing with them. It
 * measures the bandwidth a plain read of that many bytes reaches in that
 * launch shape: the ceiling of a GEMM's weight stream. sink (grid words, 4-byte
 * aligned) may be written with data-dependent values; nothing else is.
 */
int svq_stream_probe(const void *src, size_t bytes, uint32_t grid, uint32_t threads, uint32_t *sink,
                     void *stream);

/*
 * Matrix-core probe: every wave of `grid` workgroups of `threads` threads (a
 * multiple of 64, at most 1024) issues `per_wave` bf16 16x16x32 MFMAs (a
 * non-zero multiple of 8, at most 2^24) as eight independent chains on
 * register operands, with no memory traffic: the floor that MFMA issue sets
 * for a kernel doing that many MFMAs per wave in that launch shape (the
 * compute-bound batched-verify case of the autobench page "Qwen3.8-27B · vLLM ·
 * FP8 + MTP"). operands: 0 = constant (one small value in every register: the
 * issue floor at the clock the chip holds when the multipliers' inputs never
 * change), 1 = random (per chain: A random bf16 like activations, B the bf16 of
 * 128 + q for random nibbles q, the W4A16 weight operand; the matrix cores'
 * power draw then lowers the shader clock as real data does); anything else
 * is SVQ_ERR_DIM. sink (grid floats, 4-byte aligned) may be written with
 * data-dependent values; nothing else is.
 */
int svq_mfma_probe(uint32_t grid, uint32_t threads, uint32_t per_wave, int32_t operands, float *sink,
                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SVQ_H */
