// Internal launch interface between the C ABI (svq_api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "svq_device.h"

namespace svq {

// Launch shape of a GEMM call (grid and workgroup size, dynamic LDS of its
// first, main launch; the number of launches). A launch query sets the calling
// thread's capture slot: the GEMM launchers then record their shape there
// instead of launching.
struct LaunchShape {
    uint64_t grid;
    uint32_t threads;
    size_t lds;
    int launches;
};
LaunchShape *&capture_slot();  // this thread's slot (null: launch normally)

template <typename F, typename... Args>
hipError_t launch_gemm(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream, Args... args) {
    if (LaunchShape *c = capture_slot()) {
        if (c->launches++ == 0) {  // the first launch is the call's main kernel
            c->grid = (uint64_t)grid.x * grid.y * grid.z;
            c->threads = block.x * block.y * block.z;
            c->lds = lds;
        }
        return hipSuccess;
    }
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
    return hipGetLastError();
}

// Read-only stream of `bytes` (a multiple of 16) in `grid` workgroups of
// `threads` threads; sink holds `grid` words.
hipError_t launch_stream_probe(const void *src, size_t bytes, uint32_t grid, uint32_t threads, uint32_t *sink,
                               hipStream_t stream);
// `per_wave` bf16 16x16x32 MFMAs (a multiple of 8) per wave of (grid, threads);
// sink holds `grid` floats.
hipError_t launch_mfma_probe(uint32_t grid, uint32_t threads, uint32_t per_wave, int random, float *sink,
                             hipStream_t stream);

hipError_t launch_q4_repack(const int32_t *src, int32_t *dst, int64_t N, int64_t K,
                            hipStream_t stream);
hipError_t launch_mxfp8_tile(const uint8_t *src, uint8_t *dst, int64_t N, int64_t K, hipStream_t stream);

// Setup-time projection fusion (bits 4: GPTQ words -> fused tiles; bits 8: int8
// codes [N_p][K] -> [sum N_p][K]) and fp16 scale concatenation, one launch.
constexpr int kMaxFuseParts = 16;
hipError_t launch_fuse_pack(int bits, const void *const *w, const void *const *s,
                            const int64_t *widths, int parts, int64_t K, int G, void *dst_w,
                            void *dst_s, hipStream_t stream);
// Compressed-tensors [N][K/8] words and [N][K/G] scales -> GPTQ [K/8][N], [K/G][N].
hipError_t launch_ct_to_gptq(const int32_t *wp, const void *ws, int32_t *qw, void *s, int64_t N,
                             int64_t K, int G, hipStream_t stream);

// Stream-K schedule of the wide MFMA kernels: output tiles of bm x bn, `units`
// = row_tiles * col_tiles * (K/128) (tile, 128-row step) pairs split evenly over
// `grid` persistent workgroups; a workgroup touches at most `maxt` tiles.
struct WidePlan {
    int bm, bn;
    int row_tiles, col_tiles;
    int64_t units;
    int grid;
    int maxt;
    size_t workspace_bytes;  // counter region + fp32 partials (0 if no tile is shared)
};

WidePlan plan_w4a16_wide(int64_t M, int64_t N, int64_t K, int num_cus);
WidePlan plan_mxfp8_wide(int64_t M, int64_t N, int64_t K, int num_cus);

// Schedule of the small-M kernels: each 16-column block's K range is cut into
// `splits` ranges of S 128-row tiles (1 unless the matrix has too few column
// blocks to occupy the chip). Each launcher maps (block, range) pairs to
// workgroups and picks their size: the dot2 kernels one pair per workgroup
// with the largest of 16, 8 or 4 waves for which the whole grid is resident on
// `cus` compute units; the narrow kernel 4-column units over all of K; the
// skinny kernels one or more blocks per workgroup (see their launchers).
struct SmallPlan {
    int splits, S, cus;
    size_t workspace_bytes;  // arrival counters + fp32 partials (0 if splits == 1)
};

// LDS of one compute unit, and the most a skinny workgroup may take for its
// stage of x (M rows x 128*S bf16, rows padded by 16 bytes).
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr size_t kSkinnyLdsMax = 64 * 1024;
inline size_t skinny_lds_bytes(int M, int S, int waves) {
    const size_t stage = (size_t)M * ((size_t)S * 256 + 16);
    const size_t red = (size_t)waves * M * 16 * 4;
    return stage > red ? stage : red;
}
// Largest K range (in 128-row tiles) whose x stage fits kSkinnyLdsMax.
inline int64_t skinny_max_tiles(int64_t M) {
    return ((int64_t)kSkinnyLdsMax / M - 16) / 256;
}

// Workgroups of `threads` threads of `kernel` that fit on one CU at once.
template <typename F>
int resident_blocks(F kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess) return 1;
    return n > 0 ? n : 1;
}

// Waves per workgroup for `wgs` workgroups given the resident counts of the 16-
// and 8-wave instantiations.
inline int pick_waves(int64_t wgs, int cus, int res16, int res8) {
    if (wgs <= (int64_t)res16 * cus) return 16;
    if (wgs <= (int64_t)res8 * cus) return 8;
    return 4;
}

// max_tiles: the most K tiles one workgroup may take (0: no limit).
SmallPlan plan_smallm(int64_t M, int64_t N, int64_t K, int num_cus, int64_t max_tiles = 0);

// True when launch_w4a16_dot2 runs the narrow-unit GEMV for this shape (too
// few 16-column blocks to fill the chip, M <= 2) rather than the block kernel.
bool w4a16_dot2_is_narrow(const SmallPlan &plan, int M, int64_t N, int64_t K, int G);
hipError_t launch_w4a16_dot2(const SmallPlan &plan, const void *x, const int32_t *wt,
                             const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                             void *workspace, hipStream_t stream);
hipError_t launch_w4a16_skinny(const SmallPlan &plan, const void *x, const int32_t *wt,
                               const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                               void *workspace, hipStream_t stream);
hipError_t launch_w4a16_wide(const WidePlan &plan, const void *x, const int32_t *wt,
                             const void *scales, void *out, int64_t M, int64_t N, int64_t K,
                             int G, void *workspace, hipStream_t stream);

hipError_t launch_mxfp8_dot2(const SmallPlan &plan, const void *x, const uint8_t *w,
                             const uint8_t *scales, void *out, int M, int64_t N, int64_t K,
                             void *workspace, hipStream_t stream);
hipError_t launch_mxfp8_skinny(const SmallPlan &plan, const void *x, const uint8_t *w,
                               const uint8_t *scales, void *out, int M, int64_t N, int64_t K,
                               void *workspace, hipStream_t stream);

hipError_t launch_w8a16_skinny(const SmallPlan &plan, const void *x, const int8_t *w,
                               const void *scales, void *out, int M, int64_t N, int64_t K, int G,
                               void *workspace, hipStream_t stream);
hipError_t launch_mxfp8_quantize(const void *w, int optimized, uint8_t *codes, uint8_t *scales,
                                 int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_rtn_quantize(const void *w, int bits, int G, void *codes, void *scales, int64_t N,
                               int64_t K, hipStream_t stream);

// Workspace layout shared by every kernel that splits work across workgroups:
// a fixed region of arrival counters (which every kernel leaves at zero) then
// the fp32 partials. The counter region has the same size for all kernels so
// that one kernel's partials never land on another kernel's counters when
// callers reuse one workspace.
constexpr size_t kCounterBytes = 256 * 1024;
constexpr size_t kMaxCounters = kCounterBytes / 4;
inline uint32_t *ws_counters(void *ws) { return (uint32_t *)ws; }
inline void *ws_partials(void *ws) { return ws ? (void *)((char *)ws + kCounterBytes) : nullptr; }
hipError_t launch_mxfp8_wide(const WidePlan &plan, const void *x, const uint8_t *w,
                             const uint8_t *scales, void *out, int64_t M, int64_t N, int64_t K,
                             void *workspace, hipStream_t stream);

}  // namespace svq
