// Cross-workgroup reductions shared by the kernels that split work.
//
// Small-M kernels (a few K splits of a column block): handoff without fences.
// An agent-scope release/acquire fence on gfx950 writes back / invalidates the
// XCD-local L2 caches and costs tens of microseconds per workgroup when
// hundreds of workgroups do it, so partials travel with agent-coherent atomic
// stores and loads instead. A contributor stores its partial, waits until its
// stores have completed (s_waitcnt), and only then bumps the arrival counter
// with an agent-scope atomic; the workgroup that observes the final count reads
// the other partials. Partials are added in a fixed order, so results are
// deterministic, and the last arriver clears the counter.
//
// Wide kernels (M > 16): a second launch sums the partials (below).
#pragma once

#include "svq_device.h"
#include "svq_launch.h"

namespace svq {

// Wait until every outstanding memory access of this wave has completed.
__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ uint32_t arrive(uint32_t *cnt) {
    return __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_counter(uint32_t *cnt) {
    __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Stream-K: the (output tile, 128-row K step) units are split evenly over
// `grid` persistent workgroups: workgroup w owns [w*units/grid, (w+1)*units/grid).
// The workgroup whose unit range holds unit a (units >= grid >= 1).
__device__ __forceinline__ int sk_owner(int64_t a, int64_t units, int grid) {
    const int64_t w = ((a + 1) * grid - 1) / units;
    return (int)(w < grid - 1 ? w : grid - 1);
}

__device__ __forceinline__ int sk_first_tile(int w, int64_t units, int grid, int KT) {
    return (int)(((int64_t)w * units / grid) / KT);
}

// ---- split-K of the wide MFMA kernels: partials summed by a second launch ----
//
// A wide kernel's workgroup holds NV f32x4 accumulators per thread (NT threads)
// for each output tile it works on: accumulator v of thread (wave, lane) holds
// rows 16*(wr*MBW + v/CT) + 4*(lane/16) + i (i = 0..3) and column
// 16*(wc*CT + v%CT) + lane%16 of the tile, where wave = wr*WC + wc. A tile that
// one workgroup computes over all of K is written as bf16 by the wide kernel;
// for a tile whose K steps are split over several workgroups, each writes its
// fp32 partial with plain stores into its slot of the workspace
// ([workgroup][slot][v][thread], slot = the tile's index among the workgroup's
// tiles), and wide_sum_kernel, launched next on the same stream, adds the
// partials in contributor (workgroup) order and writes bf16. The launch
// boundary orders every partial's stores before its loads: nothing is
// exchanged between workgroups of one launch, no coherent memory traffic or
// arrival counter is needed, and no workgroup waits for another.
template <int NV, int NT>
__device__ __forceinline__ f32x4 *wide_partial(f32x4 *part, int wg, int maxt, int slot) {
    return part + ((size_t)wg * maxt + slot) * NV * NT;
}

// Workgroup (tile, pair) of grid row_tiles * col_tiles * NV / 2: accumulators
// 2*pair and 2*pair + 1 of every thread, summed over the tile's contributors.
// The contributors' unit ranges are consecutive and every one after the first
// starts inside the tile (its partial is in its slot 0); only the first may
// have begun in an earlier tile. Two to four contributors (the usual split)
// take one pass with exactly their loads in flight; more go eight at a time,
// with the loads past the last one clamped to it (no load behind a branch).
template <int NV, int NT>
struct WideSum {
    const f32x4 *p;  // part + thread
    size_t stride;   // f32x4 per workgroup
    int fw, slot_fw, v0;
    __device__ __forceinline__ const f32x4 *at(int w, int j) const {
        return p + (size_t)w * stride + (w == fw ? (size_t)slot_fw * NV * NT : 0) + (size_t)(v0 + j) * NT;
    }
    // contributors fw + k for k < C (C known), added in order into s
    template <int C>
    __device__ __forceinline__ void add(int w0, f32x4 (&s)[2]) const {
        f32x4 a[C][2];
#pragma unroll
        for (int k = 0; k < C; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j) a[k][j] = *at(w0 + k, j);
#pragma unroll
        for (int k = 0; k < C; ++k)
#pragma unroll
            for (int j = 0; j < 2; ++j) s[j] += a[k][j];
    }
};

template <int MBW, int WR, int WC, int CT, int BM, int BN>
__global__ __launch_bounds__(64 * WR * WC) void wide_sum_kernel(const f32x4 *__restrict__ part,
                                                                uint16_t *__restrict__ out, int M, int N,
                                                                int K, int col_tiles, int64_t units, int grid,
                                                                int maxt) {
    constexpr int NV = MBW * CT, NT = 64 * WR * WC;
    static_assert(NV % 2 == 0, "accumulators go in pairs");
    const int tile = blockIdx.x / (NV / 2), v0 = 2 * (blockIdx.x % (NV / 2));
    const int KT = K >> 7;
    const int64_t t0 = (int64_t)tile * KT;
    const int fw = sk_owner(t0, units, grid), lw = sk_owner(t0 + KT - 1, units, grid);
    if (fw == lw) return;  // one workgroup computed the whole tile
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave / WC, wc = wave % WC, r = lane & 15, g = lane >> 4;
    const WideSum<NV, NT> ws{part + tid, (size_t)maxt * NV * NT, fw, tile - sk_first_tile(fw, units, grid, KT), v0};
    f32x4 sum[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int nc = lw - fw + 1;
    if (nc == 2) {
        ws.template add<2>(fw, sum);
    } else if (nc == 3) {
        ws.template add<3>(fw, sum);
    } else if (nc == 4) {
        ws.template add<4>(fw, sum);
    } else {
        for (int w0 = fw; w0 <= lw; w0 += 8) {
            f32x4 a[8][2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int w = w0 + k < lw ? w0 + k : lw;
#pragma unroll
                for (int j = 0; j < 2; ++j) a[k][j] = *ws.at(w, j);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (w0 + k <= lw)
#pragma unroll
                    for (int j = 0; j < 2; ++j) sum[j] += a[k][j];
        }
    }
    const int rt = tile / col_tiles, cb = tile % col_tiles;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int v = v0 + j;
        const int nbg = cb * (BN / 16) + wc * CT + v % CT;
        if (nbg >= (N >> 4)) continue;
        const int colg = nbg * 16 + r;
        const int rowb = rt * BM + (wr * MBW + v / CT) * 16 + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (rowb + i < M) out[(size_t)(rowb + i) * N + colg] = f32_to_bf16_rne(sum[j][i]);
    }
}

// Split-K finish of the small-M kernels. Workgroup (nb, sp) of `splits` holds,
// in threads t < 16*M, the partial sum v of output (m = t/16, column 16*nb +
// t%16). With one split it is the result. Otherwise every split stores its
// partials in its own slot and bumps the column block's arrival counter; the
// last to arrive adds the slots in split order (deterministic), writes bf16
// and clears the counter. part: [N/16][splits][16*M] fp32; cnt: [N/16].
__device__ __forceinline__ void smallm_finish(float v, int M, int N, int nb, int sp, int splits,
                                              uint16_t *__restrict__ out, uint32_t *__restrict__ cnt,
                                              float *__restrict__ part, int *s_flag) {
    const int t = threadIdx.x;
    const bool owner = t < 16 * M;
    const int m = t >> 4, c = t & 15;
    if (splits == 1) {
        if (owner) out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(v);
        return;
    }
    float *slots = part + (size_t)nb * splits * 16 * M;
    if (owner) __hip_atomic_store(slots + (size_t)sp * 16 * M + t, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_all_memory();
    __syncthreads();
    if (t == 0) *s_flag = (arrive(&cnt[nb]) == (uint32_t)(splits - 1));
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(*s_flag) == 0) return;
    if (owner) {
        float s = 0.f;
        for (int k = 0; k < splits; ++k)
            s += (k == sp) ? v
                           : __hip_atomic_load(slots + (size_t)k * 16 * M + t, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
        out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(s);
    }
    if (t == 0) clear_counter(&cnt[nb]);
}

// The same for a workgroup that owns `nblk` consecutive column blocks
// nb0 .. nb0 + nblk - 1 (one K range of each): thread t < nblk * 16 * M holds
// the sum v of block t / (16M), row (t / 16) % M, column t % 16 of the block.
// s_flags needs nblk ints of LDS.
__device__ __forceinline__ void multiblock_finish(float v, int M, int N, int nb0, int nblk, int sp,
                                                  int splits, uint16_t *__restrict__ out,
                                                  uint32_t *__restrict__ cnt, float *__restrict__ part,
                                                  int *s_flags) {
    const int t = threadIdx.x;
    const int per = 16 * M;
    const bool owner = t < nblk * per;
    const int b = t / per, tt = t - b * per, m = tt >> 4, c = tt & 15;
    const int nb = nb0 + b;
    if (splits == 1) {
        if (owner) out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(v);
        return;
    }
    float *slots = part + (size_t)nb * splits * per;
    if (owner) __hip_atomic_store(slots + (size_t)sp * per + tt, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_all_memory();
    __syncthreads();
    if (t < nblk) s_flags[t] = (arrive(&cnt[nb0 + t]) == (uint32_t)(splits - 1));
    __syncthreads();
    if (owner && s_flags[b]) {
        float s2 = 0.f;
        for (int k = 0; k < splits; ++k)
            s2 += (k == sp) ? v
                            : __hip_atomic_load(slots + (size_t)k * per + tt, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        out[(size_t)m * N + nb * 16 + c] = f32_to_bf16_rne(s2);
    }
    if (t < nblk && s_flags[t]) clear_counter(&cnt[nb0 + t]);
}

}  // namespace svq
