// Stream-K bookkeeping shared by the wide MFMA kernels.
//
// The (output tile, 128-row K step) units are split evenly over `grid`
// persistent workgroups: workgroup w owns [w*units/grid, (w+1)*units/grid).
// A tile whose steps are spread over several workgroups is finished by the last
// one to arrive: every contributor stores its fp32 partial in its own slot, then
// bumps the tile's arrival counter; the one that sees the final count adds all
// partials in workgroup order (a fixed order, so results are deterministic),
// writes the bf16 output and clears the counter for the next call.
#pragma once

#include "svq_device.h"

namespace svq {

// The workgroup whose unit range holds unit a (units >= grid >= 1).
__device__ __forceinline__ int sk_owner(int64_t a, int64_t units, int grid) {
    const int64_t w = ((a + 1) * grid - 1) / units;
    return (int)(w < grid - 1 ? w : grid - 1);
}

__device__ __forceinline__ int sk_first_tile(int w, int64_t units, int grid, int KT) {
    return (int)(((int64_t)w * units / grid) / KT);
}

// Returns true in every thread of the workgroup that must write the tile's
// output; `acc` then holds the full sum. NV f32x4 accumulators per thread, NT
// threads; `part` slots are laid out [workgroup][slot][NV][NT] (f32x4).
template <int NV, int NT>
__device__ __forceinline__ bool sk_fixup(f32x4 (&acc)[NV], int tile, int KT, int64_t units,
                                         int grid, int maxt, uint32_t *cnt, f32x4 *part,
                                         int *s_flag) {
    const int tid = threadIdx.x;
    const int wg = blockIdx.x;
    const int slot = tile - sk_first_tile(wg, units, grid, KT);
    f32x4 *mine = part + ((size_t)(wg * maxt + slot) * NV) * NT + tid;
#pragma unroll
    for (int v = 0; v < NV; ++v) mine[(size_t)v * NT] = acc[v];
    const int fw = sk_owner((int64_t)tile * KT, units, grid);
    const int lw = sk_owner((int64_t)tile * KT + KT - 1, units, grid);
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&cnt[tile], 1u);
        *s_flag = (prev == (uint32_t)(lw - fw));
    }
    __syncthreads();
    const bool last = *s_flag != 0;
    if (!last) return false;
    __threadfence();
    f32x4 sum[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) sum[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int w = fw; w <= lw; ++w) {
        if (w == wg) {
#pragma unroll
            for (int v = 0; v < NV; ++v) sum[v] += acc[v];
        } else {
            const int wslot = tile - sk_first_tile(w, units, grid, KT);
            const f32x4 *theirs = part + ((size_t)(w * maxt + wslot) * NV) * NT + tid;
#pragma unroll
            for (int v = 0; v < NV; ++v) sum[v] += __builtin_nontemporal_load(theirs + (size_t)v * NT);
        }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = sum[v];
    if (tid == 0) cnt[tile] = 0u;
    return true;
}

}  // namespace svq
