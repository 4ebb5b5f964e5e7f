// Cross-workgroup reductions shared by the kernels that split work.
//
// Handoff without fences: an agent-scope release/acquire fence on gfx950 writes
// back / invalidates the XCD-local L2 caches and costs tens of microseconds per
// workgroup when hundreds of workgroups do it, so partials travel with
// coherent ("sc1") stores and loads that bypass the non-coherent L2 state
// instead. A contributor stores its partial coherently, waits until its stores
// have completed (s_waitcnt), and only then bumps the arrival counter with an
// agent-scope atomic; the workgroup that observes the final count reads the
// other partials with coherent loads. Partials are added in a fixed order, so
// results are deterministic, and the last arriver clears the counter.
#pragma once

#include "svq_device.h"

namespace svq {

constexpr int kCoherent = 16;  // cache-policy bits of a buffer access: sc1

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

// Returns true in every thread of the workgroup that must write the tile's
// output; `acc` then holds the full sum. NV f32x4 accumulators per thread, NT
// threads; `part` slots are laid out [workgroup][slot][NV][NT] (f32x4).
template <int NV, int NT>
__device__ __forceinline__ bool sk_fixup(f32x4 (&acc)[NV], int tile, int KT, int64_t units,
                                         int grid, int maxt, uint32_t *cnt, f32x4 *part,
                                         int *s_flag) {
    const int tid = threadIdx.x;
    const int wg = blockIdx.x;
    const uint32_t slot_bytes = (uint32_t)NV * NT * 16;
    const int slot = tile - sk_first_tile(wg, units, grid, KT);
    const __amdgpu_buffer_rsrc_t mine = make_rsrc(part + (size_t)(wg * maxt + slot) * NV * NT, slot_bytes);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        __builtin_amdgcn_raw_buffer_store_b128(acc[v], mine, (uint32_t)(v * NT + tid) * 16, 0, kCoherent);
    const int fw = sk_owner((int64_t)tile * KT, units, grid);
    const int lw = sk_owner((int64_t)tile * KT + KT - 1, units, grid);
    wait_all_memory();
    __syncthreads();
    if (tid == 0) *s_flag = (arrive(&cnt[tile]) == (uint32_t)(lw - fw));
    __syncthreads();
    // read as a wave-uniform value: the code below is then uniform control
    // flow with scalar buffer descriptors
    if (__builtin_amdgcn_readfirstlane(*s_flag) == 0) return false;
    // every contributor, this one included, stored its partial above: add
    // them all from memory in workgroup order, so that `acc` need not stay
    // live next to the running sum
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int fwu = __builtin_amdgcn_readfirstlane(fw), lwu = __builtin_amdgcn_readfirstlane(lw);
    // uniform by construction; readfirstlane lets the compiler keep the buffer
    // descriptors in scalar registers
    auto view = [&](int w) {
        const int wslot = __builtin_amdgcn_readfirstlane(tile - sk_first_tile(w, units, grid, KT));
        return make_rsrc(part + (size_t)(w * maxt + wslot) * NV * NT, slot_bytes);
    };
    // two contributors' loads in flight at a time (each load is a round trip
    // to the device-coherent level), added in workgroup order
    for (int w = fwu; w <= lwu; w += 2) {
        f32x4 a[NV], b[NV];
        const __amdgpu_buffer_rsrc_t ra = view(w);
#pragma unroll
        for (int v = 0; v < NV; ++v) a[v] = __builtin_amdgcn_raw_buffer_load_b128(ra, (uint32_t)(v * NT + tid) * 16, 0, kCoherent);
        const bool two = w + 1 <= lwu;
        if (two) {
            const __amdgpu_buffer_rsrc_t rb = view(w + 1);
#pragma unroll
            for (int v = 0; v < NV; ++v) b[v] = __builtin_amdgcn_raw_buffer_load_b128(rb, (uint32_t)(v * NT + tid) * 16, 0, kCoherent);
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) acc[v] += a[v];
        if (two) {
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[v] += b[v];
        }
    }
    if (tid == 0) clear_counter(&cnt[tile]);
    return true;
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

}  // namespace svq
