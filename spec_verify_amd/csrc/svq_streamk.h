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
#include "svq_launch.h"

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

// Finish of a tile shared by several workgroups. Counters of tile t (at
// cnt[3t..3t+2]): arrivals, a bit mask of reduced chunk ranges, departures.
//
// Every contributor stores its partial tile (NV f32x4 per thread, NT threads;
// slots laid out [workgroup][slot][NV][NT]) and arrives. The tile is reduced
// per accumulator index v (all contributors added in workgroup order, so the
// result does not depend on which workgroup reduces it). The contributors for
// which this tile is the last piece of work (the "finishing group", known
// from the schedule) split the NV indices into ranges, one each: a member
// waits, for a bounded time, until every partial is in, reduces its range and
// sets its bit. The last arriver reduces its own range if it has one, waits
// (bounded) for the other bits, and reduces every range whose bit is still
// missing, so the tile is complete whether or not the members were resident
// at the same time; a range reduced twice is written twice with the same
// values. The last contributor to depart clears the three counters.
// The two wait budgets are kernel arguments (SkWait, in ticks of the 100 MHz
// s_memrealtime clock); a budget of 0 makes every member give up at once, so
// the owner reduces every range itself.
struct SkWait {
    uint32_t arrive_ticks, range_ticks;
};
constexpr int kSkMaxRanges = 32;               // one bit each

// Spin (thread 0) until (*p & mask) == mask, or at least `want` for mask 0,
// for at most `ticks`; returns whether it happened. A budget of 0 gives up at
// once without looking.
__device__ __forceinline__ bool sk_wait(uint32_t *p, uint32_t want, uint32_t mask, uint64_t ticks) {
    if (ticks == 0) return false;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        const uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (mask ? (v & mask) == mask : v >= want) return true;
        if (__builtin_amdgcn_s_memrealtime() - t0 > ticks) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

template <int NV, int NT, typename StoreV>
__device__ __forceinline__ void sk_reduce(const f32x4 (&acc)[NV], int tile, int KT, int64_t units,
                                          int grid, int maxt, uint32_t *cnt, f32x4 *part,
                                          int *s_sk, SkWait wt, StoreV store_v) {
    const int tid = threadIdx.x;
    const int wg = blockIdx.x;
    uint32_t *c = cnt + kSkCountersPerTile * tile;
    const uint32_t slot_bytes = (uint32_t)NV * NT * 16;
    const int slot = tile - sk_first_tile(wg, units, grid, KT);
    const __amdgpu_buffer_rsrc_t mine = make_rsrc(part + (size_t)(wg * maxt + slot) * NV * NT, slot_bytes);
#pragma unroll
    for (int v = 0; v < NV; ++v)
        __builtin_amdgcn_raw_buffer_store_b128(acc[v], mine, (uint32_t)(v * NT + tid) * 16, 0, kCoherent);
    const int64_t tend = (int64_t)tile * KT + KT;  // one past the tile's last unit
    const int fw = __builtin_amdgcn_readfirstlane(sk_owner((int64_t)tile * KT, units, grid));
    const int lw = __builtin_amdgcn_readfirstlane(sk_owner(tend - 1, units, grid));
    const uint32_t nc = (uint32_t)(lw - fw + 1);
    // finishing group: fw..lw-1 (their ranges end inside the tile) and lw if
    // its range ends with the tile
    const int nf0 = lw - fw + ((int64_t)(lw + 1) * units / grid <= tend ? 1 : 0);
    const int nf = nf0 < kSkMaxRanges ? nf0 : kSkMaxRanges;
    const int me = wg - fw;  // my range, if me < nf (the ranges cover all NV indices)
    const uint32_t all = nf == 32 ? 0xffffffffu : ((1u << nf) - 1u);
    wait_all_memory();
    __syncthreads();
    if (tid == 0) s_sk[0] = (int)arrive(&c[0]);
    __syncthreads();
    const bool owner = (uint32_t)__builtin_amdgcn_readfirstlane(s_sk[0]) == nc - 1;

    auto view = [&](int w) {
        const int wslot = __builtin_amdgcn_readfirstlane(tile - sk_first_tile(w, units, grid, KT));
        return make_rsrc(part + (size_t)(w * maxt + wslot) * NV * NT, slot_bytes);
    };
    // reduce accumulator indices [v0, v1), two at a time with eight
    // contributors' loads each in flight (every load is a round trip to the
    // device-coherent level)
    auto reduce = [&](int v0, int v1) {
        for (int v = v0; v < v1; v += 2) {
            const bool two = v + 1 < v1;
            f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = sa;
            for (int w0 = fw; w0 <= lw; w0 += 8) {
                f32x4 a[8], b[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (w0 + k > lw) continue;
                    const __amdgpu_buffer_rsrc_t rs = view(w0 + k);
                    a[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)(v * NT + tid) * 16, 0, kCoherent);
                    if (two) b[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((v + 1) * NT + tid) * 16, 0, kCoherent);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    if (w0 + k > lw) continue;
                    sa += a[k];
                    if (two) sb += b[k];
                }
            }
            store_v(v, sa);
            if (two) store_v(v + 1, sb);
        }
    };
    auto range_lo = [&](int e) { return e * NV / nf; };

    bool mine_ready = owner;
    if (!owner && me < nf) {
        if (tid == 0) s_sk[1] = sk_wait(&c[0], nc, 0u, wt.arrive_ticks) ? 1 : 0;
        __syncthreads();
        mine_ready = __builtin_amdgcn_readfirstlane(s_sk[1]) != 0;
    }
    if (mine_ready && me < nf) {
        reduce(range_lo(me), range_lo(me + 1));
        __syncthreads();
        if (tid == 0) __hip_atomic_fetch_or(&c[1], 1u << me, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (owner) {
        // the other members' ranges: wait a bounded time for their bits, then
        // reduce whatever is still missing
        if (tid == 0) {
            sk_wait(&c[1], 0u, all, wt.range_ticks);
            s_sk[2] = (int)__hip_atomic_load(&c[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        const uint32_t done = (uint32_t)__builtin_amdgcn_readfirstlane(s_sk[2]);
        for (int e = 0; e < nf; ++e)
            if (!((done >> e) & 1u)) reduce(range_lo(e), range_lo(e + 1));
    }
    __syncthreads();
    if (tid == 0 && arrive(&c[2]) == nc - 1) {
        clear_counter(&c[0]);
        clear_counter(&c[1]);
        clear_counter(&c[2]);
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
