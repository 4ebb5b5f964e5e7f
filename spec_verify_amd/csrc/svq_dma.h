// LDS-DMA and LDS helpers shared by the wide MFMA kernels (gfx950).
#pragma once

#include "svq_device.h"

namespace svq {

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

}  // namespace svq
