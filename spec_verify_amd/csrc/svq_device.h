// Device-side helpers shared by the gfx950 kernels of the quantized linear layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 pattern of -136.0: the W4A16 kernels build each weight as the bf16 value
// 128 + q (q = 0..15, exact) and subtract 136 * sum(x) per group, which gives
// sum(x * (q - 8)) with zero point 8.
constexpr uint32_t kBf16Neg136Pair = 0xC308C308u;
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr uint32_t kMagic128Pair = 0x43004300u;  // two bf16 128.0
constexpr uint32_t kNibblePairMask = 0x000F000Fu;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Raw (unswizzled, byte-addressed) buffer resource over [base, base + bytes).
// Loads past `bytes` return zero, which the kernels use for padding rows.
// DWORD3 = 0x00020000: 32-bit data format, the gfx9-family value for raw loads.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// The wave index as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fp16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                          __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the sum.
__device__ __forceinline__ float row16_sum(float v) {
    v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0xB1, 0xF, 0xF, true));   // quad_perm [1,0,3,2]
    v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x4E, 0xF, 0xF, true));   // quad_perm [2,3,0,1]
    v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
    v += bits_f32(__builtin_amdgcn_mov_dpp(f32_bits(v), 0x140, 0xF, 0xF, true));  // row_mirror
    return v;
}

// Sum of the four 16-lane rows, lane c of each row; every lane gets the sum of
// its column position: (r0 + r1) + (r2 + r3), a fixed order.
__device__ __forceinline__ float rows4_sum(float v) {
    auto p = __builtin_amdgcn_permlane16_swap(f32_bits(v), f32_bits(v), false, false);
    v = bits_f32(p[0]) + bits_f32(p[1]);
    auto q = __builtin_amdgcn_permlane32_swap(f32_bits(v), f32_bits(v), false, false);
    return bits_f32(q[0]) + bits_f32(q[1]);
}

// 4x4 transpose between the 16-lane row index and the word index of a 4-word
// per-lane fragment: word j of row r becomes word r of row j.
__device__ __forceinline__ void transpose_rows_words(uint32_t &w0, uint32_t &w1, uint32_t &w2,
                                                     uint32_t &w3) {
    auto a = __builtin_amdgcn_permlane32_swap(w0, w2, false, false);
    auto b = __builtin_amdgcn_permlane32_swap(w1, w3, false, false);
    auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    w0 = c[0];
    w1 = c[1];
    w2 = d[0];
    w3 = d[1];
}

__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// s_waitcnt immediate that waits until at most k vector-memory loads of this
// wave are outstanding (gfx9 encoding; expcnt and lgkmcnt left at their max).
constexpr int vmcnt_imm(int k) { return (k & 15) | (7 << 4) | (15 << 8) | (((k >> 4) & 3) << 14); }

// Wait until at most n (wave-uniform, 0 <= n <= K) loads are outstanding:
// s_waitcnt takes an immediate, so n selects one of K+1 waits. Loads complete
// in issue order, so this waits for everything issued before the last n.
template <int K>
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
    if constexpr (K == 0) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    } else {
        if (n >= K) __builtin_amdgcn_s_waitcnt(vmcnt_imm(K));
        else wait_vmcnt_at_most<K - 1>(n);
    }
}

// Barrier after this wave's LDS accesses have completed; unlike
// __syncthreads() it does not also wait for the vector memory loads in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One 16-byte-per-lane LDS-DMA load: lane l's 16 bytes from gptr land at
// lds_base + 16*l (lds_base wave-uniform); inactive lanes write nothing.
__device__ __forceinline__ void dma16(const void *gptr, void *lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)gptr,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8). Returns a logical index such that each XCD receives one
// contiguous range of [0, n): neighbouring column blocks, which share 128-byte
// scale lines and x, then share one XCD's L2.
__device__ __forceinline__ int xcd_contiguous(int b, int n) {
    const int q = n >> 3, r = n & 7, x = b & 7, i = b >> 3;
    return x * q + (x < r ? x : r) + i;
}

// Four bf16 pairs (one MFMA B operand: 8 rows x 1 column) from a repacked word.
__device__ __forceinline__ uint4 word_to_bf16x8(uint32_t w) {
    // one v_and_or_b32 per pair (the compiler would emit v_and + v_or); the
    // trailing s_nop covers the wait states between these VALU writes and an
    // MFMA that reads them
    uint32_t a, b, c, d, t1, t2, t3;
    asm("v_and_or_b32 %0, %7, %8, %9\n\t"
        "v_lshrrev_b32 %4, 4, %7\n\t"
        "v_lshrrev_b32 %5, 8, %7\n\t"
        "v_lshrrev_b32 %6, 12, %7\n\t"
        "v_and_or_b32 %1, %4, %8, %9\n\t"
        "v_and_or_b32 %2, %5, %8, %9\n\t"
        "v_and_or_b32 %3, %6, %8, %9\n\t"
        "s_nop 1"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(t1), "=&v"(t2), "=&v"(t3)
        : "v"(w), "s"(kNibblePairMask), "v"(kMagic128Pair));
    return make_uint4(a, b, c, d);
}

// The same four pairs for VALU consumers (no trailing wait states). Written as
// asm because v_and_or_b32 takes no literal operand: left to itself the
// compiler builds each pair with three instructions.
__device__ __forceinline__ uint4 word_to_pairs(uint32_t w) {
    uint32_t a, b, c, d, t1, t2, t3;
    asm("v_and_or_b32 %0, %7, %8, %9\n\t"
        "v_lshrrev_b32 %4, 4, %7\n\t"
        "v_lshrrev_b32 %5, 8, %7\n\t"
        "v_lshrrev_b32 %6, 12, %7\n\t"
        "v_and_or_b32 %1, %4, %8, %9\n\t"
        "v_and_or_b32 %2, %5, %8, %9\n\t"
        "v_and_or_b32 %3, %6, %8, %9"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d), "=&v"(t1), "=&v"(t2), "=&v"(t3)
        : "v"(w), "s"(kNibblePairMask), "v"(kMagic128Pair));
    return make_uint4(a, b, c, d);
}

// The same four pairs as word_to_bf16x8, but holding (q - 8) * s: each weight
// is q * s + m8s in fp32 (m8s = -8 s; one rounding), then rounded to bf16
// (nearest even). The nibble masks are asm so that the byte conversions read
// them in place (left to itself the compiler extracts every nibble first).
__device__ __forceinline__ uint4 word_to_bf16x8_scaled(uint32_t w, float s, float m8s) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    uint32_t lo, hi;  // nibbles 0, 2, 4, 6 and 1, 3, 5, 7 of w, one per byte
    asm("v_and_b32 %0, %2, %3\n\t"
        "v_lshrrev_b32 %1, 4, %2\n\t"
        "v_and_b32 %1, %1, %3"
        : "=&v"(lo), "=&v"(hi)
        : "v"(w), "s"(0x0F0F0F0Fu));
    auto f = [&](uint32_t v, int byte) { return __builtin_fmaf((float)((v >> (8 * byte)) & 0xFFu), s, m8s); };
    auto pk = [](float a, float b) {
        const f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    };
    // pair i: nibble i (low half), nibble i + 4 (high half)
    return make_uint4(pk(f(lo, 0), f(lo, 2)), pk(f(hi, 0), f(hi, 2)), pk(f(lo, 1), f(lo, 3)),
                      pk(f(hi, 1), f(hi, 3)));
}

// E8M0 code -> fp32 scale 2^(b-127) (b = 0 gives the fp32 subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return bits_f32(b == 0 ? 0x00400000u : (b << 23));
}

// Two E4M3FN codes (bytes 2*HI, 2*HI+1 of w) times `scale`, as a bf16 pair.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pair_scaled(uint32_t w, float scale) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
    return __builtin_bit_cast(uint32_t, r);
}

}  // namespace svq
