// mfma_common.h -- pieces shared by the gfx950 MFMA kernels (grouped expert GEMM, router
// candidate GEMM): operand vector types, bf16 packing, and global -> LDS loads that
// bypass registers.  Internal to the library.
#pragma once
#include "moe_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // plain vector: stays in VGPRs
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

// Global -> LDS loads.  lds is the wave-uniform byte address of the destination, set in M0
// (the instruction needs one wait state after M0 is written).  Lane l's data lands at
// lds + 16 l for dwordx4 and dwordx3 (12 bytes used), and at lds + 4 l for dword and
// ushort (zero-extended to 32 bits).  The compiler does not track these writes: callers count
// them with MOE_WAIT_VMCNT.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma12(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx3 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma2(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_ushort %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The same with the address split into a wave-uniform base (SGPR pair) and a per-lane
// 32-bit byte offset: per k-step only the base moves, a scalar add.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma12s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx3 %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma2s(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(sbase),
                 "{m0}"(lds) : "memory");
}

// a pointer made wave-uniform (both halves read from the first active lane), so that it
// lives in SGPRs
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

// ---- dequantisation of packed weight codes into bf16 MFMA operands (the grouped GEMM
// and the dequantisation probe call these same functions)
// The codes of one 32-code group: int4 = 16 bytes (a), int6 = 24 bytes (a, then b),
// int3 = 12 bytes (a[0..2]), int2 = 8 bytes (a[0..1]).
template <int FMT>
struct GroupCodes {
    u32x4_t a;
    u32x2_t b;
};

// zero point of a format's codes (value = s * (code - zero point))
template <int FMT>
constexpr float kZeroPoint = FMT == MOE_FMT_INT4_G32   ? 8.0f
                             : FMT == MOE_FMT_INT6_G32 ? 32.0f
                             : FMT == MOE_FMT_INT3_G32 ? 4.0f
                                                       : 2.0f;

// Chunk c (codes 8c..8c+7) of a group, split into byte-aligned code fields: lo holds
// codes 8c, 8c+2, 8c+4, 8c+6 in bytes 0..3, hi codes 8c+1, 8c+3, 8c+5, 8c+7.
template <int FMT>
__device__ __forceinline__ void chunk_codes(const GroupCodes<FMT>& g, int c, uint32_t& lo,
                                            uint32_t& hi) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        const uint32_t w = g.a[c];      // byte i: code 8c+2i (low nibble), 8c+2i+1 (high)
        lo = w & 0x0f0f0f0fu;
        hi = (w >> 4) & 0x0f0f0f0fu;
    } else if constexpr (FMT == MOE_FMT_INT6_G32) {
        // 8 six-bit codes = bits [48c, 48c + 48) of the 24-byte group
        const uint32_t w6[6] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y};
        const int bit = 48 * c, wi = bit / 32, sh = bit % 32;
        const uint64_t v = ((uint64_t)w6[wi] | ((uint64_t)w6[wi + 1] << 32)) >> sh;
        uint32_t l = 0, h = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            l |= (uint32_t)((v >> (12 * p)) & 63u) << (8 * p);
            h |= (uint32_t)((v >> (12 * p + 6)) & 63u) << (8 * p);
        }
        lo = l;
        hi = h;
    } else if constexpr (FMT == MOE_FMT_INT3_G32) {
        // 8 three-bit codes = bits [24c, 24c + 24) of the 12-byte group
        const uint32_t w3[3] = {g.a.x, g.a.y, g.a.z};
        const int bit = 24 * c, wi = bit / 32, sh = bit % 32;
        const uint32_t nxt = wi + 1 < 3 ? w3[wi + 1 < 3 ? wi + 1 : 2] : 0u;
        const uint64_t v = ((uint64_t)w3[wi] | ((uint64_t)nxt << 32)) >> sh;
        uint32_t l = 0, h = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            l |= (uint32_t)((v >> (6 * p)) & 7u) << (8 * p);
            h |= (uint32_t)((v >> (6 * p + 3)) & 7u) << (8 * p);
        }
        lo = l;
        hi = h;
    } else {
        // 8 two-bit codes = bits [16c, 16c + 16) of the 8-byte group
        const uint32_t w = (c < 2 ? g.a.x : g.a.y) >> (16 * (c & 1));
        uint32_t l = 0, h = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            l |= ((w >> (4 * p)) & 3u) << (8 * p);
            h |= ((w >> (4 * p + 2)) & 3u) << (8 * p);
        }
        lo = l;
        hi = h;
    }
    asm volatile("" : "+v"(lo), "+v"(hi));   // keep the byte fields for byte-to-float ops
}

// Codes 8c+2b and 8c+2b+1 -> packed bf16 pair s * (code - zero point).
template <int FMT>
__device__ __forceinline__ uint32_t chunk_pair(uint32_t lo, uint32_t hi, int b, float s) {
    const float zc = -kZeroPoint<FMT> * s;
    const float e0 = (float)((lo >> (8 * b)) & 0xffu);
    const float e1 = (float)((hi >> (8 * b)) & 0xffu);
    return pack_bf16(__builtin_fmaf(e0, s, zc), __builtin_fmaf(e1, s, zc));
}

}  // namespace
}  // namespace moe

// wait until at most n of this wave's global loads are outstanding (n <= 63) and, with
// the _LDS form, until its LDS reads are done too (before a barrier after which other
// waves' loads overwrite what was read)
#define MOE_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define MOE_WAIT_VMCNT_LDS(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
