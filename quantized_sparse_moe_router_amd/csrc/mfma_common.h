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
// lds + 16 l for dwordx4 and dwordx3 (12 bytes used), and at lds + 4 l for ushort
// (zero-extended to 32 bits).  The compiler does not track these writes: callers count
// them with MOE_WAIT_VMCNT.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void dma12(const void* g, uint32_t lds) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx3 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
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

}  // namespace
}  // namespace moe

// wait until at most n of this wave's global loads are outstanding (n <= 63) and, with
// the _LDS form, until its LDS reads are done too (before a barrier after which other
// waves' loads overwrite what was read)
#define MOE_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define MOE_WAIT_VMCNT_LDS(n) \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4))
