// probe.hip -- the weight decoders of the two expert paths, run on their own over whole
// matrices, so that a test can compare every decoded weight with its exact value bit for
// bit.  Expert weights are 4-bit, some layers 6-bit [本地部署Qwen3.8-Flash-Next模型的两条路线
// (blog.cycleuser.org), section 精度和内存占用], low-bit tiers 2-3 bit [Strata 与
// Qwen3.8-Flash-Next (telli.sh)]; the code layouts are those of moe.h.
//
//   form 0 (few-token GEMV path): the group dot product dot_bits, the zero-point removal and
//     the scale, exactly as gemv_rows applies them, evaluated on one-hot activations (the
//     group's activation sum is then 1): element c of the group gives
//     s * ((128 + u_c) - kBias) in fp32, which is s * q exactly when the decoder is right.
//   form 1 (grouped GEMM path): chunk_codes + chunk_pair, the functions that form the MFMA
//     B operand, giving bf16(s * q) rounded to nearest even.
#include "gemv_common.h"
#include "mfma_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

template <int FMT>
__global__ void __launch_bounds__(256) probe_gemv_kernel(const uint8_t* __restrict__ w,
                                                         const uint16_t* __restrict__ s,
                                                         int64_t n_groups,
                                                         float* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_groups) return;
    GroupBits<FMT> bits;
    load_bits<FMT>(w + g * Fmt<FMT>::kGroupBytes, bits);
    const float sc = f16_to_f32(s[g]);
    for (int c = 0; c < 32; ++c) {
        uint32_t xp[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xp[i] = (2 * i == c) ? 0x3f80u : (2 * i + 1 == c) ? 0x3f800000u : 0u;
        if constexpr (FMT == MOE_FMT_INT4_G32) nibble_pairs16(xp);
        // opaque registers: folded into an inline constant of v_dot2c_f32_bf16, the pair
        // (bf16 1.0, 0) = 0x00003f80 is emitted as the constant 1.0, which the instruction
        // reads as the 32-bit pattern 0x3f800000 (1.0 in the other half)
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xp[i]));
        const float sx = group_sum_x(xp);
        if constexpr (kPairInRegisters<FMT>) {
            pair_in_registers<FMT>(xp);
#pragma unroll
            for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(xp[i]));
        }
        const float raw = dot_bits<FMT>(bits, xp);
        const float part = __builtin_fmaf(-Fmt<FMT>::kBias, sx, raw);
        out[g * 32 + c] = __builtin_fmaf(sc, part, 0.0f);
    }
}

template <int FMT>
__global__ void __launch_bounds__(256) probe_mfma_kernel(const uint8_t* __restrict__ w,
                                                         const uint16_t* __restrict__ s,
                                                         int64_t n_groups,
                                                         uint16_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_groups) return;
    GroupCodes<FMT> codes;
    const uint8_t* p = w + g * Fmt<FMT>::kGroupBytes;
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        codes.a = u32x4_t{v.x, v.y, v.z, v.w};
    } else if constexpr (FMT == MOE_FMT_INT6_G32) {
        const uint2* q = reinterpret_cast<const uint2*>(p);
        const uint2 a0 = q[0], a1 = q[1], b = q[2];
        codes.a = u32x4_t{a0.x, a0.y, a1.x, a1.y};
        codes.b = u32x2_t{b.x, b.y};
    } else if constexpr (FMT == MOE_FMT_INT3_G32) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        codes.a = u32x4_t{q[0], q[1], q[2], 0u};
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        codes.a = u32x4_t{v.x, v.y, 0u, 0u};
    }
    const float sc = f16_to_f32(s[g]);
    for (int c = 0; c < 4; ++c) {
        uint32_t lo, hi;
        chunk_codes<FMT>(codes, c, lo, hi);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t pair = chunk_pair<FMT>(lo, hi, b, sc);
            out[g * 32 + 8 * c + 2 * b] = (uint16_t)(pair & 0xffffu);
            out[g * 32 + 8 * c + 2 * b + 1] = (uint16_t)(pair >> 16);
        }
    }
}

}  // namespace

hipError_t launch_dequant_probe(int fmt, int form, const uint8_t* w, const uint16_t* s,
                                int64_t n_groups, void* out, hipStream_t st) {
    const unsigned blocks = (unsigned)((n_groups + 255) / 256);
#define MOE_PROBE(F)                                                                      \
    if (fmt == F) {                                                                       \
        if (form == 0)                                                                    \
            probe_gemv_kernel<F><<<blocks, 256, 0, st>>>(w, s, n_groups,                  \
                                                         static_cast<float*>(out));       \
        else                                                                              \
            probe_mfma_kernel<F><<<blocks, 256, 0, st>>>(w, s, n_groups,                  \
                                                         static_cast<uint16_t*>(out));    \
        return hipGetLastError();                                                         \
    }
    MOE_PROBE(MOE_FMT_INT4_G32)
    MOE_PROBE(MOE_FMT_INT6_G32)
    MOE_PROBE(MOE_FMT_INT3_G32)
    MOE_PROBE(MOE_FMT_INT2_G32)
#undef MOE_PROBE
    return hipErrorNotSupported;
}

}  // namespace moe
