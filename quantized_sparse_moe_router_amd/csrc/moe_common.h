// moe_common.h -- device helpers shared by the gfx950 kernels of the MoE layer, and the
// host-side prototypes of each kernel file's launcher.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
// low / high bf16 of a packed pair
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) {
    return __uint_as_float(pair & 0xffff0000u);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int m) { return __shfl_xor(v, m, kWave); }

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group
// ends with the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += shfl_xor(v, m);
    return v;
}

}  // namespace moe

// ---------------------------------------------------------------- launchers (host)
// Each returns hipSuccess or the first HIP error of its launches.  Arguments are already
// validated by the C entry points.
namespace moe {

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, hipStream_t s);

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* ws, hipStream_t s);
size_t permute_ws_bytes(int64_t P, int E);
hipError_t read_and_clear_device_error(int* flag);

// Grouped (ids/offsets/sorted_pairs non-null) or dense (all null) expert FFN.
hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, const int32_t* offsets,
                           const int32_t* sorted_pairs, uint16_t* y, uint16_t* h_ws,
                           hipStream_t s);
hipError_t launch_ffn_mfma(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           void* ws, hipStream_t s);
size_t ffn_mfma_ws_bytes(int64_t rows, int E, int F);

hipError_t launch_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* w,
                          const uint16_t* y_shared, const uint16_t* residual, int T, int k,
                          int d, uint16_t* out, hipStream_t s);

}  // namespace moe
