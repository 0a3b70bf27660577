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

// DPP lane permutations (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1] pair lanes
// whose index differs in bit 0 / bit 1; row_half_mirror pairs lane i with 7-i inside each
// 8-lane group; row_mirror pairs lane i with 15-i inside each 16-lane row.  Applied in that
// order to values that are already equal across the smaller aligned block, each step adds
// the two halves of the next aligned block, i.e. the same tree as xor offsets 1, 2, 4, 8.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf,
                                                      false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// v + v of lane (lane ^ M), M = 16 or 32, with gfx950's v_permlane16/32_swap instead of a
// round trip through the LDS crossbar: swapping a copy of v with v leaves one operand
// holding the lower lane of each pair and the other the upper, and fp addition is
// commutative, so every lane gets the same bits as v + shfl_xor(v, M).
template <int M>
__device__ __forceinline__ float add_swapped(float v) {
    const uint32_t u = __float_as_uint(v);
    uint32_t lo, hi;
    if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        lo = r[0]; hi = r[1];
    } else {
        static_assert(M == 32, "offset 16 or 32");
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        lo = r[0]; hi = r[1];
    }
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group
// ends with the group's sum, combined as the butterfly tree over xor offsets 1..G/2.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v = v + dpp<kDppXor1>(v);
    if constexpr (G >= 4) v = v + dpp<kDppXor2>(v);
    if constexpr (G >= 8) v = v + dpp<kDppHalfMirror>(v);
    if constexpr (G >= 16) v = v + dpp<kDppMirror>(v);
    if constexpr (G >= 32) v = add_swapped<16>(v);
    if constexpr (G >= 64) v = add_swapped<32>(v);
    return v;
}

}  // namespace moe

// ---------------------------------------------------------------- launchers (host)
// Each returns hipSuccess or the first HIP error of its launches.  Arguments are already
// validated by the C entry points.
namespace moe {

// Workspace area that holds an arrival counter.  It must be zero before a workspace's
// first use; every call leaves it zero.
constexpr size_t kRouteCounterBytes = 256;

// Device error word (per device): bit 0 = expert id out of range.  Returns its device
// address for the current device.
int* device_error_flag();
hipError_t read_and_clear_device_error(int* flag);

// Tokens up to which moe_route computes logits and selection in one launch (GEMV).
constexpr int kRouteGemvMaxTokens = 16;

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, unsigned* counter, hipStream_t s);
// Router logits only (fp32 [T][E], the same values launch_route computes), for T <= 64.
hipError_t launch_route_logits(const moe_router& r, const uint16_t* x, int T, float* logits,
                               hipStream_t s);

// Many tokens, logits not wanted: the bounded form.  launch_route_bounded_logits writes
// every logit to within 2^-11 (|x_t| nw[e] + |b_e|) of the fixed-order value (MFMA; planes
// is a workspace of route_bounded_planes_bytes, nw [E] the row norm bounds);
// launch_route_bounded_select recomputes in the fixed order the experts that bound cannot
// rule out and selects: ids and weights are those of launch_route, bit for bit.
size_t route_bounded_planes_bytes(int E, int d);
hipError_t launch_route_bounded_logits(const moe_router& r, const uint16_t* x, int T,
                                       uint16_t* planes, float* nw, float* lf, hipStream_t s);
hipError_t launch_route_bounded_select(const moe_router& r, const uint16_t* x, int T, int k,
                                       const float* nw, const float* lf, int32_t* ids,
                                       float* weights, hipStream_t s);

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* ws, hipStream_t s);
size_t permute_ws_bytes(int64_t P, int E);

// Small calls: weight-streaming GEMV, gate/up then down; positions come from ids
// (grouped) or the token index (dense, ids == nullptr).  ws = [h].
bool ffn_gemv_has_shape(int d_model, int d_ff);
hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, uint16_t* y, void* ws, hipStream_t s);
// Large calls: grouped MFMA GEMM.  ws = [h][tile list].
hipError_t launch_ffn_mfma(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           void* ws, hipStream_t s);
size_t ffn_mfma_ws_bytes(int64_t rows, int E, int F);

hipError_t launch_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* w,
                          const uint16_t* y_shared, const uint16_t* residual, int T, int k,
                          int d, uint16_t* out, hipStream_t s);

// Expert side of a decode step (routed + shared FFN and combine) in two launches, at most
// 64 pairs and S = T*k (+ T shared) slots whose h rows fit in kDecodeMaxLds bytes of LDS.
// Workspace: [h rows].
constexpr size_t kDecodeMaxLds = 128 * 1024;
struct DecodeWs {
    size_t h, bytes;
};
DecodeWs decode_ws_layout(int T, int k, int d_model, int d_ff);
bool decode_fits(int T, int k, int d_ff, bool shared);
// logits non-null: the selection runs inside (ids and weights are written); null: ids and
// weights are inputs.
hipError_t launch_decode_ffn(const moe_experts& routed, const moe_experts* shared,
                             const uint16_t* x, int T, int k, const float* logits,
                             int32_t* ids, float* weights, const uint16_t* residual,
                             uint16_t* out, void* ws, hipStream_t s);

}  // namespace moe
