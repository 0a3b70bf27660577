// norm_common.h -- the pre-layer RMS norm and the residual gate, as device helpers shared by
// the standalone norm kernel (norm.hip), the decode router that computes the norm itself
// (route.hip) and the combines (combine_common.h, decode.hip), so that every path rounds
// alike and the fused decode block equals its composition bit for bit.
//
// The pages keep a gated residual on the GPU next to the router [本地部署Qwen3.8-Flash-Next
// 模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法] with no formula; the
// reading here: the layer runs on xn = RMSNorm(x) and its output joins the stream as
// x + sigmoid(z) * out.  Fixed fp32 order for the norm (routing on xn must be reproducible):
//   ss   = sum of x_c^2: the row cut into chunks of 4 bf16, chunk v to lane v mod 64, one
//          fused multiply-add chain per lane over its chunks in ascending order, then the
//          butterfly over lanes with offsets 1..32 (group_sum<64>);
//   r    = fl(1 / fl(sqrt(fl(fl(ss / d) + eps)))), IEEE division and square root (the
//          compiler's default single-precision sqrt and division are correctly rounded);
//   xn_c = bf16(fl(fl(x_c * r) * gamma_c)).
// (Inputs are finite; an all-zero row needs eps > 0.)
// The gate logit z = <gate_w, xn> + gate_b takes the router's fp32 order, whose 16-byte
// weight vectors are the same 4-element chunks.
#pragma once
#include "moe_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// This lane's part of the sum of squares of a bf16 row of NC * 256 elements (chunks
// lane + 64 j, j = 0 .. NC-1); x4[j] receives chunk j as two bf16 pairs.
template <int NC>
__device__ __forceinline__ float rms_lane_sumsq(const uint16_t* x, int lane, uint2* x4) {
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) x4[j] = *reinterpret_cast<const uint2*>(x + (lane + 64 * j) * 4);
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const float a = bf16lo(x4[j].x), b = bf16hi(x4[j].x);
        const float c = bf16lo(x4[j].y), e = bf16hi(x4[j].y);
        acc = __builtin_fmaf(a, a, acc);
        acc = __builtin_fmaf(b, b, acc);
        acc = __builtin_fmaf(c, c, acc);
        acc = __builtin_fmaf(e, e, acc);
    }
    return acc;
}

__device__ __forceinline__ float rms_scale(float ss, int d, float eps) {
    const float ms = ss / (float)d;
    return 1.0f / sqrtf(ms + eps);
}

typedef __bf16 norm_bf16x2 __attribute__((ext_vector_type(2)));

// xn of two elements, fl(fl(x * r) * gamma) each, rounded to bf16 (to nearest even) by one
// v_cvt_pk_bf16_f32; returns the pair packed (first element in the low half)
__device__ __forceinline__ uint32_t rms_apply_pair(float x0, float x1, float r, float g0,
                                                   float g1) {
    const float a0 = x0 * r, a1 = x1 * r;
    const norm_bf16x2 p = {(__bf16)(a0 * g0), (__bf16)(a1 * g1)};
    return __builtin_bit_cast(uint32_t, p);
}

// One wave, one token: xn of the whole row in the chunk order (stored if xn_row is not
// null) and, if gw is not null, the gate logit <gw, xn> + gb in the router's fp32 order
// (every lane returns it).  r is the token's norm scale.
template <int NC>
__device__ __forceinline__ float rms_row_and_gate(const uint2* x4, int lane, float r,
                                                  const float* gamma, const float* gw,
                                                  float gb, uint16_t* xn_row) {
    // every gamma and gate chunk requested before the first is used (left alone, the
    // compiler awaits each chunk before requesting the next)
    float4 g4[NC], w4[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c0 = (lane + 64 * j) * 4;
        g4[j] = *reinterpret_cast<const float4*>(gamma + c0);
        w4[j] = gw ? *reinterpret_cast<const float4*>(gw + c0) : make_float4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NC; ++j)
        asm volatile("" : "+v"(g4[j].x), "+v"(g4[j].y), "+v"(g4[j].z), "+v"(g4[j].w),
                     "+v"(w4[j].x), "+v"(w4[j].y), "+v"(w4[j].z), "+v"(w4[j].w));
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < NC; ++j) {
        const int c0 = (lane + 64 * j) * 4;
        const uint32_t n01 = rms_apply_pair(bf16lo(x4[j].x), bf16hi(x4[j].x), r, g4[j].x,
                                            g4[j].y);
        const uint32_t n23 = rms_apply_pair(bf16lo(x4[j].y), bf16hi(x4[j].y), r, g4[j].z,
                                            g4[j].w);
        if (xn_row) *reinterpret_cast<uint2*>(xn_row + c0) = make_uint2(n01, n23);
        acc = __builtin_fmaf(bf16lo(n01), w4[j].x, acc);
        acc = __builtin_fmaf(bf16hi(n01), w4[j].y, acc);
        acc = __builtin_fmaf(bf16lo(n23), w4[j].z, acc);
        acc = __builtin_fmaf(bf16hi(n23), w4[j].w, acc);
    }
    if (!gw) return 0.0f;
    return group_sum<64>(acc) + gb;
}

// sigmoid of the gate logit, the factor on the layer's output
__device__ __forceinline__ float gate_value(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace
}  // namespace moe
