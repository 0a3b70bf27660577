// combine_common.h -- the weighted combine of one token's expert outputs for 8 consecutive
// output columns.  The decode layer's down kernel repeats these operations element by
// element, so both round exactly alike.
//
// out = bf16( sum_{j<k} w_j * y[q_j]  + y_shared ), summed in fp32 in slot order; slots are
// taken in chunks of 8 (all index/weight loads, then all row loads, then the fused
// multiply-adds in slot order), and the padding slots of the last chunk, like dropped
// pairs (q_j < 0), add 0 * row 0.  With a residual-gate logit z the sum is scaled once,
// sum = fl(sigmoid(z) * sum), before rounding.  With a residual: bf16(residual + bf16(sum)).
#pragma once
#include "moe_common.h"
#include "norm_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// Columns 8 c8 .. 8 c8 + 7 of one token.  pos / w: the token's k sorted positions and gate
// weights; y_shared_row / residual_row / z (the token's residual-gate logit) may be null.
__device__ __forceinline__ uint4 combine8(const uint16_t* y_pairs, const int32_t* pos,
                                          const float* w, int k, int d, int c8,
                                          const uint16_t* y_shared_row,
                                          const uint16_t* residual_row,
                                          const float* z = nullptr) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        int q[8];
        float wj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int jj = min(j0 + j, k - 1);
            q[j] = pos[jj];
            wj[j] = w[jj];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j0 + j >= k || q[j] < 0) wj[j] = 0.0f;
            q[j] = max(q[j], 0);
        }
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = *reinterpret_cast<const uint4*>(y_pairs + (size_t)q[j] * d + 8 * c8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t vv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __builtin_fmaf(wj[j], bf16lo(vv[i]), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(wj[j], bf16hi(vv[i]), acc[2 * i + 1]);
            }
        }
    }
    if (y_shared_row) {
        const uint4 v = *reinterpret_cast<const uint4*>(y_shared_row + 8 * c8);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16lo(vv[i]);
            acc[2 * i + 1] += bf16hi(vv[i]);
        }
    }
    if (z) {
        const float g = gate_value(*z);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = g * acc[i];
    }
    uint32_t o[4];
    if (residual_row) {
        const uint4 r = *reinterpret_cast<const uint4*>(residual_row + 8 * c8);
        const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = bf16lo(rr[i]) + bf16_to_f32(f32_to_bf16(acc[2 * i]));
            const float hi = bf16hi(rr[i]) + bf16_to_f32(f32_to_bf16(acc[2 * i + 1]));
            o[i] = f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            o[i] = f32_to_bf16(acc[2 * i]) | (f32_to_bf16(acc[2 * i + 1]) << 16);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace
}  // namespace moe
