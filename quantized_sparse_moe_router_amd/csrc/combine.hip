// combine.hip -- weighted combine of the selected experts' outputs with the shared expert.
//
// Each token's output is the gate-weighted sum of its 10 selected experts plus the shared
// expert, which always contributes with weight one [Strata 与 Qwen3.8-Flash-Next
// (telli.sh), section 稀疏架构创造了机会].  The sum is a gather in slot order (no atomics),
// so the result does not depend on scheduling; it is bound by reading the pair outputs.
#include "moe_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// One thread = 8 consecutive outputs (16 bytes) of one token.
__global__ void __launch_bounds__(256) combine_kernel(
    const uint16_t* __restrict__ y_pairs, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ w, const uint16_t* __restrict__ y_shared,
    const uint16_t* residual, int T, int k, int d, uint16_t* out) {
    const int per_row = d / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * per_row) return;
    const int t = (int)(idx / per_row);
    const int c8 = (int)(idx % per_row);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // slots in chunks of 8: all index/weight loads, then all row loads, then the sums in
    // slot order, so a chunk's loads are in flight together.  Padding slots and dropped
    // pairs (bad ids) read row 0 and add it with weight 0.
    for (int j0 = 0; j0 < k; j0 += 8) {
        int q[8];
        float wj[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int jj = min(j0 + j, k - 1);
            q[j] = pair_pos[(size_t)t * k + jj];
            wj[j] = w[(size_t)t * k + jj];
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
    if (y_shared) {
        const uint4 v = *reinterpret_cast<const uint4*>(y_shared + (size_t)t * d + 8 * c8);
        const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += bf16lo(vv[i]);
            acc[2 * i + 1] += bf16hi(vv[i]);
        }
    }
    uint32_t o[4];
    if (residual) {
        const uint4 r = *reinterpret_cast<const uint4*>(residual + (size_t)t * d + 8 * c8);
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
    *reinterpret_cast<uint4*>(out + (size_t)t * d + 8 * c8) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* w,
                          const uint16_t* y_shared, const uint16_t* residual, int T, int k,
                          int d, uint16_t* out, hipStream_t s) {
    const int64_t n = (int64_t)T * (d / 8);
    const int blocks = (int)((n + 255) / 256);
    combine_kernel<<<blocks, 256, 0, s>>>(y_pairs, pair_pos, w, y_shared, residual, T, k, d,
                                          out);
    return hipGetLastError();
}

}  // namespace moe
