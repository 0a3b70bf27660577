// combine.hip -- weighted combine of the selected experts' outputs with the shared expert.
//
// Each token's output is the gate-weighted sum of its 10 selected experts plus the shared
// expert, which always contributes with weight one [Strata 与 Qwen3.8-Flash-Next
// (telli.sh), section 稀疏架构创造了机会].  The sum is a gather in slot order (no atomics),
// so the result does not depend on scheduling; it is bound by reading the pair outputs.
// The arithmetic is combine8 (combine_common.h).
#include "combine_common.h"

namespace moe {
namespace {

// One thread = 8 consecutive outputs (16 bytes) of one token.
__global__ void __launch_bounds__(256) combine_kernel(
    const uint16_t* __restrict__ y_pairs, const int32_t* __restrict__ pair_pos,
    const float* __restrict__ w, const uint16_t* __restrict__ y_shared,
    const uint16_t* residual, const float* __restrict__ z, int T, int k, int d,
    uint16_t* out) {
    const int per_row = d / 8;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)T * per_row) return;
    const int t = (int)(idx / per_row);
    const int c8 = (int)(idx % per_row);
    const uint4 o = combine8(y_pairs, pair_pos + (size_t)t * k, w + (size_t)t * k, k, d,
                                    c8, y_shared ? y_shared + (size_t)t * d : nullptr,
                                    residual ? residual + (size_t)t * d : nullptr,
                                    z ? z + t : nullptr);
    *reinterpret_cast<uint4*>(out + (size_t)t * d + 8 * c8) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* w,
                          const uint16_t* y_shared, const uint16_t* residual, const float* z,
                          int T, int k, int d, uint16_t* out, hipStream_t s) {
    const int64_t n = (int64_t)T * (d / 8);
    const int blocks = (int)((n + 255) / 256);
    combine_kernel<<<blocks, 256, 0, s>>>(y_pairs, pair_pos, w, y_shared, residual, z, T, k,
                                          d, out);
    return hipGetLastError();
}

}  // namespace moe
