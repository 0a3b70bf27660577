// norm.hip -- the pre-layer RMS norm of T tokens and their residual-gate logits (the
// arithmetic and its reading are in norm_common.h).  One wave per token: the row is read
// once in the norm's chunk order, and the same chunks of xn feed the gate's dot product,
// whose fixed order deals the same 4-element chunks to the same lanes.
#include "norm_common.h"

namespace moe {
namespace {

template <int NC>
__global__ void __launch_bounds__(256) rmsnorm_kernel(const uint16_t* __restrict__ x, int T,
                                                      int d, const float* __restrict__ gamma,
                                                      float eps, const float* __restrict__ gw,
                                                      float gb, uint16_t* __restrict__ xn,
                                                      float* __restrict__ z) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    uint2 x4[NC];
    const float ss = group_sum<64>(rms_lane_sumsq<NC>(x + (size_t)t * d, lane, x4));
    const float r = rms_scale(ss, d, eps);
    const float zt = rms_row_and_gate<NC>(x4, lane, r, gamma, gw, gb, xn + (size_t)t * d);
    if (gw && lane == 0) z[t] = zt;
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, int T, int d, const float* gamma, float eps,
                          const float* gw, float gb, uint16_t* xn, float* z, hipStream_t s) {
    const unsigned blocks = (unsigned)((T + 3) / 4);
#define MOE_NC(N)                                                                        \
    if (d == 256 * N) {                                                                  \
        rmsnorm_kernel<N><<<blocks, 256, 0, s>>>(x, T, d, gamma, eps, gw, gb, xn, z);    \
        return hipGetLastError();                                                        \
    }
    MOE_NC(1)
    MOE_NC(2)
    MOE_NC(4)
    MOE_NC(8)
    MOE_NC(16)
#undef MOE_NC
    return hipErrorInvalidValue;
}

}  // namespace moe
