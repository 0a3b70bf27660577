// ffn_gemv.hip -- expert FFN for few tokens (decode): stream the selected experts'
// packed weights once, dequantise in registers, reduce across the wavefront.
//
// Decode reads every active weight once per step and is bound by memory bandwidth
// [Halogen Flash Server配置與實測 (lcz.me), replies comparing decode with bandwidth];
// only the selected experts are touched, which is what sparse routing saves
// [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].
//
// The per-row arithmetic lives in gemv_common.h.  Two launches: gate/up + SwiGLU -> h (bf16), then down -> y.  In each, a block owns one
// slot and a block of rows and issues all its weight loads before it reads activations.
//
// Grouped mode (at most 64 pairs): a slot is a pair p.  A block reads the whole ids vector
// with one load, so the expert e = ids[p] is known after one memory round trip and the
// weight loads start at once; the pairs routed to e form a ballot mask, every MT-th of
// them leads a chunk of MT pairs and the others return.  A pair's row is its
// expert-sorted position (valid pairs with a smaller id, plus earlier pairs with the same
// id), the same position moe_permute assigns.
// Dense mode (shared expert): a slot is a chunk of MT tokens.
#include "gemv_common.h"

namespace moe {
namespace {

// grid.x = slots, grid.y = row blocks
template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_gateup_kernel(
    const uint8_t* __restrict__ wg, const uint16_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint16_t* __restrict__ su,
    const uint16_t* __restrict__ x, int T, int k, const int32_t* __restrict__ ids, int E,
    uint16_t* __restrict__ h) {
    using GU = Shape<D>;   // gate/up rows have K = d_model
    Slot sl;
    if (!resolve_slot<MT>(blockIdx.x, T, k, ids, E, sl)) return;
    gemv_rows<FMT, kModeGateUp, GU::LPR, GU::GPL, GU::ITERS, MT>(wg, sg, wu, su, x, k, F,
                                                                blockIdx.y, sl, h);
}

template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_down_kernel(
    const uint8_t* __restrict__ wd, const uint16_t* __restrict__ sd,
    const uint16_t* __restrict__ h, int T, int k, const int32_t* __restrict__ ids, int E,
    uint16_t* __restrict__ y) {
    using DN = Shape<F>;   // down rows have K = d_ff
    Slot sl;
    if (!resolve_slot<MT>(blockIdx.x, T, k, ids, E, sl)) return;
    gemv_rows<FMT, kModeDown, DN::LPR, DN::GPL, DN::ITERS, MT>(wd, sd, nullptr, nullptr, h, k,
                                                              D, blockIdx.y, sl, y);
}

template <int FMT, int D, int F, int MT>
hipError_t launch_mt(const moe_experts& ex, const uint16_t* x, int T, int k, const int32_t* ids,
                     uint16_t* y, uint16_t* h, hipStream_t s) {
    const int nslots = ids ? T * k : (T + MT - 1) / MT;
    constexpr int n_gu = (F + Shape<D>::RPB - 1) / Shape<D>::RPB;
    constexpr int n_dn = (D + Shape<F>::RPB - 1) / Shape<F>::RPB;
    ffn_gateup_kernel<FMT, D, F, MT><<<dim3(nslots, n_gu), 256, 0, s>>>(
        ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x, T, k, ids, ex.n_experts, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_down_kernel<FMT, D, F, MT><<<dim3(nslots, n_dn), 256, 0, s>>>(
        ex.w_down, ex.s_down, h, T, k, ids, ex.n_experts, y);
    return hipGetLastError();
}

// MT: a slot never holds more pairs than tokens (a token picks an expert at most once)
template <int FMT, int D, int F>
hipError_t launch_shape(const moe_experts& ex, const uint16_t* x, int T, int k,
                        const int32_t* ids, uint16_t* y, void* ws, hipStream_t s) {
    uint16_t* h = static_cast<uint16_t*>(ws);
    if (T == 1) return launch_mt<FMT, D, F, 1>(ex, x, T, k, ids, y, h, s);
    if (T == 2) return launch_mt<FMT, D, F, 2>(ex, x, T, k, ids, y, h, s);
    return launch_mt<FMT, D, F, 4>(ex, x, T, k, ids, y, h, s);
}

template <int FMT>
hipError_t launch_fmt(const moe_experts& ex, const uint16_t* x, int T, int k,
                      const int32_t* ids, uint16_t* y, void* ws, hipStream_t s) {
#define MOE_DEC(DV, FV)                                                                  \
    if (ex.d_model == DV && ex.d_ff == FV)                                               \
        return launch_shape<FMT, DV, FV>(ex, x, T, k, ids, y, ws, s);
    MOE_DEC(2048, 512)
    MOE_DEC(256, 128)
    MOE_DEC(2048, 1024)
    MOE_DEC(4096, 1024)
    MOE_DEC(1024, 512)
    MOE_DEC(2048, 2048)
#undef MOE_DEC
    return hipErrorNotSupported;
}

}  // namespace

bool ffn_gemv_has_shape(int d, int F) {
    return (d == 2048 && (F == 512 || F == 1024 || F == 2048)) || (d == 256 && F == 128) ||
           (d == 4096 && F == 1024) || (d == 1024 && F == 512);
}

hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, uint16_t* y, void* ws, hipStream_t s) {
    if (ex.fmt == MOE_FMT_INT4_G32)
        return launch_fmt<MOE_FMT_INT4_G32>(ex, x, T, k, ids, y, ws, s);
    return launch_fmt<MOE_FMT_INT6_G32>(ex, x, T, k, ids, y, ws, s);
}

}  // namespace moe
