// route.hip -- router logits, top-k selection and gate weights on gfx950.
//
// The pages keep the router on the GPU and send each token to 10 of 512 routed experts
// [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法;
//  Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].  They fix no
// summation order; selection compares fp32 logits, so the order is part of the contract
// (see include/moe.h): 16-byte vectors dealt round-robin to 64 lanes, one fused
// multiply-add chain per lane, then a butterfly over lanes with offsets 1..32.  Both
// kernels below realise exactly that order, so decode (few tokens) and prefill (many
// tokens) produce identical logits for the same token.
#include "moe_common.h"
#include "topk_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// ------------------------------------------------------------------ few tokens: GEMV
// One wave per expert row.  Lane l holds its vectors v = l + 64 j of the row in
// registers and walks them for every token; the butterfly is a shuffle-xor tree.
// PV = elements per 16-byte vector (4 fp32 or 16 int8); NV = vectors per lane.
template <int FMT, int NV, bool DEVICE_SCOPE_STORE>
__device__ __forceinline__ void router_gemv_rows(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* logits) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;

    float w[NV][PV];
    if constexpr (FMT == MOE_FMT_INT8_ROW) {
        const uint4* row = reinterpret_cast<const uint4*>(
            static_cast<const int8_t*>(W) + (size_t)e * d);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            uint4 v = row[lane + 64 * j];
            uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 16; ++i)
                w[j][i] = (float)(int8_t)((wd[i >> 2] >> (8 * (i & 3))) & 0xffu);
        }
    } else {
        const float4* row = reinterpret_cast<const float4*>(
            static_cast<const float*>(W) + (size_t)e * d);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float4 v = row[lane + 64 * j];
            w[j][0] = v.x; w[j][1] = v.y; w[j][2] = v.z; w[j][3] = v.w;
        }
    }
    const float b = bias ? bias[e] : 0.0f;
    const float se = (FMT == MOE_FMT_INT8_ROW) ? f16_to_f32(scale[e]) : 1.0f;

    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (size_t)t * d;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c0 = (lane + 64 * j) * PV;
            if constexpr (PV == 4) {
                uint2 xv = *reinterpret_cast<const uint2*>(xt + c0);
                acc = __builtin_fmaf(bf16lo(xv.x), w[j][0], acc);
                acc = __builtin_fmaf(bf16hi(xv.x), w[j][1], acc);
                acc = __builtin_fmaf(bf16lo(xv.y), w[j][2], acc);
                acc = __builtin_fmaf(bf16hi(xv.y), w[j][3], acc);
            } else {
                const uint4* xp = reinterpret_cast<const uint4*>(xt + c0);
                uint4 a = xp[0], bq = xp[1];
                uint32_t xs[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc = __builtin_fmaf(bf16lo(xs[i]), w[j][2 * i], acc);
                    acc = __builtin_fmaf(bf16hi(xs[i]), w[j][2 * i + 1], acc);
                }
            }
        }
        acc = group_sum<64>(acc);     // butterfly over xor offsets 1..32
        if (lane == 0) {
            float l = acc;
            if constexpr (FMT == MOE_FMT_INT8_ROW) l = l * se;
            if (bias) l = l + b;
            if constexpr (DEVICE_SCOPE_STORE)
                __hip_atomic_store(logits + (size_t)t * E + e, l, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            else
                logits[(size_t)t * E + e] = l;
        }
    }
}

// ------------------------------------------------------------------ many tokens: GEMM
// A 64-token x 64-expert tile per block of 256 threads; each thread owns 4 tokens x 4
// experts.  The reduction is walked lane by lane of the contract's 64 virtual lanes:
// for virtual lane l the thread runs the fma chain over that lane's EL elements (in the
// contract's order), then folds the lane sum into a 6-deep pairwise stack, which
// reproduces the butterfly's tree ((a0+a1)+(a2+a3))+... exactly.
// The chunk staged in LDS holds KC = 64 chain elements = LC virtual lanes.
constexpr int RT_TM = 64, RT_TE = 64, RT_KC = 64;

template <int FMT, int NV>
__global__ void __launch_bounds__(256) router_gemm_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    constexpr int EL = NV * PV;          // chain elements per virtual lane
    constexpr int LC = RT_KC / EL;       // virtual lanes per chunk
    static_assert(RT_KC % EL == 0, "lane chain must divide the chunk");

    __shared__ float xs[RT_KC][RT_TM];
    __shared__ float ws[RT_KC][RT_TE];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int t0 = blockIdx.x * RT_TM, e0 = blockIdx.y * RT_TE;

    float stk[6][4][4];
    float acc[4][4];

    // staging: (row, j) pieces of LC*PV contiguous elements
    constexpr int PIECE = LC * PV;       // elements per piece
    constexpr int PIECES = NV;           // pieces per row per chunk

    for (int l0 = 0; l0 < 64; l0 += LC) {
        __syncthreads();
        // x tile: RT_TM rows x PIECES pieces of PIECE bf16
        for (int q = tid; q < RT_TM * PIECES * (PIECE / 4); q += 256) {
            const int r = q / (PIECES * (PIECE / 4));
            const int rem = q % (PIECES * (PIECE / 4));
            const int j = rem / (PIECE / 4);
            const int c4 = rem % (PIECE / 4);               // 4-element slot in the piece
            const int t = t0 + r;
            uint2 v = make_uint2(0u, 0u);
            const int cbase = (l0 + 64 * j) * PV + 4 * c4;
            if (t < T) v = *reinterpret_cast<const uint2*>(x + (size_t)t * d + cbase);
            // element e_in_piece = 4*c4 + i belongs to virtual lane l0 + (4*c4+i)/PV at
            // chain position j*PV + (4*c4+i)%PV
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ep = 4 * c4 + i;
                const int kk = (ep / PV) * EL + j * PV + (ep % PV);
                const uint32_t word = (i < 2) ? v.x : v.y;
                xs[kk][r] = (i & 1) ? bf16hi(word) : bf16lo(word);
            }
        }
        // w tile
        if constexpr (FMT == MOE_FMT_INT8_ROW) {
            for (int q = tid; q < RT_TE * PIECES * (PIECE / 4); q += 256) {
                const int r = q / (PIECES * (PIECE / 4));
                const int rem = q % (PIECES * (PIECE / 4));
                const int j = rem / (PIECE / 4);
                const int c4 = rem % (PIECE / 4);
                const int e = e0 + r;
                uint32_t v = 0u;
                const int cbase = (l0 + 64 * j) * PV + 4 * c4;
                if (e < E)
                    v = *reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(W) +
                                                           (size_t)e * d + cbase);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ep = 4 * c4 + i;
                    const int kk = (ep / PV) * EL + j * PV + (ep % PV);
                    ws[kk][r] = (float)(int8_t)((v >> (8 * i)) & 0xffu);
                }
            }
        } else {
            for (int q = tid; q < RT_TE * PIECES * (PIECE / 4); q += 256) {
                const int r = q / (PIECES * (PIECE / 4));
                const int rem = q % (PIECES * (PIECE / 4));
                const int j = rem / (PIECE / 4);
                const int c4 = rem % (PIECE / 4);
                const int e = e0 + r;
                float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                const int cbase = (l0 + 64 * j) * PV + 4 * c4;
                if (e < E)
                    v = *reinterpret_cast<const float4*>(static_cast<const float*>(W) +
                                                         (size_t)e * d + cbase);
                const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ep = 4 * c4 + i;
                    const int kk = (ep / PV) * EL + j * PV + (ep % PV);
                    ws[kk][r] = vv[i];
                }
            }
        }
        __syncthreads();

#pragma unroll
        for (int ll = 0; ll < LC; ++ll) {
            const int l = l0 + ll;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
#pragma unroll 8
            for (int kk = ll * EL; kk < (ll + 1) * EL; ++kk) {
                const float4 xv = *reinterpret_cast<const float4*>(&xs[kk][ty * 4]);
                const float4 wv = *reinterpret_cast<const float4*>(&ws[kk][tx * 4]);
                const float xa[4] = {xv.x, xv.y, xv.z, xv.w};
                const float wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc[a][b] = __builtin_fmaf(xa[a], wa[b], acc[a][b]);
            }
            // fold lane l's sum into the pairwise stack
            const int nlev = __builtin_ctz(~l);   // trailing one bits of l
#pragma unroll
            for (int lev = 0; lev < 6; ++lev) {
                if (lev < nlev) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) acc[a][b] = stk[lev][a][b] + acc[a][b];
                }
            }
#pragma unroll
            for (int lev = 0; lev < 6; ++lev) {
                if (lev == nlev) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
#pragma unroll
                        for (int b = 0; b < 4; ++b) stk[lev][a][b] = acc[a][b];
                }
            }
        }
    }
    // after l = 63 the full tree sum is in acc (nlev = 6 -> not stored)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int t = t0 + ty * 4 + a;
        if (t >= T) continue;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e = e0 + tx * 4 + b;
            if (e >= E) continue;
            float l = acc[a][b];
            if constexpr (FMT == MOE_FMT_INT8_ROW) l = l * f16_to_f32(scale[e]);
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
    }
}

// ------------------------------------------------------------------ top-k + weights
// One wave per token: topk_wave (topk_common.h).
template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
    __shared__ uint64_t scratch[4][128];
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int e;
    float w;
    topk_wave<NPL, false>(logits + (size_t)t * E, E, k, scratch[threadIdx.x >> 6], e, w);
    const int lane = threadIdx.x & 63;
    if (lane < k) {
        ids[(size_t)t * k + lane] = e;
        weights[(size_t)t * k + lane] = w;
    }
}

// Few tokens: logits and selection in one launch.  Every block computes its rows' logits
// for all tokens, writes them with device-scope stores, waits for those stores, then
// counts itself in; the last block to arrive reads every logit with device-scope loads,
// runs the selection for all tokens and resets the counter, leaving the workspace as it
// found it.  No cache-wide flush or invalidation is involved.
template <int FMT, int NV, int NPL>
__global__ void __launch_bounds__(256) router_gemv_topk_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d, int k,
    float* logits, int32_t* __restrict__ ids, float* __restrict__ weights, unsigned* counter) {
    router_gemv_rows<FMT, NV, true>(W, scale, bias, x, T, E, d, logits);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // this block's stores done
    __syncthreads();
    __shared__ int is_last;
    __shared__ uint64_t scratch[4][128];
    if (threadIdx.x == 0) is_last = (atomicAdd(counter, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (!is_last) return;
    const int lane = threadIdx.x & 63;
    for (int t = threadIdx.x >> 6; t < T; t += 4) {
        int e;
        float w;
        topk_wave<NPL, true>(logits + (size_t)t * E, E, k, scratch[threadIdx.x >> 6], e, w);
        if (lane < k) {
            ids[(size_t)t * k + lane] = e;
            weights[(size_t)t * k + lane] = w;
        }
    }
    if (threadIdx.x == 0) atomicExch(counter, 0u);
}

// Logits only, for a consumer that runs the selection itself (the decode layer).
template <int FMT, int NV>
__global__ void __launch_bounds__(256) router_gemv_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits) {
    router_gemv_rows<FMT, NV, false>(W, scale, bias, x, T, E, d, logits);
}

template <int FMT, int NV>
hipError_t launch_nv(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                     float* weights, float* logits, unsigned* counter, hipStream_t s) {
    const int E = r.n_experts, d = r.d_model;
    const int npl = (E + 63) / 64;
    if (T <= 16) {   // few tokens: one wave per expert row, selection by the last block
        const dim3 grid((E + 3) / 4), block(256);
#define MOE_GT(N)                                                                         \
    router_gemv_topk_kernel<FMT, NV, N><<<grid, block, 0, s>>>(r.w, r.scale, r.bias, x, T, \
                                                               E, d, k, logits, ids, weights, \
                                                               counter)
        if (npl <= 1) MOE_GT(1);
        else if (npl <= 2) MOE_GT(2);
        else if (npl <= 4) MOE_GT(4);
        else if (npl <= 8) MOE_GT(8);
        else MOE_GT(16);
#undef MOE_GT
        return hipGetLastError();
    }
    router_gemm_kernel<FMT, NV>
        <<<dim3((T + RT_TM - 1) / RT_TM, (E + RT_TE - 1) / RT_TE), dim3(256), 0, s>>>(
            r.w, r.scale, r.bias, x, T, E, d, logits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid((T + 3) / 4), block(256);
    if (npl <= 1)
        topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
    else if (npl <= 2)
        topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
    else if (npl <= 4)
        topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
    else if (npl <= 8)
        topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
    else
        topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, ids, weights);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                      float* weights, float* logits, unsigned* counter, hipStream_t s) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int nv = r.d_model / (64 * PV);
    // chain length per lane must divide the GEMM kernel's 64-element chunk
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        if constexpr (RT_KC % (N * PV) == 0)                                              \
            return launch_nv<FMT, N>(r, x, T, k, ids, weights, logits, counter, s);       \
        else                                                                              \
            return hipErrorInvalidValue;                                                  \
    }
    MOE_NV(1)
    MOE_NV(2)
    MOE_NV(4)
    MOE_NV(8)
    MOE_NV(16)
#undef MOE_NV
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_logits_fmt(const moe_router& r, const uint16_t* x, int T, float* logits,
                             hipStream_t s) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int nv = r.d_model / (64 * PV);
    const dim3 grid((r.n_experts + 3) / 4), block(256);
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        router_gemv_kernel<FMT, N><<<grid, block, 0, s>>>(r.w, r.scale, r.bias, x, T,     \
                                                          r.n_experts, r.d_model, logits);\
        return hipGetLastError();                                                         \
    }
    MOE_NV(1)
    MOE_NV(2)
    MOE_NV(4)
    MOE_NV(8)
    MOE_NV(16)
#undef MOE_NV
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route_logits(const moe_router& r, const uint16_t* x, int T, float* logits,
                               hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW) return launch_logits_fmt<MOE_FMT_INT8_ROW>(r, x, T, logits, s);
    return launch_logits_fmt<MOE_FMT_FP32>(r, x, T, logits, s);
}

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, unsigned* counter, hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_fmt<MOE_FMT_INT8_ROW>(r, x, T, k, ids, weights, logits, counter, s);
    return launch_fmt<MOE_FMT_FP32>(r, x, T, k, ids, weights, logits, counter, s);
}

}  // namespace moe
