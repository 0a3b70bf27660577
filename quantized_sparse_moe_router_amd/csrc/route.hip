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
// One wave per token.  Each (logit, expert) becomes a 64-bit key whose unsigned order is
// the selection order: the logit's bits mapped to an order-preserving unsigned integer
// (-0 first turned into +0 so the two compare equal) in the high word, and 0xffffffff - e
// in the low word so that equal logits favour the lower expert id.  k rounds of a wave
// max over the lanes' best untaken keys pick the experts in slot order; then the weights
// are the softmax over the k selected logits in fp32, shifted by the largest.
__device__ __forceinline__ uint32_t order_bits(float v) {
    uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

// Selection and weights of one token by one wave.  Keys are 64-bit: the logit's bits mapped
// to an order-preserving unsigned integer in the high word, 0xffffffff - e in the low word,
// so "larger key" is "larger logit, then lower id".  Each lane sorts its NPL keys once;
// each of the k rounds takes the wave maximum of the lanes' heads (DPP inside 16-lane rows,
// then the four row maxima on the scalar unit) and the owning lane advances its head.
template <int NPL, bool DEVICE_SCOPE_LOAD>
__device__ __forceinline__ void topk_token(const float* lt, int E, int k, int32_t* ids_t,
                                           float* w_t) {
    const int lane = threadIdx.x & 63;
    uint64_t key[NPL];
    float v[NPL];
    // all loads first, unconditionally (clamped index), so they are in flight together
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        if constexpr (DEVICE_SCOPE_LOAD)
            v[i] = __hip_atomic_load(const_cast<float*>(lt) + e, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        else
            v[i] = lt[e];
    }
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? (((uint64_t)order_bits(v[i]) << 32) | (0xffffffffu - (uint32_t)e))
                         : 0ull;                       // padding keys lose to every id
    }
    // descending sort of the lane's keys (odd-even transposition network)
#pragma unroll
    for (int r = 0; r < NPL; ++r)
#pragma unroll
        for (int i = r & 1; i + 1 < NPL; i += 2) {
            const uint64_t a = key[i], b = key[i + 1];
            key[i] = a > b ? a : b;
            key[i + 1] = a > b ? b : a;
        }
    uint64_t mine = 0ull;
    int head = 0;                                      // index of the lane's next key
    for (int j = 0; j < k; ++j) {
        uint64_t b = 0ull;
#pragma unroll
        for (int i = 0; i < NPL; ++i) b = (head == i) ? key[i] : b;
        const uint64_t cand = b;
        uint64_t o;
        o = dpp64<kDppXor1>(b);       b = o > b ? o : b;
        o = dpp64<kDppXor2>(b);       b = o > b ? o : b;
        o = dpp64<kDppHalfMirror>(b); b = o > b ? o : b;
        o = dpp64<kDppMirror>(b);     b = o > b ? o : b;
        uint64_t win = readlane64(b, 0);
#pragma unroll
        for (int r = 16; r < 64; r += 16) {
            const uint64_t c = readlane64(b, r);
            win = c > win ? c : win;
        }
        // keys are unique (the low word holds the id): exactly one lane owns the winner
        head += (cand == win) ? 1 : 0;
        if (lane == j) mine = win;
    }
    const uint32_t my_hi = (uint32_t)(mine >> 32), my_lo = (uint32_t)mine;
    const int my_e = (int)(0xffffffffu - my_lo);
    const uint32_t vbits = (my_hi & 0x80000000u) ? (my_hi & 0x7fffffffu) : ~my_hi;
    const float my_v = (lane < k) ? __uint_as_float(vbits) : 0.0f;
    const float vmax = __shfl(my_v, 0, 64);
    const float ex = (lane < k) ? expf(my_v - vmax) : 0.0f;
    const float sum = group_sum<64>(ex);
    if (lane < k) {
        ids_t[lane] = my_e;
        w_t[lane] = ex / sum;
    }
}

template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    topk_token<NPL, false>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                           weights + (size_t)t * k);
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
    if (threadIdx.x == 0) is_last = (atomicAdd(counter, 1u) == gridDim.x - 1) ? 1 : 0;
    __syncthreads();
    if (!is_last) return;
    for (int t = threadIdx.x >> 6; t < T; t += 4)
        topk_token<NPL, true>(logits + (size_t)t * E, E, k, ids + (size_t)t * k,
                              weights + (size_t)t * k);
    if (threadIdx.x == 0) atomicExch(counter, 0u);
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

}  // namespace

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, unsigned* counter, hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_fmt<MOE_FMT_INT8_ROW>(r, x, T, k, ids, weights, logits, counter, s);
    return launch_fmt<MOE_FMT_FP32>(r, x, T, k, ids, weights, logits, counter, s);
}

}  // namespace moe
