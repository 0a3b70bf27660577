// route.hip -- router logits, top-k selection and gate weights on gfx950.
//
// The pages keep the router on the GPU and send each token to 10 of 512 routed experts
// [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法;
//  Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].  They fix no
// summation order; selection compares fp32 logits, so the order is part of the contract
// (see include/moe.h): 16-byte vectors dealt round-robin to 64 lanes, one fused
// multiply-add chain per lane, then a butterfly over lanes with offsets 1..32.  The GEMV
// (few tokens) and the LDS-tiled GEMM (many tokens, logits wanted) realise exactly that
// order, so they produce identical logits for the same token; the bounded selection (many
// tokens, no logits wanted) recomputes in that order every expert its MFMA logits cannot
// rule out, so all forms select alike.
#include "moe_common.h"
#include "norm_common.h"
#include "topk_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

// ------------------------------------------------------------------ few tokens: GEMV
// One wave per expert row.  Lane l holds its vectors v = l + 64 j of the row in
// registers and walks them for every token, a few tokens at a time (their activation loads
// issued together, one unchanged chain per token); the butterfly is a shuffle-xor tree.
// PV = elements per 16-byte vector (4 fp32 or 16 int8); NV = vectors per lane.
//
// NORM: the tokens are the layer's un-normalised input; every wave computes a token's
// norm scale itself (norm_common.h) and uses xn = RMSNorm(x) in its dot products, the wave
// of row 0 stores xn [T][d], and the wave of row E (one past the experts) computes the
// residual-gate logit z [T] instead of an expert logit.
struct RouteNorm {
    const float* gamma;   // [d]
    float eps;
    const float* gw;      // [d] gate row, or null: no gate logit
    float gb;
    uint16_t* xn;         // [T][d]
    float* z;             // [T]
};

// Row e's vectors lane + 64 j, j < NV, of the lane into registers (int8 codes as floats).
template <int FMT, int NV, int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4>
__device__ __forceinline__ void router_row_regs(const void* __restrict__ W, int e, int d,
                                                int lane, float (&w)[NV][PV]) {
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
}

template <int FMT, int NV, bool DEVICE_SCOPE_STORE, int WPB = 4, bool NORM = false>
__device__ __forceinline__ void router_gemv_rows(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* logits, const RouteNorm& nm = RouteNorm{}) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    constexpr int NC = NV * PV / 4;          // the norm's 4-element chunks per lane
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * WPB + (threadIdx.x >> 6);   // WPB rows (waves) per block
    if constexpr (NORM) {
        if (e == E && nm.gw) {               // the gate row
            for (int t = 0; t < T; ++t) {
                uint2 x4[NC];
                const float ss = group_sum<64>(rms_lane_sumsq<NC>(x + (size_t)t * d, lane, x4));
                const float r = rms_scale(ss, d, nm.eps);
                const float zt = rms_row_and_gate<NC>(x4, lane, r, nm.gamma, nm.gw, nm.gb,
                                                      nullptr);
                if (lane == 0) nm.z[t] = zt;
            }
            return;
        }
    }
    if (e >= E) return;

    float w[NV][PV];
    router_row_regs<FMT, NV>(W, e, d, lane, w);
    const float b = bias ? bias[e] : 0.0f;
    const float se = (FMT == MOE_FMT_INT8_ROW) ? f16_to_f32(scale[e]) : 1.0f;
    // NORM: gamma of the lane's elements, in registers for every token
    float gam[NORM ? NV : 1][NORM ? PV : 1];
    if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int q = 0; q < PV / 4; ++q) {
                const float4 g4 =
                    *reinterpret_cast<const float4*>(nm.gamma + (lane + 64 * j) * PV + 4 * q);
                gam[j][4 * q] = g4.x; gam[j][4 * q + 1] = g4.y;
                gam[j][4 * q + 2] = g4.z; gam[j][4 * q + 3] = g4.w;
            }
    }
    // NORM: the norm's chunks of the next token, requested before the current token's work
    uint2 x4n[NORM ? NC : 1];
    if constexpr (NORM) {
#pragma unroll
        for (int j = 0; j < NC; ++j)
            x4n[j] = *reinterpret_cast<const uint2*>(x + (lane + 64 * j) * 4);
        // the row, gamma and the first token's chunks stay in these registers for the whole
        // token loop: all requested above, awaited here once (left alone, the compiler
        // issues and awaits them piece by piece inside the loop)
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int i = 0; i < PV; ++i) asm volatile("" : "+v"(w[j][i]), "+v"(gam[j][i]));
#pragma unroll
        for (int j = 0; j < NC; ++j) asm volatile("" : "+v"(x4n[j].x), "+v"(x4n[j].y));
    }

    if constexpr (!NORM) {
        // G tokens at a time: every activation load of the group is issued before the first
        // fma, and the G chains (each in its own, unchanged order) run interleaved
        constexpr int G = (NV * PV <= 32) ? 4 : (NV * PV <= 64) ? 2 : 1;
        constexpr int XW = PV / 2;           // 32-bit words of activations per vector
        for (int t0 = 0; t0 < T; t0 += G) {
            uint32_t xq[G][NV][XW];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint16_t* xt = x + (size_t)min(t0 + g, T - 1) * d;
#pragma unroll
                for (int j = 0; j < NV; ++j) {
                    const int c0 = (lane + 64 * j) * PV;
                    if constexpr (PV == 4) {
                        const uint2 v = *reinterpret_cast<const uint2*>(xt + c0);
                        xq[g][j][0] = v.x; xq[g][j][1] = v.y;
                    } else {
                        const uint4* xp = reinterpret_cast<const uint4*>(xt + c0);
                        const uint4 a = xp[0], bq = xp[1];
                        xq[g][j][0] = a.x; xq[g][j][1] = a.y; xq[g][j][2] = a.z;
                        xq[g][j][3] = a.w; xq[g][j][4] = bq.x; xq[g][j][5] = bq.y;
                        xq[g][j][6] = bq.z; xq[g][j][7] = bq.w;
                    }
                }
            }
            float acc[G];
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = 0.0f;
#pragma unroll
            for (int j = 0; j < NV; ++j)
#pragma unroll
                for (int i = 0; i < XW; ++i)
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        acc[g] = __builtin_fmaf(bf16lo(xq[g][j][i]), w[j][2 * i], acc[g]);
                        acc[g] = __builtin_fmaf(bf16hi(xq[g][j][i]), w[j][2 * i + 1], acc[g]);
                    }
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = group_sum<64>(acc[g]);
            if (lane == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int t = t0 + g;
                    if (t >= T) break;
                    float l = acc[g];
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
        return;
    }
    for (int t = 0; t < T; ++t) {
        const uint16_t* xt = x + (size_t)t * d;
        float r = 1.0f;
        uint2 x4[NORM ? NC : 1];
        if constexpr (NORM) {
#pragma unroll
            for (int j = 0; j < NC; ++j) x4[j] = x4n[j];
            if (t + 1 < T) {
#pragma unroll
                for (int j = 0; j < NC; ++j)
                    x4n[j] = *reinterpret_cast<const uint2*>(xt + d + (lane + 64 * j) * 4);
            }
            float ss = 0.0f;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const float a0 = bf16lo(x4[j].x), a1 = bf16hi(x4[j].x);
                const float a2 = bf16lo(x4[j].y), a3 = bf16hi(x4[j].y);
                ss = __builtin_fmaf(a0, a0, ss);
                ss = __builtin_fmaf(a1, a1, ss);
                ss = __builtin_fmaf(a2, a2, ss);
                ss = __builtin_fmaf(a3, a3, ss);
            }
            r = rms_scale(group_sum<64>(ss), d, nm.eps);
        }
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int c0 = (lane + 64 * j) * PV;
            if constexpr (PV == 4) {
                // under NORM the router's vectors are the norm's chunks: x4[j]
                uint2 xv;
                if constexpr (NORM) xv = x4[j];
                else xv = *reinterpret_cast<const uint2*>(xt + c0);
                if constexpr (NORM) {
                    xv.x = rms_apply_pair(bf16lo(xv.x), bf16hi(xv.x), r, gam[j][0], gam[j][1]);
                    xv.y = rms_apply_pair(bf16lo(xv.y), bf16hi(xv.y), r, gam[j][2], gam[j][3]);
                    if (e == 0) *reinterpret_cast<uint2*>(nm.xn + (size_t)t * d + c0) = xv;
                }
                acc = __builtin_fmaf(bf16lo(xv.x), w[j][0], acc);
                acc = __builtin_fmaf(bf16hi(xv.x), w[j][1], acc);
                acc = __builtin_fmaf(bf16lo(xv.y), w[j][2], acc);
                acc = __builtin_fmaf(bf16hi(xv.y), w[j][3], acc);
            } else {
                const uint4* xp = reinterpret_cast<const uint4*>(xt + c0);
                uint4 a = xp[0], bq = xp[1];
                uint32_t qs[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
                if constexpr (NORM) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        qs[i] = rms_apply_pair(bf16lo(qs[i]), bf16hi(qs[i]), r, gam[j][2 * i],
                                               gam[j][2 * i + 1]);
                    if (e == 0) {
                        uint4* dst = reinterpret_cast<uint4*>(nm.xn + (size_t)t * d + c0);
                        dst[0] = make_uint4(qs[0], qs[1], qs[2], qs[3]);
                        dst[1] = make_uint4(qs[4], qs[5], qs[6], qs[7]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    acc = __builtin_fmaf(bf16lo(qs[i]), w[j][2 * i], acc);
                    acc = __builtin_fmaf(bf16hi(qs[i]), w[j][2 * i + 1], acc);
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
// The contract's reduction laid out across a wave: lane l runs virtual lane l's fma chain
// (its vectors l + 64 j, elements in order) for every (token, expert) of the wave's tile,
// so each chain is a plain register accumulator; at the end the 64 lane sums of each
// output go through LDS and are added in the contract's tree (pairs of lanes, then pairs
// of pairs, ...), which is the butterfly's tree.
// Block = 8 waves, 4 along tokens x 2 along experts; wave tile TW tokens x EW experts.
// Step j stages the 64 vectors of index j (a contiguous slice of the reduction dim) of
// the block's token and expert rows in LDS, double-buffered; a step is taken in quarters
// of 4 elements per lane (one quarter for fp32 vectors, four for int8 vectors).
template <int FMT>
struct RgShape {
    static constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;   // elements per vector
    static constexpr int NQ = PV / 4;                                // quarters per step
    static constexpr int TW = (FMT == MOE_FMT_INT8_ROW) ? 4 : 8;     // tokens per wave
    static constexpr int EW = (FMT == MOE_FMT_INT8_ROW) ? 16 : 12;   // experts per wave
    static constexpr int BT = 4 * TW, BE = 2 * EW;                   // block tile
    static constexpr int WB = (FMT == MOE_FMT_INT8_ROW) ? 1 : 4;     // bytes per weight
    // one stage: x [BT][NQ][64][4] bf16, then W [BE][NQ][64][4]
    static constexpr int XS = BT * 64 * PV * 2;
    static constexpr int WS = BE * 64 * PV * WB;
    static constexpr int STAGE = XS + WS;
    static constexpr int RS = 68;          // reduction scratch row stride (floats)
    static_assert(8 * 32 * RS * 4 <= 2 * STAGE, "reduction scratch fits in the stages");
};

template <int FMT, int NV>
__global__ void __launch_bounds__(512) router_gemm_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits) {
    using R = RgShape<FMT>;
    constexpr int PV = R::PV, NQ = R::NQ, TW = R::TW, EW = R::EW, BT = R::BT, BE = R::BE;
    constexpr int SL = 64 * PV;                       // slice elements per step
    constexpr int XCH = BT * SL / 8 / 512;            // 16-byte x chunks per thread
    constexpr int WCH = BE * SL * R::WB / 16 / 512;   // 16-byte W chunks per thread
    static_assert(XCH >= 1 && WCH >= 1, "every thread stages whole chunks");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * BT, e0 = blockIdx.y * BE;
    const int tw0 = (wave >> 1) * TW, ew0 = (wave & 1) * EW;   // wave tile inside the block

    // ---- staging: this thread's chunks of step j -> registers; registers -> LDS stage
    // native 4-vectors: an array of HIP's uint4 struct is not kept in registers
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x4 xr[XCH], wr[WCH];
    auto load_step = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < XCH; ++u) {
            const int c = tid + 512 * u, row = c / (SL / 8), cc = c % (SL / 8);
            const int t = min(t0 + row, T - 1);
            xr[u] = *reinterpret_cast<const u32x4*>(x + (size_t)t * d + (size_t)SL * j + 8 * cc);
        }
#pragma unroll
        for (int u = 0; u < WCH; ++u) {
            constexpr int CPR = SL * R::WB / 16;      // chunks per W row
            const int c = tid + 512 * u, row = c / CPR, cc = c % CPR;
            const int e = min(e0 + row, E - 1);
            wr[u] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(W) +
                                                    ((size_t)e * d + (size_t)SL * j) * R::WB +
                                                    16 * cc);
        }
    };
    auto store_step = [&](int st) __attribute__((always_inline)) {
        uint8_t* xs = smem + st * R::STAGE;
        uint8_t* ws = xs + R::XS;
#pragma unroll
        for (int u = 0; u < XCH; ++u) {
            const int c = tid + 512 * u, row = c / (SL / 8), cc = c % (SL / 8);
            if constexpr (PV == 4) {
                // elements 8 cc .. 8 cc + 7 = lanes 2 cc, 2 cc + 1, quarter 0
                *reinterpret_cast<u32x4*>(xs + ((row * 64 + 2 * cc) * 4) * 2) = xr[u];
            } else {
                // lane cc / 2, quarters 2 (cc % 2) and 2 (cc % 2) + 1
                const int l = cc >> 1, q0 = 2 * (cc & 1);
                *reinterpret_cast<u32x2*>(xs + (((row * NQ + q0) * 64 + l) * 4) * 2) =
                    u32x2{xr[u].x, xr[u].y};
                *reinterpret_cast<u32x2*>(xs + (((row * NQ + q0 + 1) * 64 + l) * 4) * 2) =
                    u32x2{xr[u].z, xr[u].w};
            }
        }
#pragma unroll
        for (int u = 0; u < WCH; ++u) {
            constexpr int CPR = SL * R::WB / 16;
            const int c = tid + 512 * u, row = c / CPR, cc = c % CPR;
            if constexpr (PV == 4) {
                // fp32: 4 elements = lane cc, quarter 0
                *reinterpret_cast<u32x4*>(ws + ((row * 64 + cc) * 4) * 4) = wr[u];
            } else {
                // int8: 16 elements = lane cc, quarters 0..3, 4 bytes each
                const uint32_t v[4] = {wr[u].x, wr[u].y, wr[u].z, wr[u].w};
#pragma unroll
                for (int q = 0; q < NQ; ++q)
                    *reinterpret_cast<uint32_t*>(ws + ((row * NQ + q) * 64 + cc) * 4) = v[q];
            }
        }
    };

    float acc[TW][EW];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int e = 0; e < EW; ++e) acc[t][e] = 0.0f;

    load_step(0);
    store_step(0);
    __syncthreads();
    for (int j = 0; j < NV; ++j) {
        const int st = j & 1;
        if (j + 1 < NV) load_step(j + 1);
        const uint8_t* xs = smem + st * R::STAGE;
        const uint8_t* ws = xs + R::XS;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float xv[TW][4];
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const uint2 p = *reinterpret_cast<const uint2*>(
                    xs + ((((tw0 + t) * NQ + q) * 64 + lane) * 4) * 2);
                xv[t][0] = bf16lo(p.x); xv[t][1] = bf16hi(p.x);
                xv[t][2] = bf16lo(p.y); xv[t][3] = bf16hi(p.y);
            }
#pragma unroll
            for (int e = 0; e < EW; ++e) {
                float wv[4];
                if constexpr (PV == 4) {
                    const float4 f = *reinterpret_cast<const float4*>(
                        ws + (((ew0 + e) * 64 + lane) * 4) * 4);
                    wv[0] = f.x; wv[1] = f.y; wv[2] = f.z; wv[3] = f.w;
                } else {
                    const uint32_t b = *reinterpret_cast<const uint32_t*>(
                        ws + (((ew0 + e) * NQ + q) * 64 + lane) * 4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) wv[r] = (float)(int8_t)((b >> (8 * r)) & 0xffu);
                }
#pragma unroll
                for (int t = 0; t < TW; ++t)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        acc[t][e] = __builtin_fmaf(xv[t][r], wv[r], acc[t][e]);
            }
        }
        if (j + 1 < NV) store_step(st ^ 1);
        __syncthreads();
    }

    // ---- the 64 lane sums of each output, in the tree, 32 outputs at a time: lane L
    // adds lanes 32 (L / 32) .. + 31 of output L % 32 pairwise, then the two halves
    float* scr = reinterpret_cast<float*>(smem) + wave * 32 * R::RS;
    const int ol = lane & 31, half = lane >> 5;
#pragma unroll
    for (int c0 = 0; c0 < TW * EW; c0 += 32) {
#pragma unroll
        for (int i = 0; i < 32; ++i) scr[i * R::RS + lane] = acc[(c0 + i) / EW][(c0 + i) % EW];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float v[32];
#pragma unroll
        for (int m = 0; m < 32; m += 4) {
            const float4 f = *reinterpret_cast<const float4*>(scr + ol * R::RS + 32 * half + m);
            v[m] = f.x; v[m + 1] = f.y; v[m + 2] = f.z; v[m + 3] = f.w;
        }
#pragma unroll
        for (int w = 1; w < 32; w <<= 1)
#pragma unroll
            for (int m = 0; m < 32; m += 2 * w) v[m] = v[m] + v[m + w];
        const float other = __shfl_xor(v[0], 32, 64);
        const float sum = v[0] + other;
        const int o = c0 + ol, t = t0 + tw0 + o / EW, e = e0 + ew0 + o % EW;
        if (half == 0 && t < T && e < E) {
            float l = sum;
            if constexpr (FMT == MOE_FMT_INT8_ROW) l = l * f16_to_f32(scale[e]);
            if (bias) l = l + bias[e];
            logits[(size_t)t * E + e] = l;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// ------------------------------------------------------------------ many tokens: bounded
// Selection from the MFMA logits lf (route_mfma.hip), which satisfy
//     |lf[t][e] - logit[t][e]| <= B_e = 2^-11 (|x_t| nw[e] + |b_e|)
// where logit is the fixed-order value.  One wave per token:
//   1. lo_e = lf - B_e, hi_e = lf + B_e; theta = the k-th largest of the lanes' largest lo
//      (so at least k experts have logit >= lo >= theta);
//   2. candidates: hi_e >= theta (any other expert's logit is below theta, hence below k
//      others: it cannot be selected, and cannot tie a selected one); experts whose
//      bound is not finite, or whose |x_t| nw[e] is so small (below 2^-90) that products
//      may underflow, are candidates whatever their value;
//   3. each candidate's logit recomputed exactly in the fixed order (the wave holds x_t
//      in the order's layout, as the few-token kernel holds the weight row);
//   4. the selection among the candidates (exact values; rank_candidates, or the general
//      selection over the row when more than 64): every non-candidate value is below theta
//      and at least k candidates are at or above it, so the k selected are the k largest
//      exact logits, in the same order and with the same weights as the exact path computes.
template <int FMT, int NV, int NPL>
__global__ void __launch_bounds__(256) route_bounded_select_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x,
    const float* __restrict__ nw, const float* __restrict__ lf, int T, int E, int d, int k,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;   // elements per 16-byte vector
    constexpr int XW = PV / 2;                                 // x words (bf16 pairs) per vector
    __shared__ uint64_t scratch[4][128];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;

    // ---- loads: x_t in the fixed order's layout (lane l: vectors l + 64 j), the bounded
    // logits, the row norms and the bias
    uint32_t xw[NV][XW];
    const uint16_t* xt = x + (size_t)t * d;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(xt + (lane + 64 * j) * PV);
        if constexpr (PV == 4) {
            const uint2 q = *reinterpret_cast<const uint2*>(src);
            xw[j][0] = q.x; xw[j][1] = q.y;
        } else {
            const uint4 a = reinterpret_cast<const uint4*>(src)[0];
            const uint4 b = reinterpret_cast<const uint4*>(src)[1];
            xw[j][0] = a.x; xw[j][1] = a.y; xw[j][2] = a.z; xw[j][3] = a.w;
            xw[j][4] = b.x; xw[j][5] = b.y; xw[j][6] = b.z; xw[j][7] = b.w;
        }
    }
    float v[NPL], nwe[NPL], be[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        v[i] = lf[(size_t)t * E + e];
        nwe[i] = nw[e];
        be[i] = bias ? bias[e] : 0.0f;
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int w = 0; w < XW; ++w) {
            const float a = bf16lo(xw[j][w]), b = bf16hi(xw[j][w]);
            ss = __builtin_fmaf(a, a, ss);
            ss = __builtin_fmaf(b, b, ss);
        }
    const float nx = sqrtf(group_sum<64>(ss)) * (1.0f + 0x1p-10f);

    // ---- 1, 2: threshold and candidates
    uint32_t lokey[NPL], hikey[NPL];
    bool force[NPL];
    uint32_t lmax = 0u;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const bool valid = lane + 64 * i < E;
        const float xn = nx * nwe[i];
        const float B = 0x1p-11f * (xn + fabsf(be[i]));
        const float lo = v[i] - B, hi = v[i] + B;
        const bool fin = __builtin_isfinite(lo) && __builtin_isfinite(hi);
        const bool tiny = xn > 0.0f && xn < 0x1p-90f;
        force[i] = valid && (!fin || tiny);
        lokey[i] = (valid && fin) ? order_bits(lo) : 0u;
        hikey[i] = (valid && fin) ? order_bits(hi) : 0u;
        lmax = lokey[i] > lmax ? lokey[i] : lmax;
    }
    uint32_t theta = 0u;
#pragma unroll
    for (int b = 31; b >= 0; --b) {
        const uint32_t c = theta | (1u << b);
        if (__popcll(__ballot(lmax >= c)) >= k) theta = c;
    }
    uint64_t bal[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i)
        bal[i] = __ballot(lane + 64 * i < E && (force[i] || hikey[i] >= theta));

    // ---- 3: exact logits of the candidates, NB at a time (raw 16-byte vectors of their
    // rows in flight together, converted inside the chain)
    constexpr int NB = (FMT == MOE_FMT_INT8_ROW) ? 4 : 2;
    uint64_t rest[NPL];
    int C = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        rest[i] = bal[i];
        C += __popcll(bal[i]);
    }
    auto pop = [&]() __attribute__((always_inline)) {
        int e = -1;
#pragma unroll
        for (int i = 0; i < NPL; ++i)
            if (e < 0 && rest[i]) {
                e = 64 * i + (int)__builtin_ctzll(rest[i]);
                rest[i] &= rest[i] - 1;
            }
        return e;
    };
    for (int done = 0; done < C; done += NB) {
        int ec[NB];
        uint4 raw[NB][NV];
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            const int e = pop();
            ec[c] = e;
            const int er = e >= 0 ? e : 0;
            const uint4* row = reinterpret_cast<const uint4*>(
                static_cast<const uint8_t*>(W) + (size_t)er * d * (PV == 4 ? 4 : 1));
#pragma unroll
            for (int j = 0; j < NV; ++j) raw[c][j] = row[lane + 64 * j];
        }
#pragma unroll
        for (int c = 0; c < NB; ++c) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const uint32_t wd[4] = {raw[c][j].x, raw[c][j].y, raw[c][j].z, raw[c][j].w};
#pragma unroll
                for (int w = 0; w < XW; ++w) {
                    float w0, w1;
                    if constexpr (FMT == MOE_FMT_INT8_ROW) {
                        w0 = (float)(int8_t)((wd[w >> 1] >> (16 * (w & 1))) & 0xffu);
                        w1 = (float)(int8_t)((wd[w >> 1] >> (16 * (w & 1) + 8)) & 0xffu);
                    } else {
                        w0 = __uint_as_float(wd[2 * w]);
                        w1 = __uint_as_float(wd[2 * w + 1]);
                    }
                    acc = __builtin_fmaf(bf16lo(xw[j][w]), w0, acc);
                    acc = __builtin_fmaf(bf16hi(xw[j][w]), w1, acc);
                }
            }
            acc = group_sum<64>(acc);     // butterfly over xor offsets 1..32
            const int e = ec[c];
            if (e >= 0) {
                float l = acc;
                if constexpr (FMT == MOE_FMT_INT8_ROW) l = l * f16_to_f32(scale[e]);
                if (bias) l = l + bias[e];
                if (lane == (e & 63)) {
#pragma unroll
                    for (int i = 0; i < NPL; ++i)
                        if (i == (e >> 6)) v[i] = l;
                }
            }
        }
    }

    // ---- 4: selection and weights among the candidates (exact values); more than 64
    // candidates (many equal logits) take the general selection over the whole row
    int sel_e;
    float sel_w;
    uint64_t key[NPL];
    make_keys<NPL>(v, E, key);
    const uint64_t mine = C <= 64 ? rank_candidates<NPL>(key, bal, C, k, scratch[wave])
                                  : select_keys<NPL>(key, k, scratch[wave]);
    finish_selection(mine, k, sel_e, sel_w);
    if (lane < k) {
        ids[(size_t)t * k + lane] = sel_e;
        weights[(size_t)t * k + lane] = sel_w;
    }
}

// Few tokens: logits and selection in one launch.  Every block computes its rows' logits
// for all tokens and writes them with device-scope atomic stores, which go through to the
// device's point of coherence.  Each wave then waits until its stores have completed
// (s_waitcnt vmcnt(0)), the block meets at a barrier, and one thread counts the block in
// with a device-scope atomic increment.  The last block to arrive reads every logit with
// device-scope atomic loads (served from the point of coherence, not from a stale cache),
// runs the selection for all tokens and resets the counter, leaving the workspace as it
// found it.  A release fence at device scope would also write back the whole L2 of each
// XCD (buffer_wbl2), measured at 3.7 us per call here; the completed device-scope
// stores already give the last block every logit.
template <int FMT, int NV, int NPL, bool NORM = false>
__global__ void __launch_bounds__(256) router_gemv_topk_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d, int k,
    float* logits, int32_t* __restrict__ ids, float* __restrict__ weights, unsigned* counter,
    RouteNorm nm) {
    router_gemv_rows<FMT, NV, true, 4, NORM>(W, scale, bias, x, T, E, d, logits, nm);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's stores have completed
    __syncthreads();
    __shared__ int is_last;
    __shared__ uint64_t scratch[4][128];
    if (threadIdx.x == 0)
        is_last = (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) ? 1 : 0;
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

// Logits only, for a consumer that runs the selection itself (the decode layer).  One
// wave (one expert row) per block: E blocks reach every CU, where blocks of 4 rows would
// leave half of them idle at E = 512.
template <int FMT, int NV, bool NORM = false>
__global__ void __launch_bounds__(64) router_gemv_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits, RouteNorm nm) {
    router_gemv_rows<FMT, NV, false, 1, NORM>(W, scale, bias, x, T, E, d, logits, nm);
}

// Logits of more tokens (the split form): block (c, b) computes rows NE c .. NE c + NE - 1
// for tokens [kRouteTokensPerWave b, kRouteTokensPerWave (b + 1)), so the token loop is
// short and ceil(E / NE) x ceil(T / kRouteTokensPerWave) waves share the work.  Every
// activation vector a wave loads serves its NE rows: the activations are the bulk of what
// the waves read (E T d bf16 over all waves with one row each, d fp32 per row).  Each
// (token, expert) chain and its butterfly are the GEMV's, so the logits are the same bits.
// From kRouteSplitBlockMinTokens tokens (and d <= 2048) blocks of kRouteSplitWaves waves
// take WB NE consecutive rows: the token group's activations go to LDS once per block and
// each wave reads them there, which divides the activation traffic through the caches by
// WB; below that a block of WB waves would leave CUs without work.
constexpr int kRouteTokensPerWave = 8;
constexpr int kRouteSplitWaves = 4;
constexpr int kRouteSplitBlockMinTokens = 17;
template <int FMT, int NV>
struct SplitShape {
    static constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    static constexpr int NE = (NV * PV <= 32) ? 2 : 1;                     // rows per wave
    static constexpr int G = (NV * PV <= 32) ? 4 : (NV * PV <= 64) ? 2 : 1;   // tokens per pass
};
template <int FMT, int NV, int WB>
__global__ void __launch_bounds__(64 * WB) router_gemv_split_kernel(
    const void* __restrict__ W, const uint16_t* __restrict__ scale,
    const float* __restrict__ bias, const uint16_t* __restrict__ x, int T, int E, int d,
    float* __restrict__ logits) {
    using SS = SplitShape<FMT, NV>;
    constexpr int PV = SS::PV, NE = SS::NE, G = SS::G;
    constexpr int XW = PV / 2;                  // 32-bit words of activations per vector
    constexpr int D = NV * 64 * PV;             // d of this instantiation
    constexpr int TPW = kRouteTokensPerWave;
    const int lane = threadIdx.x & 63;
    const int e0 = (blockIdx.x * WB + (threadIdx.x >> 6)) * NE;
    const int t_lo = blockIdx.y * TPW;
    const int t_hi = min(T, t_lo + TPW);
    // WB > 1: tokens t_lo .. t_lo + TPW - 1 (past T: the last token again, unused) in LDS
    __shared__ __attribute__((aligned(16))) uint16_t xs[WB > 1 ? TPW * D : 8];
    constexpr int XPT = WB > 1 ? TPW * D / 8 / (64 * WB) : 1;   // 16-byte pieces per thread
    static_assert(WB == 1 || XPT * 64 * WB * 8 == TPW * D, "whole pieces per thread");
    uint4 xv[XPT];
    if constexpr (WB > 1) {
        // requested before the rows, so that both round trips overlap
#pragma unroll
        for (int p = 0; p < XPT; ++p) {
            const int idx = (int)threadIdx.x + 64 * WB * p, tok = idx / (D / 8);
            xv[p] = reinterpret_cast<const uint4*>(x + (size_t)min(t_lo + tok, T - 1) * D)
                [idx % (D / 8)];
        }
    }
    float w[NE][NV][PV];
    float b[NE], se[NE];
#pragma unroll
    for (int r = 0; r < NE; ++r) {
        const int e = min(e0 + r, E - 1);       // a row past E repeats the last, unstored
        router_row_regs<FMT, NV>(W, e, d, lane, w[r]);
        b[r] = bias ? bias[e] : 0.0f;
        se[r] = (FMT == MOE_FMT_INT8_ROW) ? f16_to_f32(scale[e]) : 1.0f;
    }
    if constexpr (WB > 1) {
#pragma unroll
        for (int p = 0; p < XPT; ++p)
            reinterpret_cast<uint4*>(xs)[(int)threadIdx.x + 64 * WB * p] = xv[p];
        __syncthreads();
    }
    for (int t0 = t_lo; t0 < t_hi; t0 += G) {
        // every activation load of the pass before the first fma
        uint32_t xq[G][NV][XW];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint16_t* xt = WB > 1 ? xs + (size_t)min(t0 + g - t_lo, TPW - 1) * D
                                        : x + (size_t)min(t0 + g, T - 1) * d;
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int c0 = (lane + 64 * j) * PV;
                if constexpr (PV == 4) {
                    const uint2 v = *reinterpret_cast<const uint2*>(xt + c0);
                    xq[g][j][0] = v.x; xq[g][j][1] = v.y;
                } else {
                    const uint4* xp = reinterpret_cast<const uint4*>(xt + c0);
                    const uint4 a = xp[0], bq = xp[1];
                    xq[g][j][0] = a.x; xq[g][j][1] = a.y; xq[g][j][2] = a.z;
                    xq[g][j][3] = a.w; xq[g][j][4] = bq.x; xq[g][j][5] = bq.y;
                    xq[g][j][6] = bq.z; xq[g][j][7] = bq.w;
                }
            }
        }
        // acc[r * G + g]: row e0 + r, token t0 + g; NE x G chains, each in the GEMV's order
        float acc[NE * G][1];
#pragma unroll
        for (int q = 0; q < NE * G; ++q) acc[q][0] = 0.0f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int i = 0; i < XW; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float lo = bf16lo(xq[g][j][i]), hi = bf16hi(xq[g][j][i]);
#pragma unroll
                    for (int r = 0; r < NE; ++r) {
                        float& a = acc[r * G + g][0];
                        a = __builtin_fmaf(lo, w[r][j][2 * i], a);
                        a = __builtin_fmaf(hi, w[r][j][2 * i + 1], a);
                    }
                }
        // the butterflies of all NE x G chains at once (same tree, same bits); one lane
        // per (row, token) finishes it
        group_sum_many<64, NE * G, 1>(acc, lane);
        const int q = tr_index<64, NE * G>(lane);
        const int r = q / G, t = t0 + q % G;
        float l = acc[0][0], bb = b[0], ss = se[0];
#pragma unroll
        for (int rr = 1; rr < NE; ++rr)
            if (r == rr) {
                bb = b[rr];
                ss = se[rr];
            }
        if (tr_writer<64, NE * G>(lane) && t < t_hi && e0 + r < E) {
            if constexpr (FMT == MOE_FMT_INT8_ROW) l = l * ss;
            if (bias) l = l + bb;
            logits[(size_t)t * E + e0 + r] = l;
        }
    }
}

// the selection kernels for T <= kRouteGemvMaxTokens; NORM: with the fused norm (one more
// row for the gate logit when there is a gate)
template <int FMT, int NV, bool NORM>
hipError_t launch_gemv_topk(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                            float* weights, float* logits, unsigned* counter,
                            const RouteNorm& nm, hipStream_t s) {
    const int E = r.n_experts, d = r.d_model;
    const int npl = (E + 63) / 64;
    const int rows = E + ((NORM && nm.gw) ? 1 : 0);
    const dim3 grid((rows + 3) / 4), block(256);
#define MOE_GT(N)                                                                          \
    router_gemv_topk_kernel<FMT, NV, N, NORM><<<grid, block, 0, s>>>(                      \
        r.w, r.scale, r.bias, x, T, E, d, k, logits, ids, weights, counter, nm)
    if (npl <= 1) MOE_GT(1);
    else if (npl <= 2) MOE_GT(2);
    else if (npl <= 4) MOE_GT(4);
    else if (npl <= 8) MOE_GT(8);
    else MOE_GT(16);
#undef MOE_GT
    return hipGetLastError();
}

template <int FMT, int NV>
hipError_t launch_nv(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                     float* weights, float* logits, unsigned* counter, hipStream_t s) {
    const int E = r.n_experts, d = r.d_model;
    const int npl = (E + 63) / 64;
    if (T <= kRouteOneLaunchMaxTokens)   // one wave per expert row, the last block selects
        return launch_gemv_topk<FMT, NV, false>(r, x, T, k, ids, weights, logits, counter,
                                                RouteNorm{}, s);
    if (T <= kRouteSplitMaxTokens) {   // one wave per expert row, then the selection kernel
        constexpr int NE = SplitShape<FMT, NV>::NE;
        constexpr int PV = SplitShape<FMT, NV>::PV;
        const int ty = (T + kRouteTokensPerWave - 1) / kRouteTokensPerWave;
        bool block_form = false;
        if constexpr (NV * 64 * PV <= 2048) {
            if (T >= kRouteSplitBlockMinTokens) {
                constexpr int RB = NE * kRouteSplitWaves;   // rows per block
                router_gemv_split_kernel<FMT, NV, kRouteSplitWaves>
                    <<<dim3((E + RB - 1) / RB, ty), dim3(64 * kRouteSplitWaves), 0, s>>>(
                        r.w, r.scale, r.bias, x, T, E, d, logits);
                block_form = true;
            }
        }
        if (!block_form)
            router_gemv_split_kernel<FMT, NV, 1>
                <<<dim3((E + NE - 1) / NE, ty), dim3(64), 0, s>>>(r.w, r.scale, r.bias, x, T,
                                                                   E, d, logits);
    } else {
        using R = RgShape<FMT>;
        constexpr int kLds = 2 * R::STAGE;
        constexpr int kMaxDev = 64;
        static bool attr_set[kMaxDev] = {};
        int dev = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err != hipSuccess) return err;
        if (dev >= kMaxDev || !attr_set[dev]) {   // more than 64 KiB of LDS: opt in once
            err = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_gemm_kernel<FMT, NV>),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
            if (err != hipSuccess) return err;
            if (dev < kMaxDev) attr_set[dev] = true;
        }
        router_gemm_kernel<FMT, NV>
            <<<dim3((T + R::BT - 1) / R::BT, (E + R::BE - 1) / R::BE), dim3(512), kLds, s>>>(
                r.w, r.scale, r.bias, x, T, E, d, logits);
    }
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
    // at most 64 chain elements per lane (the few-token kernel holds them in registers)
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        if constexpr (N * PV <= 64)                                                       \
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

template <int FMT, bool NORM>
hipError_t launch_logits_fmt(const moe_router& r, const uint16_t* x, int T, float* logits,
                             const RouteNorm& nm, hipStream_t s) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int nv = r.d_model / (64 * PV);
    const dim3 grid(r.n_experts + ((NORM && nm.gw) ? 1 : 0)), block(64);
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        router_gemv_kernel<FMT, N, NORM><<<grid, block, 0, s>>>(                          \
            r.w, r.scale, r.bias, x, T, r.n_experts, r.d_model, logits, nm);              \
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

template <int FMT, int NV>
hipError_t launch_bounded_nv(const moe_router& r, const uint16_t* x, int T, int k,
                             const float* nw, const float* lf, int32_t* ids, float* weights,
                             hipStream_t s) {
    const int E = r.n_experts, npl = (E + 63) / 64;
    const dim3 grid((T + 3) / 4), block(256);
#define MOE_BS(N)                                                                          \
    route_bounded_select_kernel<FMT, NV, N><<<grid, block, 0, s>>>(                        \
        r.w, r.scale, r.bias, x, nw, lf, T, E, r.d_model, k, ids, weights)
    if (npl <= 1) MOE_BS(1);
    else if (npl <= 2) MOE_BS(2);
    else if (npl <= 4) MOE_BS(4);
    else if (npl <= 8) MOE_BS(8);
    else MOE_BS(16);
#undef MOE_BS
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_bounded_fmt(const moe_router& r, const uint16_t* x, int T, int k,
                              const float* nw, const float* lf, int32_t* ids, float* weights,
                              hipStream_t s) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int nv = r.d_model / (64 * PV);
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        if constexpr (N * PV <= 64)                                                       \
            return launch_bounded_nv<FMT, N>(r, x, T, k, nw, lf, ids, weights, s);        \
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

hipError_t launch_route_bounded_select(const moe_router& r, const uint16_t* x, int T, int k,
                                       const float* nw, const float* lf, int32_t* ids,
                                       float* weights, hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_bounded_fmt<MOE_FMT_INT8_ROW>(r, x, T, k, nw, lf, ids, weights, s);
    return launch_bounded_fmt<MOE_FMT_FP32>(r, x, T, k, nw, lf, ids, weights, s);
}

hipError_t launch_route_logits(const moe_router& r, const uint16_t* x, int T, float* logits,
                               hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_logits_fmt<MOE_FMT_INT8_ROW, false>(r, x, T, logits, RouteNorm{}, s);
    return launch_logits_fmt<MOE_FMT_FP32, false>(r, x, T, logits, RouteNorm{}, s);
}

namespace {
template <int FMT>
hipError_t launch_topk_norm_fmt(const moe_router& r, const uint16_t* x, int T, int k,
                                int32_t* ids, float* weights, float* logits, unsigned* counter,
                                const RouteNorm& nm, hipStream_t s) {
    constexpr int PV = (FMT == MOE_FMT_INT8_ROW) ? 16 : 4;
    const int nv = r.d_model / (64 * PV);
#define MOE_NV(N)                                                                         \
    if (nv == N) {                                                                        \
        if constexpr (N * PV <= 64)                                                       \
            return launch_gemv_topk<FMT, N, true>(r, x, T, k, ids, weights, logits,       \
                                                  counter, nm, s);                        \
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

hipError_t launch_route_norm(const moe_router& r, const uint16_t* x, int T, int k,
                             const float* gamma, float eps, const float* gw, float gb,
                             uint16_t* xn, float* z, int32_t* ids, float* weights,
                             float* logits, unsigned* counter, hipStream_t s) {
    const RouteNorm nm{gamma, eps, gw, gb, xn, z};
    if (T <= kDecodeSelectMaxTokens) {   // logits only: the decode gate/up kernel selects
        if (r.fmt == MOE_FMT_INT8_ROW)
            return launch_logits_fmt<MOE_FMT_INT8_ROW, true>(r, x, T, logits, nm, s);
        return launch_logits_fmt<MOE_FMT_FP32, true>(r, x, T, logits, nm, s);
    }
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_topk_norm_fmt<MOE_FMT_INT8_ROW>(r, x, T, k, ids, weights, logits, counter,
                                                      nm, s);
    return launch_topk_norm_fmt<MOE_FMT_FP32>(r, x, T, k, ids, weights, logits, counter, nm, s);
}

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, unsigned* counter, hipStream_t s) {
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_fmt<MOE_FMT_INT8_ROW>(r, x, T, k, ids, weights, logits, counter, s);
    return launch_fmt<MOE_FMT_FP32>(r, x, T, k, ids, weights, logits, counter, s);
}

}  // namespace moe
