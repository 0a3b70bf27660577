// route_mfma.hip -- candidate router logits for many tokens on gfx950 MFMA.
//
// The selection compares fp32 logits summed in one fixed order (include/moe.h), and
// summing every logit in that order is fp32 VALU work (2·d·E flops per token).  The pages
// send each token to 10 of 512 experts [Strata 与 Qwen3.8-Flash-Next (telli.sh), section
// 稀疏架构创造了机会], so only a handful of a token's logits decide its selection.  Here
// the matrix cores compute every logit to within a stated error bound; the selection
// kernel (route.hip) then recomputes, in the fixed order, only the experts that the bound
// cannot rule out, and selects among exact values.  This file holds the two kernels that
// produce the bounded logits:
//
//   router_planes_kernel  router rows -> bf16 "plane rows" + a norm bound per row.
//       FP32 rows: w = hi + mid + lo exactly, hi = bf16(w), mid = bf16(w - hi) (w - hi is
//       exact in fp32), |lo| <= 2^-17 |w|; plane rows 2e (hi) and 2e+1 (mid), lo dropped.
//       INT8_ROW rows: one plane row e, the codes as bf16 (exact).
//       nw[e] >= Euclidean norm of the row's values (fp32 w, or |s_e| * q).
//   router_mfma_kernel    lf[t][e] = sum over k of x[t][k] * plane rows, fp32 accumulate
//       (v_mfma_f32_32x32x16_bf16; bf16 x bf16 products are exact in fp32), then the
//       planes of e added, then + b_e (FP32) or fl(fl(acc * s_e) + b_e) (INT8_ROW).
//
// Bound (used by the selection): |lf - logit| <= 2^-11 (|x_t|·nw[e] + |b_e|).  Its terms:
// the dropped lo part (2^-17 |x||w|), MFMA accumulation in fp32 over d/16 steps of 16
// exact products (below 2^-14 |x||w| even if every step truncated instead of rounding),
// the fixed order's own rounding (d/64 + 6 roundings, below 2^-16 |x||w|), and the final
// scale / bias roundings; 2^-11 leaves a factor of 8 over their sum.  Cauchy-Schwarz gives
// sum |x_k w_k| <= |x|·|w|.
#include "mfma_common.h"

#include <type_traits>

#pragma clang fp contract(off)

namespace moe {
namespace {

// ------------------------------------------------------------------ planes + norms
// One wave per router row.
template <int FMT>
__global__ void __launch_bounds__(256) router_planes_kernel(const void* __restrict__ W,
                                                            const uint16_t* __restrict__ scale,
                                                            int E, int d,
                                                            uint16_t* __restrict__ planes,
                                                            float* __restrict__ nw) {
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= E) return;
    float ss = 0.0f;
    if constexpr (FMT == MOE_FMT_FP32) {
        const float4* row = reinterpret_cast<const float4*>(static_cast<const float*>(W) +
                                                            (size_t)e * d);
        uint16_t* hi_row = planes + (size_t)(2 * e) * d;
        uint16_t* mid_row = hi_row + d;
        for (int c = lane; c < d / 4; c += 64) {
            const float4 v = row[c];
            const float w[4] = {v.x, v.y, v.z, v.w};
            uint32_t hb[2], mb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t h2 = pack_bf16(w[2 * i], w[2 * i + 1]);
                const float r0 = w[2 * i] - __uint_as_float(h2 << 16);
                const float r1 = w[2 * i + 1] - __uint_as_float(h2 & 0xffff0000u);
                hb[i] = h2;
                mb[i] = pack_bf16(r0, r1);
                ss = __builtin_fmaf(w[2 * i], w[2 * i], ss);
                ss = __builtin_fmaf(w[2 * i + 1], w[2 * i + 1], ss);
            }
            *reinterpret_cast<u32x2_t*>(hi_row + 4 * c) = u32x2_t{hb[0], hb[1]};
            *reinterpret_cast<u32x2_t*>(mid_row + 4 * c) = u32x2_t{mb[0], mb[1]};
        }
    } else {
        const uint4* row = reinterpret_cast<const uint4*>(static_cast<const int8_t*>(W) +
                                                          (size_t)e * d);
        uint16_t* prow = planes + (size_t)e * d;
        for (int c = lane; c < d / 16; c += 64) {
            const uint4 v = row[c];
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q0 = (float)(int8_t)((wd[i >> 1] >> (16 * (i & 1))) & 0xffu);
                const float q1 = (float)(int8_t)((wd[i >> 1] >> (16 * (i & 1) + 8)) & 0xffu);
                o[i] = pack_bf16(q0, q1);
                ss = __builtin_fmaf(q0, q0, ss);
                ss = __builtin_fmaf(q1, q1, ss);
            }
            *reinterpret_cast<u32x4_t*>(prow + 16 * c) = u32x4_t{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<u32x4_t*>(prow + 16 * c + 8) = u32x4_t{o[4], o[5], o[6], o[7]};
        }
    }
    ss = group_sum<64>(ss);
    // sqrt and the sums above are each within a few ulps; the factor covers them
    float n = sqrtf(ss) * (1.0f + 0x1p-10f);
    if constexpr (FMT == MOE_FMT_INT8_ROW) n = n * fabsf(f16_to_f32(scale[e]));
    if (lane == 0) nw[e] = n;
}

// ------------------------------------------------------------------ candidate GEMM
// Tile = 128 tokens x 256 plane rows, 4 waves: wave w covers tokens 64 (w & 1) .. + 63 and
// plane rows 128 (w >> 1) .. + 127, i.e. 2 x 4 MFMA blocks of 32 x 32 (128 fp32
// accumulators).  Per k-step of 64, x rows and plane rows are copied global -> LDS
// directly, 128 bytes per row with the 16-byte chunks XOR-swizzled by (row / 2) % 8 so
// that operand reads are free of bank conflicts; three stages, the loads of step ks + 2
// issued during step ks.  Inside a step, lane half h of every operand covers
// k = 32 h + 8 ss .. + 7 in sub-step ss (the same permutation on both sides).
constexpr int RBM = 128;              // tokens per tile
constexpr int RBN = 256;              // plane rows per tile
constexpr int RBK = 64;               // reduction step
constexpr int RSTAGES = 3;
constexpr int RA = RBM * RBK * 2;     // LDS bytes of x per stage
constexpr int RB = RBN * RBK * 2;     // LDS bytes of plane rows per stage
constexpr int RSTAGE = RA + RB;
constexpr int kRouterMfmaLds = RSTAGES * RSTAGE;
constexpr int RNG = RBM / 32 + RBN / 32;   // global -> LDS loads per wave per k-step (12)
constexpr int kXcd = 8;
static_assert(kRouterMfmaLds <= 160 * 1024, "LDS");

template <int FMT>
__global__ void __launch_bounds__(256, 1) router_mfma_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ planes,
    const float* __restrict__ bias, const uint16_t* __restrict__ scale, int T, int E, int d,
    int n_tt, int n_pt, float* __restrict__ lf) {
    constexpr int PL = (FMT == MOE_FMT_FP32) ? 2 : 1;   // plane rows per expert
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // XCD-aware order (workgroups go round-robin to the 8 XCDs): when n_pt divides 8, each
    // XCD keeps one plane tile, so its L2 holds that tile's rows only
    int tt, pt;
    if (kXcd % n_pt == 0) {
        const int xcd = blockIdx.x % kXcd, q = blockIdx.x / kXcd, g = kXcd / n_pt;
        pt = xcd % n_pt;
        tt = q * g + xcd / n_pt;
    } else {
        pt = blockIdx.x % n_pt;
        tt = blockIdx.x / n_pt;
    }
    if (tt >= n_tt) return;
    const int NP = E * PL, nk = d / RBK;
    const int t0 = tt * RBM, p0 = pt * RBN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1, h = lane >> 5;
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // load q of a step: q < 4 -> x rows 32 q + 8 wave + lane / 8, else plane rows
    // 32 (q - 4) + 8 wave + lane / 8; rows past the end repeat the last one
    const uint16_t* src[RNG];
#pragma unroll
    for (int q = 0; q < RNG; ++q) {
        const int qq = q < 4 ? q : q - 4;
        const int r = 32 * qq + 8 * wave + (lane >> 3);
        const int chunk = (lane & 7) ^ ((r >> 1) & 7);
        if (q < 4)
            src[q] = x + (size_t)min(t0 + r, T - 1) * d + 8 * chunk;
        else
            src[q] = planes + (size_t)min(p0 + r, NP - 1) * d + 8 * chunk;
    }
    auto issue = [&](int q, int step, int st) __attribute__((always_inline)) {
        const uint32_t base = lds0 + st * RSTAGE;
        const int qq = q < 4 ? q : q - 4;
        dma16(src[q] + step * RBK, base + (q < 4 ? 0 : RA) + (32 * qq + 8 * wave) * 128);
    };
    // operand of 32-row block rb (of the x or plane region), sub-step ss
    const uint32_t rd = (uint32_t)(lane & 31) * 128;
    auto frag = [&](int st, int region, int rb, int ss) __attribute__((always_inline)) {
        const uint32_t chunk = (uint32_t)((4 * h + ss) ^ ((lane >> 1) & 7));
        return *reinterpret_cast<const bf16x8_t*>(smem + st * RSTAGE + region + rb * 4096 +
                                                  rd + (chunk << 4));
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // operands of the current sub-step (buffer B) and the next (B ^ 1)
    bf16x8_t fa[2][2], fb[2][4];
    auto read_ops = [&](int st, int ss, int B, int t) __attribute__((always_inline)) {
        if (t < 2) fa[B][t] = frag(st, 0, 2 * wm + t, ss);
        else if (t < 6) fb[B][t - 2] = frag(st, RA, 4 * wn + t - 2, ss);
    };
    // plane rows as the first operand: lane l of block (i, j) then holds token 32 i + l % 32
    // and plane rows 32 j + 8 (r / 4) + 4 (l / 32) + r % 4
    auto mfma = [&](int B, int t) __attribute__((always_inline)) {
        const int i = t / 4, j = t % 4;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[B][j], fa[B][i], acc[i][j],
                                                            0, 0, 0);
    };

#pragma unroll
    for (int q = 0; q < RNG; ++q) issue(q, 0, 0);
#pragma unroll
    for (int q = 0; q < RNG; ++q) issue(q, 1, 1);
    MOE_WAIT_VMCNT(RNG);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 6; ++t) read_ops(0, 0, 0, t);

    // One k-step = 4 sub-steps x 8 slots, each slot one MFMA; the next sub-step's operands
    // are read from LDS during the current one, and the 12 loads of step ks + 2 go out one
    // every other slot of sub-steps 0..2 (PF: all but the last two steps, which wait for
    // everything instead).  sched_barrier keeps the compiler from regrouping the slots.
    int st = 0;
    auto kstep = [&](int ks, auto pf) __attribute__((always_inline)) {
        constexpr bool PF = decltype(pf)::value;
        const int st1 = st == RSTAGES - 1 ? 0 : st + 1;
        const int st2 = st1 == RSTAGES - 1 ? 0 : st1 + 1;
#pragma unroll
        for (int u = 0; u < 24; ++u) {            // sub-steps 0..2
            const int ss = u / 8, t = u % 8, B = ss & 1;
            mfma(B, t);
            read_ops(st, ss + 1, B ^ 1, t);
            if (PF && u % 2 == 0) issue(u / 2, ks + 2, st2);
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wave's loads of step ks + 1 have landed and its reads of stage st are done;
        // after the barrier every wave's have
        if constexpr (PF) MOE_WAIT_VMCNT_LDS(RNG);
        else MOE_WAIT_VMCNT_LDS(0);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 8; ++t) {             // sub-step 3, and step ks + 1's operands
            mfma(1, t);
            read_ops(st1, 0, 0, t);
            __builtin_amdgcn_sched_barrier(0);
        }
        st = st1;
    };
    for (int ks = 0; ks + 2 < nk; ++ks) kstep(ks, std::true_type{});
    for (int ks = nk - 2; ks < nk; ++ks) kstep(ks, std::false_type{});

    // ---- epilogue: planes of an expert are adjacent accumulators of one lane
    const bool vec = (E % 4) == 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = t0 + 64 * wm + 32 * i + (lane & 31);
        if (t >= T) continue;
        float* orow = lf + (size_t)t * E;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = p0 + 128 * wn + 32 * j + 8 * q + 4 * h;   // plane row of r = 4q
                float l[4 / PL];
                const int e0 = p / PL;
#pragma unroll
                for (int u = 0; u < 4 / PL; ++u) {
                    const int e = min(e0 + u, E - 1);
                    float a;
                    if constexpr (PL == 2)
                        a = acc[i][j][4 * q + 2 * u] + acc[i][j][4 * q + 2 * u + 1];
                    else
                        a = acc[i][j][4 * q + u];
                    if constexpr (FMT == MOE_FMT_INT8_ROW) a = a * f16_to_f32(scale[e]);
                    if (bias) a = a + bias[e];
                    l[u] = a;
                }
                if constexpr (PL == 2) {
                    if (vec && e0 + 1 < E) {
                        *reinterpret_cast<float2*>(orow + e0) = make_float2(l[0], l[1]);
                    } else {
                        if (e0 < E) orow[e0] = l[0];
                        if (e0 + 1 < E) orow[e0 + 1] = l[1];
                    }
                } else {
                    if (vec && e0 + 3 < E) {
                        *reinterpret_cast<float4*>(orow + e0) =
                            make_float4(l[0], l[1], l[2], l[3]);
                    } else {
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (e0 + u < E) orow[e0 + u] = l[u];
                    }
                }
            }
        }
    }
}

template <int FMT>
hipError_t launch_fmt(const moe_router& r, const uint16_t* x, int T, uint16_t* planes,
                      float* nw, float* lf, hipStream_t s) {
    constexpr int PL = (FMT == MOE_FMT_FP32) ? 2 : 1;
    const int E = r.n_experts, d = r.d_model;
    router_planes_kernel<FMT><<<(E + 3) / 4, 256, 0, s>>>(r.w, r.scale, E, d, planes, nw);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int kMaxDev = 64;
    static bool attr_set[kMaxDev] = {};
    int dev = 0;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev >= kMaxDev || !attr_set[dev]) {   // more than 64 KiB of LDS: opt in once
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(&router_mfma_kernel<FMT>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kRouterMfmaLds);
        if (err != hipSuccess) return err;
        if (dev < kMaxDev) attr_set[dev] = true;
    }
    const int n_tt = (T + RBM - 1) / RBM, n_pt = (E * PL + RBN - 1) / RBN;
    int grid;
    if (kXcd % n_pt == 0) {
        const int g = kXcd / n_pt;
        grid = (n_tt + g - 1) / g * kXcd;
    } else {
        grid = n_tt * n_pt;
    }
    router_mfma_kernel<FMT><<<grid, 256, kRouterMfmaLds, s>>>(x, planes, r.bias, r.scale, T, E,
                                                             d, n_tt, n_pt, lf);
    return hipGetLastError();
}

}  // namespace

size_t route_bounded_planes_bytes(int E, int d) { return (size_t)E * 2 * (size_t)d * 2; }

hipError_t launch_route_bounded_logits(const moe_router& r, const uint16_t* x, int T,
                                       uint16_t* planes, float* nw, float* lf,
                                       hipStream_t s) {
    if (r.d_model % RBK != 0) return hipErrorInvalidValue;
    if (r.fmt == MOE_FMT_INT8_ROW)
        return launch_fmt<MOE_FMT_INT8_ROW>(r, x, T, planes, nw, lf, s);
    return launch_fmt<MOE_FMT_FP32>(r, x, T, planes, nw, lf, s);
}

}  // namespace moe
