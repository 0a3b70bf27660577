// ffn_gemv.hip -- expert FFN for few tokens (decode): stream the selected experts'
// packed weights once, dequantise in registers, reduce across the wavefront.
//
// Decode reads every active weight once per step and is bound by memory bandwidth
// [Halogen Flash Server配置與實測 (lcz.me), replies comparing decode with bandwidth];
// only the selected experts are touched, which is what sparse routing saves
// [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].
//
// Layout of the work: a row of K packed codes is read by LPR = min(64, K/32) lanes, one
// 32-code group (16 bytes int4, 24 bytes int6) per lane per step, so a wave covers
// 64/LPR rows per load instruction with fully used 16-byte loads.  Codes become bf16
// pairs (128 + u) with a byte permute, are multiplied against bf16 activation pairs by
// v_dot2_f32_bf16, and the offset (128 + zero point) times the group's activation sum is
// removed afterwards; the fp16 group scale is applied once per group.
//
// Grouped mode: block x = a position in the expert-sorted pair list; only the first
// position of each expert's segment does work (the others return at once), looping over
// the segment's pairs MT at a time so each weight row is read once per MT tokens.
// Dense mode (shared expert): block x = a chunk of MT tokens.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int kMT = 4;   // tokens per pass over the weights

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 16 bytes of int4 codes (32 elements) against 32 bf16 activations (16 pairs).
// Returns sum_i (128 + u_i) * x_i.
__device__ __forceinline__ float group_dot_int4(const uint4 w, const uint32_t* xp) {
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t lo = wd[q] & 0x0f0f0f0fu;
        const uint32_t hi = (wd[q] >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t sel = 0x0c000c00u | (uint32_t)p | ((uint32_t)(4 + p) << 16);
            const uint32_t pair = __builtin_amdgcn_perm(hi, lo, sel) | 0x43004300u;
            acc = dot2(pair, xp[4 * q + p], acc);
        }
    }
    return acc;
}

// 24 bytes of int6 codes (32 elements, little-endian bit string) against 32 bf16.
__device__ __forceinline__ float group_dot_int6(const uint32_t* w6, const uint32_t* xp) {
    float acc = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint64_t lo64 = (uint64_t)w6[3 * half] | ((uint64_t)w6[3 * half + 1] << 32);
        const uint64_t hi32 = w6[3 * half + 2];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            uint32_t u[2];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int bit = 6 * (2 * p + s);          // bit inside these 96 bits
                uint32_t v;
                if (bit + 6 <= 64)
                    v = (uint32_t)(lo64 >> bit);
                else if (bit >= 64)
                    v = (uint32_t)(hi32 >> (bit - 64));
                else
                    v = (uint32_t)(lo64 >> bit) | (uint32_t)(hi32 << (64 - bit));
                u[s] = v & 63u;
            }
            const uint32_t pair = (u[0] | (u[1] << 16)) | 0x43004300u;
            acc = dot2(pair, xp[8 * half + p], acc);
        }
    }
    return acc;
}

__device__ __forceinline__ float group_sum_x(const uint32_t* xp) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += bf16lo(xp[i]) + bf16hi(xp[i]);
    return s;
}

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOE_FMT_INT4_G32> {
    static constexpr int kGroupBytes = 16;
    static constexpr float kBias = 136.0f;    // 128 (bf16 magic) + 8 (zero point)
};
template <>
struct Fmt<MOE_FMT_INT6_G32> {
    static constexpr int kGroupBytes = 24;
    static constexpr float kBias = 160.0f;    // 128 + 32
};

template <int FMT>
__device__ __forceinline__ float group_dot(const uint8_t* gptr, const uint32_t* xp) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        return group_dot_int4(*reinterpret_cast<const uint4*>(gptr), xp);
    } else {
        const uint2* p = reinterpret_cast<const uint2*>(gptr);
        const uint2 a = p[0], b = p[1], c = p[2];
        const uint32_t w6[6] = {a.x, a.y, b.x, b.y, c.x, c.y};
        return group_dot_int6(w6, xp);
    }
}

enum { kModeGateUp = 0, kModeDown = 1 };

// One projection pass.  K = input length; rows = output rows of the projection.
//   GateUp: rows = d_ff, inputs = x rows of the tokens, output h (bf16) per pair row.
//   Down  : rows = d_model, inputs = h rows of the pairs, output y (bf16) per pair row.
template <int FMT, int MODE, int LPR, int GPL, int ITERS>
__global__ void __launch_bounds__(256) ffn_gemv_kernel(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const uint16_t* __restrict__ act, int T, int k, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs, int E,
    int rows, uint16_t* __restrict__ out) {
    constexpr int K = LPR * GPL * 32;
    constexpr int RPW = 64 / LPR;                  // rows per load instruction
    constexpr int ROWS_PER_BLOCK = 4 * ITERS * RPW;
    constexpr int GB = Fmt<FMT>::kGroupBytes;
    constexpr size_t ROW_BYTES = (size_t)K / 32 * GB;
    constexpr int NMAT = (MODE == kModeGateUp) ? 2 : 1;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gp = lane % LPR;                      // group slot in the row
    const int rsub = lane / LPR;                    // row inside a load instruction

    // ---- which expert and which activation rows
    int e, seg_begin, seg_end;
    const bool grouped = offsets != nullptr;
    if (grouped) {
        const int pos = blockIdx.x;
        const int nvalid = offsets[E];
        if (pos >= nvalid) return;
        e = ids[sorted_pairs[pos]];
        seg_begin = offsets[e];
        if (pos != seg_begin) return;
        seg_end = offsets[e + 1];
    } else {
        e = 0;
        seg_begin = blockIdx.x * kMT;
        if (seg_begin >= T) return;
        seg_end = min(T, seg_begin + kMT);
    }

    const int row_base = blockIdx.y * ROWS_PER_BLOCK + wave * ITERS * RPW + rsub;
    const size_t mat_row0 = (size_t)e * rows;

    for (int c0 = seg_begin; c0 < seg_end; c0 += kMT) {
        const int mcount = min(kMT, seg_end - c0);
        // activations: for each token slot and group, 16 packed bf16 pairs
        uint32_t xv[kMT][GPL][16];
        float sx[kMT][GPL];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
            if (m < mcount) {
                const int r = c0 + m;
                size_t arow;
                if (MODE == kModeGateUp)
                    arow = grouped ? (size_t)(sorted_pairs[r] / k) : (size_t)r;
                else
                    arow = (size_t)r;
                const uint16_t* ap = act + arow * K;
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const uint4* src = reinterpret_cast<const uint4*>(ap + 32 * (gp + LPR * i));
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint4 q = src[v];
                        xv[m][i][4 * v + 0] = q.x;
                        xv[m][i][4 * v + 1] = q.y;
                        xv[m][i][4 * v + 2] = q.z;
                        xv[m][i][4 * v + 3] = q.w;
                    }
                    sx[m][i] = group_sum_x(xv[m][i]);
                }
            }
        }

#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int row = row_base + it * RPW;
            const bool rv = row < rows;
            const size_t mrow = mat_row0 + (rv ? row : 0);
            float acc[NMAT][kMT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int m = 0; m < kMT; ++m) acc[mt][m] = 0.0f;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt) {
                const uint8_t* wbase = (mt == 0 ? wa : wb) + mrow * ROW_BYTES;
                const uint16_t* sbase = (mt == 0 ? sa : sb) + mrow * (K / 32);
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const int g = gp + LPR * i;
                    const float s = f16_to_f32(sbase[g]);
                    const uint8_t* gptr = wbase + (size_t)g * GB;
#pragma unroll
                    for (int m = 0; m < kMT; ++m) {
                        if (m < mcount) {
                            const float raw = group_dot<FMT>(gptr, xv[m][i]);
                            acc[mt][m] = __builtin_fmaf(
                                s, raw - Fmt<FMT>::kBias * sx[m][i], acc[mt][m]);
                        }
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < kMT; ++m) {
                if (m < mcount) {
                    float v0 = group_sum<LPR>(acc[0][m]);
                    float res;
                    if constexpr (MODE == kModeGateUp) {
                        const float u = group_sum<LPR>(acc[NMAT - 1][m]);
                        res = v0 / (1.0f + expf(-v0)) * u;
                    } else {
                        res = v0;
                    }
                    if (rv && gp == 0)
                        out[(size_t)(c0 + m) * rows + row] = (uint16_t)f32_to_bf16(res);
                }
            }
        }
    }
}

template <int FMT, int MODE>
hipError_t launch_pass(const uint8_t* wa, const uint16_t* sa, const uint8_t* wb,
                       const uint16_t* sb, const uint16_t* act, int K, int T, int k,
                       const int32_t* ids, const int32_t* offsets, const int32_t* sorted_pairs,
                       int E, int rows, uint16_t* out, int nslots, hipStream_t s) {
#define MOE_GEMV_CASE(KV, LPRV, GPLV, ITV)                                                  \
    case KV: {                                                                              \
        constexpr int RPB = 4 * ITV * (64 / LPRV);                                          \
        dim3 grid(nslots, (rows + RPB - 1) / RPB);                                          \
        ffn_gemv_kernel<FMT, MODE, LPRV, GPLV, ITV><<<grid, 256, 0, s>>>(                   \
            wa, sa, wb, sb, act, T, k, ids, offsets, sorted_pairs, E, rows, out);           \
        break;                                                                              \
    }
    switch (K) {
        MOE_GEMV_CASE(128, 4, 1, 1)
        MOE_GEMV_CASE(256, 8, 1, 1)
        MOE_GEMV_CASE(512, 16, 1, 2)
        MOE_GEMV_CASE(1024, 32, 1, 2)
        MOE_GEMV_CASE(2048, 64, 1, 4)
        MOE_GEMV_CASE(4096, 64, 2, 2)
        default:
            return hipErrorInvalidValue;
    }
#undef MOE_GEMV_CASE
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_ffn(const moe_experts& ex, const uint16_t* x, int T, int k,
                      const int32_t* ids, const int32_t* offsets, const int32_t* sorted_pairs,
                      uint16_t* y, uint16_t* h_ws, hipStream_t s) {
    const int d = ex.d_model, F = ex.d_ff, E = ex.n_experts;
    const bool grouped = offsets != nullptr;
    const int nslots = grouped ? T * k : (T + kMT - 1) / kMT;
    hipError_t err = launch_pass<FMT, kModeGateUp>(ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x,
                                                   d, T, k, ids, offsets, sorted_pairs, E, F,
                                                   h_ws, nslots, s);
    if (err != hipSuccess) return err;
    return launch_pass<FMT, kModeDown>(ex.w_down, ex.s_down, nullptr, nullptr, h_ws, F, T, k,
                                       ids, offsets, sorted_pairs, E, d, y, nslots, s);
}

}  // namespace

hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, const int32_t* offsets,
                           const int32_t* sorted_pairs, uint16_t* y, uint16_t* h_ws,
                           hipStream_t s) {
    if (ex.fmt == MOE_FMT_INT4_G32)
        return launch_ffn<MOE_FMT_INT4_G32>(ex, x, T, k, ids, offsets, sorted_pairs, y, h_ws, s);
    return launch_ffn<MOE_FMT_INT6_G32>(ex, x, T, k, ids, offsets, sorted_pairs, y, h_ws, s);
}

}  // namespace moe
