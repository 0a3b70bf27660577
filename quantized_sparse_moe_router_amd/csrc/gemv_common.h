// gemv_common.h -- building blocks of the weight-streaming GEMV for few tokens: group
// dot products on packed int4 / int6 codes, slot resolution, and one projection over a
// block of rows.  Shared by the per-call GEMV kernels and the decode layer kernels, so
// both compute every output with exactly the same operations in the same order.
//
// A row of K packed codes is read by LPR = min(64, K/32) lanes, one 32-code group (16
// bytes int4, 24 bytes int6) per lane per step, so a wave covers 64/LPR rows per load
// instruction with fully used 16-byte loads.  Codes become bf16 pairs (128 + u) with a
// shift and one and-or (int4: the two nibbles 16 bits apart in a word of codes, i.e.
// elements p and p + 4 of its 8, so the activations are paired the same way, see
// nibble_pairs), are multiplied against bf16 activation pairs by v_dot2_f32_bf16, and the
// offset (128 + zero point) times the group's activation sum is removed afterwards; the
// fp16 group scale is applied once per group.
//
// Every fused multiply-add is written out and contraction is off, so a token's arithmetic
// is the same whatever the number of tokens that share a pass (batch invariance).
#pragma once
#include "moe_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Activation pairs in the order group_dot_int4 takes them: within each block of 8
// elements, (x_p, x_{p+4}) for p = 0..3.  a0..a3: the block's pairs in natural order,
// (x0, x1) .. (x6, x7).  v_perm_b32 bytes 0-3 come from its second operand, 4-7 from its
// first.
__device__ __forceinline__ uint4 nibble_pairs(uint32_t a0, uint32_t a1, uint32_t a2,
                                              uint32_t a3) {
    return make_uint4(__builtin_amdgcn_perm(a2, a0, 0x05040100u),
                      __builtin_amdgcn_perm(a2, a0, 0x07060302u),
                      __builtin_amdgcn_perm(a3, a1, 0x05040100u),
                      __builtin_amdgcn_perm(a3, a1, 0x07060302u));
}
__device__ __forceinline__ void nibble_pairs16(uint32_t* xp) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 v = nibble_pairs(xp[4 * q], xp[4 * q + 1], xp[4 * q + 2], xp[4 * q + 3]);
        xp[4 * q] = v.x; xp[4 * q + 1] = v.y; xp[4 * q + 2] = v.z; xp[4 * q + 3] = v.w;
    }
}

// 16 bytes of int4 codes (32 elements, element i in bits 4i..4i+3 of the group) against 32
// bf16 activations in nibble_pairs order.  Returns sum_i (128 + u_i) * x_i, accumulated
// pair by pair: (0, 4), (1, 5), (2, 6), (3, 7), (8, 12), ...
__device__ __forceinline__ float group_dot_int4(const uint4 w, const uint32_t* xp) {
    // the two constants live in registers so that each pair is one v_and_or_b32 (after a
    // shift): a VOP3 instruction cannot take literal operands on gfx9
    uint32_t mask, bias;
    asm("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t pair = ((wd[q] >> (4 * p)) & mask) | bias;
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

enum { kModeGateUp = 0, kModeDown = 1 };

template <int FMT>
struct GroupBits {
    uint4 a;
    uint2 b;   // int6: bytes 16..23 of the group
};

template <int FMT>
__device__ __forceinline__ void load_bits(const uint8_t* p, GroupBits<FMT>& g) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        g.a = *reinterpret_cast<const uint4*>(p);
    } else {
        const uint2* q = reinterpret_cast<const uint2*>(p);
        const uint2 x0 = q[0], x1 = q[1], x2 = q[2];
        g.a = make_uint4(x0.x, x0.y, x1.x, x1.y);
        g.b = x2;
    }
}

template <int FMT>
__device__ __forceinline__ float dot_bits(const GroupBits<FMT>& g, const uint32_t* xp) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        return group_dot_int4(g.a, xp);
    } else {
        const uint32_t w6[6] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y};
        return group_dot_int6(w6, xp);
    }
}

struct Slot {
    int e;              // expert (grouped) or 0 (dense)
    uint64_t members;   // grouped: pairs routed to e, bit q = pair q
    int seg0;           // grouped: sorted position of e's first pair
    int first;          // grouped: rank (among e's pairs) of this chunk's first pair
    int dense0, dense_n;
};

// Resolve slot s; returns false if this block has nothing to do.
template <int MT>
__device__ __forceinline__ bool resolve_slot(int s, int T, int k, const int32_t* ids, int E,
                                             Slot& sl) {
    const int lane = threadIdx.x & 63;
    if (ids) {
        const int P = T * k;
        const int my = (lane < P) ? ids[lane] : -1;
        const int e = __builtin_amdgcn_readlane(my, s);
        if (e < 0 || e >= E) return false;
        const bool valid = lane < P && my >= 0 && my < E;
        sl.members = __ballot(valid && my == e);
        // rank of pair s among e's pairs; the pairs of rank 0, MT, 2MT, ... each lead a
        // chunk of MT pairs, the others return
        const int rank = __popcll(sl.members & ((1ull << s) - 1ull));
        if (rank % MT != 0) return false;
        sl.first = rank;
        sl.seg0 = __popcll(__ballot(valid && my < e));
        sl.e = e;
        sl.dense0 = sl.dense_n = 0;
    } else {
        sl.e = 0;
        sl.members = 0;
        sl.seg0 = 0;
        sl.first = 0;
        sl.dense0 = s * MT;
        if (sl.dense0 >= T) return false;
        sl.dense_n = min(MT, T - sl.dense0);
    }
    return true;
}

// One projection over a block of rows.  K = input length; rows = output rows.
//   GateUp: rows = d_ff, inputs = x rows of the tokens, output h (bf16) per pair row.
//   Down  : rows = d_model, inputs = h rows of the pairs, output y (bf16) per pair row.
// MT = tokens per pass over the weights (a slot's pairs are taken MT at a time).
// NW = waves per block; wave w owns ITERS consecutive groups of 64 / LPR rows.
// PAIRED: int4 activations are already in nibble_pairs order (else they are put in it
// after loading).
template <int FMT, int MODE, int LPR, int GPL, int ITERS, int MT, int NW = 4,
          bool PAIRED = false>
__device__ __forceinline__ void gemv_rows(const uint8_t* __restrict__ wa,
                                          const uint16_t* __restrict__ sa,
                                          const uint8_t* __restrict__ wb,
                                          const uint16_t* __restrict__ sb,
                                          const uint16_t* act, int k, int rows,
                                          int rb, const Slot& sl, uint16_t* out) {
    constexpr int K = LPR * GPL * 32;
    constexpr int RPW = 64 / LPR;                  // rows per load instruction
    constexpr int ROWS_PER_BLOCK = NW * ITERS * RPW;
    constexpr int GB = Fmt<FMT>::kGroupBytes;
    constexpr size_t ROW_BYTES = (size_t)K / 32 * GB;
    constexpr int NMAT = (MODE == kModeGateUp) ? 2 : 1;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gp = lane % LPR;                      // group slot in the row
    const int rsub = lane / LPR;                    // row inside a load instruction
    const bool grouped = sl.members != 0;

    // ---- activation rows of this block's chunk (at most MT pairs / tokens); requested
    // before the weights so both are in flight together
    int arow[MT], orow[MT];
    int mcount = 0;
    uint32_t xv[MT][GPL][16];
    if (grouped) {
        uint64_t rest = sl.members;
        for (int skip = 0; skip < sl.first; ++skip) rest &= rest - 1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            arow[m] = 0;
            orow[m] = 0;
            if (rest) {
                const int q = (int)__builtin_ctzll(rest);
                rest &= rest - 1;
                const int srow = sl.seg0 + sl.first + m;        // expert-sorted position
                arow[m] = (MODE == kModeGateUp) ? q / k : srow;
                orow[m] = srow;
                ++mcount;
            }
        }
    } else {
        mcount = sl.dense_n;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            arow[m] = sl.dense0 + min(m, mcount - 1);
            orow[m] = arow[m];
        }
    }
    auto load_act = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (m < mcount) {
                const uint16_t* ap = act + (size_t)arow[m] * K;
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const uint16_t* src = ap + 32 * (gp + LPR * i);
                    const uint4* s4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint4 q = s4[v];
                        xv[m][i][4 * v + 0] = q.x;
                        xv[m][i][4 * v + 1] = q.y;
                        xv[m][i][4 * v + 2] = q.z;
                        xv[m][i][4 * v + 3] = q.w;
                    }
                    if constexpr (FMT == MOE_FMT_INT4_G32 && !PAIRED) nibble_pairs16(xv[m][i]);
                }
            }
        }
    };
    load_act();

    // ---- every weight load of this wave
    const int row_base = rb * ROWS_PER_BLOCK + wave * ITERS * RPW + rsub;
    const size_t mat_row0 = (size_t)sl.e * rows;
    GroupBits<FMT> wbits[ITERS][NMAT][GPL];
    uint16_t sbits[ITERS][NMAT][GPL];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int row = row_base + it * RPW;
        const size_t mrow = mat_row0 + (row < rows ? row : 0);
#pragma unroll
        for (int mt = 0; mt < NMAT; ++mt) {
            const uint8_t* wbase = (mt == 0 ? wa : wb) + mrow * ROW_BYTES;
            const uint16_t* sbase = (mt == 0 ? sa : sb) + mrow * (K / 32);
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = gp + LPR * i;
                load_bits<FMT>(wbase + (size_t)g * GB, wbits[it][mt][i]);
                sbits[it][mt][i] = sbase[g];
            }
        }
    }
    // every load above is issued before any arithmetic: left to itself the scheduler
    // interleaves the dot products with the loads to save registers, which turns one
    // memory round trip into several
    __builtin_amdgcn_sched_barrier(0);

    // ---- compute
    {
        float sx[MT][GPL];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < mcount)
#pragma unroll
                for (int i = 0; i < GPL; ++i) sx[m][i] = group_sum_x(xv[m][i]);

#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int row = row_base + it * RPW;
            float acc[NMAT][MT];
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int m = 0; m < MT; ++m) acc[mt][m] = 0.0f;
#pragma unroll
            for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const float s = f16_to_f32(sbits[it][mt][i]);
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        if (m < mcount) {
                            const float raw = dot_bits<FMT>(wbits[it][mt][i], xv[m][i]);
                            const float part = __builtin_fmaf(-Fmt<FMT>::kBias, sx[m][i], raw);
                            acc[mt][m] = __builtin_fmaf(s, part, acc[mt][m]);
                        }
                }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < mcount) {
                    const float v0 = group_sum<LPR>(acc[0][m]);
                    float res;
                    if constexpr (MODE == kModeGateUp) {
                        const float u = group_sum<LPR>(acc[NMAT - 1][m]);
                        res = v0 / (1.0f + expf(-v0)) * u;
                    } else {
                        res = v0;
                    }
                    if (row < rows && gp == 0) {
                        out[(size_t)orow[m] * rows + row] = (uint16_t)f32_to_bf16(res);
                    }
                }
            }
        }
    }
}

template <int K>
struct Shape {
    static constexpr int LPR = K >= 2048 ? 64 : K / 32;
    static constexpr int GPL = K >= 2048 ? K / 2048 : 1;
    static constexpr int ITERS = K >= 4096 ? 2 : 1;
    static constexpr int RPB = 4 * ITERS * (64 / LPR);
};

}  // namespace
}  // namespace moe
