// gemv_common.h -- building blocks of the weight-streaming GEMV for few tokens: group
// dot products on packed int4 / int6 / int3 / int2 codes, slot resolution, and one projection over a
// block of rows.  Shared by the per-call GEMV kernels and the decode layer kernels, so
// both compute every output with exactly the same operations in the same order.
//
// A row of K packed codes is read by LPR = min(64, K/32) lanes, one whole 32-code group
// (16 bytes int4, 24 int6, 12 int3, 8 int2) per lane per step, so a wave covers 64/LPR
// rows per load instruction and every byte loaded is used.  Codes become bf16 pairs
// (128 + u) with shifts and and-ors (int4: the two nibbles 16 bits apart in a word of
// codes, i.e. elements p and p + 4 of its 8, so the activations are paired the same way,
// see nibble_pairs; int6, int3, int2: neighbouring codes 2p, 2p + 1), are multiplied against bf16 activation pairs by v_dot2_f32_bf16, and the
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

// A group's 32 codes as 16 bf16 pairs (128 + u_a, 128 + u_b), in the order dot_pairs takes
// them against the activation pairs.  Decoded once per group and reused for every token of a
// pass (the decode is independent of the token).
//
// int4: 16 bytes, element i in bits 4i..4i+3; pair 4q + p = elements (8q + p, 8q + p + 4)
// (the nibbles 16 bits apart in word q), so the activations come in nibble_pairs order.
__device__ __forceinline__ void pairs_int4(const uint4 w, uint32_t* pr) {
    // the two constants live in registers so that each pair is one v_and_or_b32 (after a
    // shift): a VOP3 instruction cannot take literal operands on gfx9
    uint32_t mask, bias;
    asm("s_mov_b32 %0, 0x000f000f" : "=s"(mask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int p = 0; p < 4; ++p) pr[4 * q + p] = ((wd[q] >> (4 * p)) & mask) | bias;
}

// int6: 24 bytes, a little-endian bit string; pair p = codes 2p, 2p + 1.
__device__ __forceinline__ void pairs_int6(const uint32_t* w6, uint32_t* pr) {
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
            pr[8 * half + p] = (u[0] | (u[1] << 16)) | 0x43004300u;
        }
    }
}

// int3: 12 bytes, a little-endian bit string, code i at bits 3i..3i+2; pair i = codes
// (i, i + 16), i = 0..15.  With A = the string and B = the string from bit 48 on, code i is
// bits 3i of A and code i + 16 bits 3i of B: a word holding 16 bits of A in its low half
// and the same 16 bits of B in its high half (one v_perm_b32) gives five pairs, each with
// one shift and one v_and_or_b32.  The activations come in int3_pairs16 order.
__device__ __forceinline__ void pairs_int3(const uint32_t* w3, uint32_t* pr) {
    uint32_t mask, bias;
    asm("s_mov_b32 %0, 0x00070007" : "=s"(mask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
    const uint32_t d0 = w3[0], d1 = w3[1], d2 = w3[2];
    const uint32_t b_lo = __builtin_amdgcn_alignbit(d2, d1, 16);   // string bits 48..79
    const uint32_t b_hi = d2 >> 16;                                 // string bits 80..95
    // window k: bits 15k .. 15k + 15 of A and of B (codes 5k .. 5k + 4 and their partners)
    const uint32_t a_w[4] = {d0, __builtin_amdgcn_alignbit(d1, d0, 15),
                             __builtin_amdgcn_alignbit(d1, d0, 30), d1 >> 13};
    const uint32_t b_w[4] = {b_lo, __builtin_amdgcn_alignbit(b_hi, b_lo, 15),
                             __builtin_amdgcn_alignbit(b_hi, b_lo, 30), b_hi >> 13};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t q = __builtin_amdgcn_perm(b_w[k], a_w[k], 0x05040100u);
#pragma unroll
        for (int p = 0; p < 5 && 5 * k + p < 16; ++p) pr[5 * k + p] = ((q >> (3 * p)) & mask) | bias;
    }
}

// int2: 8 bytes, code i at bits 2i..2i+1 (word i / 16); pair 8w + j = codes (16w + j,
// 16w + j + 8), the 2-bit fields 16 bits apart in word w: one shift and one v_and_or_b32.
// The activations come in int2_pairs16 order.
__device__ __forceinline__ void pairs_int2(const uint32_t* w2, uint32_t* pr) {
    uint32_t mask, bias;
    asm("s_mov_b32 %0, 0x00030003" : "=s"(mask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(bias));
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int j = 0; j < 8; ++j) pr[8 * w + j] = ((w2[w] >> (2 * j)) & mask) | bias;
}

// Activation pairs in the order pairs_int3 takes the codes: pair i = (x_i, x_{i + 16}).
// xp: the group's 16 pairs in natural order, (x0, x1) .. (x30, x31).
__device__ __forceinline__ void int3_pairs16(uint32_t* xp) {
    uint32_t o[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        o[i] = __builtin_amdgcn_perm(xp[8 + i / 2], xp[i / 2], (i & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = o[i];
}

// ... in the order pairs_int2 takes them: pair 8w + j = (x_{16w + j}, x_{16w + j + 8}).
__device__ __forceinline__ void int2_pairs16(uint32_t* xp) {
    uint32_t o[16];
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            o[8 * w + j] = __builtin_amdgcn_perm(xp[8 * w + 4 + j / 2], xp[8 * w + j / 2],
                                                 (j & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
    for (int i = 0; i < 16; ++i) xp[i] = o[i];
}

// int3 and int2 activations are put in pair order in registers, after the group's sum has
// been taken in natural order (int4 ones are stored in pair order where they are staged, and
// summed in that order; int6 pairs are neighbours)
template <int FMT>
constexpr bool kPairInRegisters = FMT == MOE_FMT_INT3_G32 || FMT == MOE_FMT_INT2_G32;
template <int FMT>
__device__ __forceinline__ void pair_in_registers(uint32_t* xp) {
    if constexpr (FMT == MOE_FMT_INT3_G32) int3_pairs16(xp);
    else if constexpr (FMT == MOE_FMT_INT2_G32) int2_pairs16(xp);
}

// sum_i (128 + u_i) * x_i over a group: 16 v_dot2_f32_bf16, pair by pair in ascending order.
__device__ __forceinline__ float dot_pairs(const uint32_t* pr, const uint32_t* xp) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc = dot2(pr[i], xp[i], acc);
    return acc;
}

// sum of a group's 32 activations, pair by pair in ascending order: one v_dot2_f32_bf16
// per pair against (1.0, 1.0) (the products are exact), where unpacking both halves and
// adding them takes four instructions.  The pair (1.0, 1.0) is kept in a register: as an
// inline constant the instruction would read it as one fp32 value.
__device__ __forceinline__ float group_sum_x(const uint32_t* xp) {
    uint32_t ones;
    asm("v_mov_b32 %0, 0x3f803f80" : "=v"(ones));
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s = dot2(xp[i], ones, s);
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
template <>
struct Fmt<MOE_FMT_INT3_G32> {
    static constexpr int kGroupBytes = 12;
    static constexpr float kBias = 132.0f;    // 128 + 4
};
template <>
struct Fmt<MOE_FMT_INT2_G32> {
    static constexpr int kGroupBytes = 8;
    static constexpr float kBias = 130.0f;    // 128 + 2
};

enum { kModeGateUp = 0, kModeDown = 1 };

template <int FMT>
struct GroupBits {
    uint4 a;   // int4: the group; int3: bytes 0..11 in x, y, z; int2: bytes 0..7 in x, y
    uint2 b;   // int6: bytes 16..23 of the group
};

// Expert weights (codes and scales) are loaded non-temporal (the `nt` cache policy): a decode
// step reads each selected expert's rows once, so they should not displace what every step
// reads again (the router rows, activations, h).  Measured on one token through 32 rotated
// layer copies: 17.3 -> 16.1 us per decode step, and the same gain per block of the 48-block
// sweep; no change at 64 tokens.
typedef uint32_t nt_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t nt_u32x2 __attribute__((ext_vector_type(2)));
// 12 bytes at a 4-byte aligned address: one dwordx3 load (three 4-byte loads would be merged
// into one without the cache policy)
typedef uint32_t nt_u32x3 __attribute__((ext_vector_type(3), aligned(4)));

template <int FMT>
__device__ __forceinline__ void load_bits(const uint8_t* p, GroupBits<FMT>& g) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
        g.a = make_uint4(v[0], v[1], v[2], v[3]);
    } else if constexpr (FMT == MOE_FMT_INT6_G32) {
        const nt_u32x2* q = reinterpret_cast<const nt_u32x2*>(p);
        const nt_u32x2 x0 = __builtin_nontemporal_load(q);
        const nt_u32x2 x1 = __builtin_nontemporal_load(q + 1);
        const nt_u32x2 x2 = __builtin_nontemporal_load(q + 2);
        g.a = make_uint4(x0[0], x0[1], x1[0], x1[1]);
        g.b = make_uint2(x2[0], x2[1]);
    } else if constexpr (FMT == MOE_FMT_INT3_G32) {
        const nt_u32x3 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x3*>(p));
        g.a = make_uint4(v[0], v[1], v[2], 0u);
    } else {
        const nt_u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
        g.a = make_uint4(v[0], v[1], 0u, 0u);
    }
}

// one fp16 group scale, non-temporal like the codes
__device__ __forceinline__ uint16_t load_scale(const uint16_t* p) {
    return __builtin_nontemporal_load(p);
}

template <int FMT>
__device__ __forceinline__ void decode_pairs(const GroupBits<FMT>& g, uint32_t* pr) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        pairs_int4(g.a, pr);
    } else if constexpr (FMT == MOE_FMT_INT6_G32) {
        const uint32_t w6[6] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y};
        pairs_int6(w6, pr);
    } else if constexpr (FMT == MOE_FMT_INT3_G32) {
        const uint32_t w3[3] = {g.a.x, g.a.y, g.a.z};
        pairs_int3(w3, pr);
    } else {
        const uint32_t w2[2] = {g.a.x, g.a.y};
        pairs_int2(w2, pr);
    }
}

// one group against one token's activations: sum_i (128 + u_i) * x_i
template <int FMT>
__device__ __forceinline__ float dot_bits(const GroupBits<FMT>& g, const uint32_t* xp) {
    uint32_t pr[16];
    decode_pairs<FMT>(g, pr);
    return dot_pairs(pr, xp);
}

struct Slot {
    int e;              // expert (grouped) or 0 (dense)
    uint64_t members;   // grouped: pairs routed to e, bit q = pair q
    int seg0;           // grouped: sorted position of e's first pair
    int first;          // grouped: rank (among e's pairs) of this chunk's first pair
    int dense0, dense_n;
    // sorted mode (more pairs than a ballot covers): this chunk is the sorted positions
    // q0 .. q0 + sn - 1 of expert e (sn > 0), and tok[m] the token of position q0 + m
    // (for m >= sn, the token of the last position)
    int sn = 0, q0 = 0;
    int tok[4];
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
    if (sl.sn > 0) {
        static_assert(MT <= 4, "a sorted-mode chunk holds at most 4 pairs");
        mcount = sl.sn;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int mm = min(m, mcount - 1);
            arow[m] = (MODE == kModeGateUp) ? sl.tok[m] : sl.q0 + mm;   // tok repeats its last
            orow[m] = sl.q0 + mm;
        }
    } else if (grouped) {
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
                sbits[it][mt][i] = load_scale(sbase + g);
            }
        }
    }
    // every load above is issued before any arithmetic: left to itself the scheduler
    // interleaves the dot products with the loads to save registers, which turns one
    // memory round trip into several
    __builtin_amdgcn_sched_barrier(0);

    // ---- compute
    {
        // int4: the activations into nibble_pairs order, only now: done where they are
        // loaded, it makes the wave wait for them before it requests the weights
        if constexpr (FMT == MOE_FMT_INT4_G32 && !PAIRED) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < mcount)
#pragma unroll
                    for (int i = 0; i < GPL; ++i) nibble_pairs16(xv[m][i]);
        }
        float sx[MT][GPL];
#pragma unroll
        for (int m = 0; m < MT; ++m)
            if (m < mcount)
#pragma unroll
                for (int i = 0; i < GPL; ++i) sx[m][i] = group_sum_x(xv[m][i]);
        if constexpr (kPairInRegisters<FMT>) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (m < mcount)
#pragma unroll
                    for (int i = 0; i < GPL; ++i) pair_in_registers<FMT>(xv[m][i]);
        }

        // rows are taken RB at a time: acc[b * MTP + m][mt] is this lane's part of row
        // it0 + b's sum for token m, matrix mt (MTP: MT rounded up to a power of two for the
        // reduction; the padding sums stay 0 and are not stored); at most 16 sums are live
        constexpr int MTP = MT <= 1 ? 1 : MT <= 2 ? 2 : MT <= 4 ? 4 : 8;
        constexpr int RB = (MTP * NMAT * ITERS <= 16) ? ITERS
                         : (16 / (MTP * NMAT) >= 1 ? 16 / (MTP * NMAT) : 1);
        static_assert(ITERS % RB == 0, "row batches divide the rows");
        constexpr int NR = RB * MTP;
#pragma unroll
        for (int it0 = 0; it0 < ITERS; it0 += RB) {
            float acc[NR][NMAT];
#pragma unroll
            for (int r = 0; r < NR; ++r)
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt) acc[r][mt] = 0.0f;
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int mt = 0; mt < NMAT; ++mt)
#pragma unroll
                    for (int i = 0; i < GPL; ++i) {
                        const int it = it0 + b;
                        const float s = f16_to_f32(sbits[it][mt][i]);
                        // the group's pairs once for every token of the chunk (held in
                        // registers: left to itself the compiler rebuilds them per token)
                        uint32_t pr[16];
                        decode_pairs<FMT>(wbits[it][mt][i], pr);
                        if constexpr (MT > 1) {
#pragma unroll
                            for (int j = 0; j < 16; ++j) asm volatile("" : "+v"(pr[j]));
                        }
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            if (m < mcount) {
                                const float raw = dot_pairs(pr, xv[m][i]);
                                const float part =
                                    __builtin_fmaf(-Fmt<FMT>::kBias, sx[m][i], raw);
                                acc[b * MTP + m][mt] =
                                    __builtin_fmaf(s, part, acc[b * MTP + m][mt]);
                            }
                    }
            // the row sums over the row's LPR lanes, all (row, token) pairs of the batch at
            // once; each sum ends on one lane of the group (tr_writer), which finishes it
            // (SwiGLU, rounding, store), so the epilogues run side by side
            group_sum_many<LPR, NR, NMAT>(acc, lane);
            constexpr int R = NR > LPR ? NR / LPR : 1;
            const int idx0 = tr_index<LPR, NR>(lane) * R;
            const bool writer = tr_writer<LPR, NR>(lane);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int idx = idx0 + r, m = idx % MTP;
                const int row = row_base + (it0 + idx / MTP) * RPW;
                int orr = orow[0];
#pragma unroll
                for (int mm = 1; mm < MT; ++mm)
                    if (m == mm) orr = orow[mm];
                if (writer && row < rows && m < mcount) {
                    const float v0 = acc[r][0];
                    float res;
                    if constexpr (MODE == kModeGateUp)
                        res = v0 / (1.0f + expf(-v0)) * acc[r][NMAT - 1];
                    else
                        res = v0;
                    out[(size_t)orr * rows + row] = (uint16_t)f32_to_bf16(res);
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

// Sorted mode: more rows per wave (a block streams 4x the bytes of a ballot-mode block, so
// the slot lookup and the activation loads are paid over more weights); a row's
// arithmetic does not depend on ITERS.
template <int K, int FMT>
struct SortedShape {
    static constexpr int LPR = Shape<K>::LPR;
    static constexpr int GPL = Shape<K>::GPL;
    // int6 groups take 6 registers: half the rows keep the wave out of scratch
    static constexpr int ITERS = (GPL >= 2 || FMT == MOE_FMT_INT6_G32) ? 2 : 4;
    static constexpr int RPB = 4 * ITERS * (64 / LPR);
};

}  // namespace
}  // namespace moe
