// topk_common.h -- top-k expert selection and gate weights of one token by one wavefront.
//
// Every token goes to k of E routed experts [Strata 与 Qwen3.8-Flash-Next (telli.sh),
// section 稀疏架构创造了机会]; the gate weights are the softmax over the k selected
// logits, renormalised over the selection.  The result is exact (no approximation): the k
// largest logits in descending order, equal logits taken lower expert id first.
//
// Keys: each (logit, expert) becomes a 64-bit key whose unsigned order is the selection
// order -- the logit mapped to an order-preserving unsigned integer (-0 first turned into
// +0, so the two compare equal) in the high word, 0xffffffff - e in the low word.  Lane l
// of the wave holds experts l, l + 64, ...; keys are unique, so the selection is the k
// largest keys in descending order.
#pragma once
#include "moe_common.h"

#pragma clang fp contract(off)

namespace moe {
namespace {

__device__ __forceinline__ uint32_t order_bits(float v) {
    uint32_t u = (v == 0.0f) ? 0u : __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP row broadcasts (gfx9): lane 15 of each row to the next row, lane 31 to rows 2 and 3
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// wave maximum of an unsigned 32-bit value, returned uniform: row maxima by DPP, then two
// row broadcasts carry the maximum to lane 63
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    uint32_t o;
    o = (uint32_t)dpp<kDppXor1>((int)v);       v = o > v ? o : v;
    o = (uint32_t)dpp<kDppXor2>((int)v);       v = o > v ? o : v;
    o = (uint32_t)dpp<kDppHalfMirror>((int)v); v = o > v ? o : v;
    o = (uint32_t)dpp<kDppMirror>((int)v);     v = o > v ? o : v;
    // rows 1 and 3 take the previous row's maximum; then rows 2 and 3 take lane 31's
    o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast15, 0xa, 0xf, false);
    v = o > v ? o : v;
    o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kDppRowBcast31, 0xc, 0xf, false);
    v = o > v ? o : v;
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Descending sort of N (a power of two) keys held by one lane: Batcher's odd-even merge
// sort network (19 comparators for N = 8).
template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[N]) {
#pragma unroll
    for (int p = 1; p < N; p <<= 1)
#pragma unroll
        for (int kk = p; kk >= 1; kk >>= 1)
#pragma unroll
            for (int j = kk % p; j + kk < N; j += 2 * kk)
#pragma unroll
                for (int i = 0; i < kk; ++i)
                    if (i + j + kk < N && (i + j) / (2 * p) == (i + j + kk) / (2 * p)) {
                        const uint64_t x = key[i + j], y = key[i + j + kk];
                        key[i + j] = x > y ? x : y;
                        key[i + j + kk] = x > y ? y : x;
                    }
}

// Lane j < k of the calling wave holds the j-th selected key (descending); the rest hold 0.
// Serial form: each lane sorts its keys once; each of k rounds takes the wave maximum of
// the lanes' first keys on the high words alone, and only when several lanes tie on the
// high word a second round on the low words decides; the winning lane drops its key.
template <int NPL>
__device__ __forceinline__ uint64_t select_serial(uint64_t (&key)[NPL], int k) {
    const int lane = threadIdx.x & 63;
    sort_desc<NPL>(key);
    uint32_t khi[NPL], klo[NPL];
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        khi[i] = (uint32_t)(key[i] >> 32);
        klo[i] = (uint32_t)key[i];
    }
    uint32_t mine_hi = 0u, mine_lo = 0u;
    for (int j = 0; j < k; ++j) {
        const uint32_t m = wave_max_u32(khi[0]);
        uint64_t wmask = __ballot(khi[0] == m);
        if (__popcll(wmask) > 1) {
            // equal high words: the larger low word (the lower id) wins; low words are
            // unique among real keys, and a real key's low word beats padding's 0
            const uint32_t lm = wave_max_u32(khi[0] == m ? klo[0] : 0u);
            wmask = __ballot(khi[0] == m && klo[0] == lm);
        }
        const int wl = (int)__builtin_ctzll(wmask);
        const uint32_t wl_lo = (uint32_t)__builtin_amdgcn_readlane((int)klo[0], wl);
        if (lane == j) {
            mine_hi = m;
            mine_lo = wl_lo;
        }
        if (lane == wl) {
#pragma unroll
            for (int i = 0; i + 1 < NPL; ++i) {
                khi[i] = khi[i + 1];
                klo[i] = klo[i + 1];
            }
            khi[NPL - 1] = 0u;
            klo[NPL - 1] = 0u;
        }
    }
    return ((uint64_t)mine_hi << 32) | mine_lo;
}

// Selection and weights of one token's E logits (lt, fp32) by the calling wave; every lane
// of the wave must call it.  Lane j < k returns the j-th selected expert and its weight.
// Needs 1 <= k <= min(E, 64) and E <= 64 * NPL; `scratch` is 128 keys of LDS owned by the
// calling wave.  COHERENT: the logits were just stored by other blocks of the same launch
// (device-scope stores), so they are read device-scope.
//
// Fast form (exact, for any input): let T be the largest multiple of 2^16 such that at
// least k of the 64 lanes' largest high words are >= T (a bitwise search over the top 16
// bits, one value per lane).  At least k keys have a high word >= T, so every selected key
// does; these candidates (usually a few more than k) are compacted into LDS and each one's
// rank among them is counted.  When there are more than 64 candidates (many equal logits)
// the serial form runs instead.
//
// topk_regs takes the logits in registers (v[i] = logit of expert lane + 64 i);
// topk_wave loads them first.  The pieces below are also used on their own by a caller
// that already knows a candidate set containing the k largest (route.hip).

// keys of the lane's experts lane + 64 i (padding keys 0)
template <int NPL>
__device__ __forceinline__ void make_keys(const float (&v)[NPL], int E, uint64_t (&key)[NPL]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = (e < E) ? (((uint64_t)order_bits(v[i]) << 32) | (0xffffffffu - (uint32_t)e))
                         : 0ull;                       // padding keys lose to every id
    }
}

// The k largest of the C <= 64 candidate keys marked by bal (one ballot per key slot i),
// which must include the k largest keys overall: lane j < k returns the j-th, others 0.
// Compaction in (i, lane) order, then each candidate's rank among the candidates (keys
// are unique).
template <int NPL>
__device__ __forceinline__ uint64_t rank_candidates(const uint64_t (&key)[NPL],
                                                    const uint64_t (&bal)[NPL], int C, int k,
                                                    uint64_t* scratch) {
    const int lane = threadIdx.x & 63;
    int base = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        if ((bal[i] >> lane) & 1ull)
            scratch[base + __popcll(bal[i] & ((1ull << lane) - 1ull))] = key[i];
        base += __popcll(bal[i]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane c holds candidate c; its rank counts the larger candidates, read lane by lane
    const uint64_t ck = lane < C ? scratch[lane] : 0ull;
    const uint32_t ck_hi = (uint32_t)(ck >> 32), ck_lo = (uint32_t)ck;
    int rank = 0;
    for (int c = 0; c < C; ++c) {
        const uint32_t o_hi = (uint32_t)__builtin_amdgcn_readlane((int)ck_hi, c);
        const uint32_t o_lo = (uint32_t)__builtin_amdgcn_readlane((int)ck_lo, c);
        rank += (o_hi > ck_hi || (o_hi == ck_hi && o_lo > ck_lo)) ? 1 : 0;
    }
    if (lane < C && rank < k) scratch[64 + rank] = ck;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    return lane < k ? scratch[64 + lane] : 0ull;
}

// expert and weight of the selection's lane j < k: softmax over the k selected logits in
// fp32, shifted by the largest
__device__ __forceinline__ void finish_selection(uint64_t mine, int k, int& out_e,
                                                 float& out_w) {
    const int lane = threadIdx.x & 63;
    const uint32_t my_hi = (uint32_t)(mine >> 32), my_lo = (uint32_t)mine;
    const uint32_t vbits = (my_hi & 0x80000000u) ? (my_hi & 0x7fffffffu) : ~my_hi;
    const float my_v = (lane < k) ? __uint_as_float(vbits) : 0.0f;
    const float vmax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, my_v), 0));
    const float ex = (lane < k) ? expf(my_v - vmax) : 0.0f;
    // lanes k.. hold exact zeros: for k <= 16 the sum over the first 16 lanes is the same
    // value the full butterfly gives (its further levels add zeros)
    const float sum = k <= 16 ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                    __builtin_bit_cast(int, group_sum<16>(ex)), 0))
                              : group_sum<64>(ex);
    out_e = (int)(0xffffffffu - my_lo);
    out_w = ex / sum;
}

// The whole selection from keys: fast form when at most 64 keys reach the threshold T,
// serial form otherwise.
template <int NPL>
__device__ __forceinline__ uint64_t select_keys(uint64_t (&key)[NPL], int k,
                                                uint64_t* scratch) {
    uint32_t lmax = 0u;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const uint32_t h = (uint32_t)(key[i] >> 32);
        lmax = h > lmax ? h : lmax;
    }
    // T: the largest multiple of 2^16 with at least k lane maxima >= T (a search over the
    // top 16 bits; a lower threshold only admits a few more candidates)
    uint32_t T = 0u;
#pragma unroll
    for (int b = 31; b >= 16; --b) {
        const uint32_t c = T | (1u << b);
        if (__popcll(__ballot(lmax >= c)) >= k) T = c;
    }
    uint64_t bal[NPL];
    int C = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        bal[i] = __ballot((uint32_t)(key[i] >> 32) >= T);
        C += __popcll(bal[i]);
    }
    if (C <= 64) return rank_candidates<NPL>(key, bal, C, k, scratch);
    return select_serial<NPL>(key, k);
}

template <int NPL>
__device__ __forceinline__ void topk_regs(const float (&v)[NPL], int E, int k,
                                          uint64_t* scratch, int& out_e, float& out_w) {
    uint64_t key[NPL];
    make_keys<NPL>(v, E, key);
    finish_selection(select_keys<NPL>(key, k, scratch), k, out_e, out_w);
}

template <int NPL, bool COHERENT>
__device__ __forceinline__ void topk_wave(const float* lt, int E, int k, uint64_t* scratch,
                                          int& out_e, float& out_w) {
    const int lane = threadIdx.x & 63;
    float v[NPL];
    // all loads first, unconditionally (clamped index), so they are in flight together
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
        const int e = min(lane + 64 * i, E - 1);
        if constexpr (COHERENT)
            v[i] = __hip_atomic_load(const_cast<float*>(lt) + e, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        else
            v[i] = lt[e];
    }
    topk_regs<NPL>(v, E, k, scratch, out_e, out_w);
}

}  // namespace
}  // namespace moe
