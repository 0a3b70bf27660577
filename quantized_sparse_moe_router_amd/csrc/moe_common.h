// moe_common.h -- device helpers shared by the gfx950 kernels of the MoE layer, and the
// host-side prototypes of each kernel file's launcher.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}
// low / high bf16 of a packed pair
__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) {
    return __uint_as_float(pair & 0xffff0000u);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int shfl_xor(int v, int m) { return __shfl_xor(v, m, kWave); }

// DPP lane permutations (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1] pair lanes
// whose index differs in bit 0 / bit 1; row_half_mirror pairs lane i with 7-i inside each
// 8-lane group; row_mirror pairs lane i with 15-i inside each 16-lane row.  Applied in that
// order to values that are already equal across the smaller aligned block, each step adds
// the two halves of the next aligned block, i.e. the same tree as xor offsets 1, 2, 4, 8.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf,
                                                      false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// v + v of lane (lane ^ M), M = 16 or 32, with gfx950's v_permlane16/32_swap instead of a
// round trip through the LDS crossbar: swapping a copy of v with v leaves one operand
// holding the lower lane of each pair and the other the upper, and fp addition is
// commutative, so every lane gets the same bits as v + shfl_xor(v, M).
template <int M>
__device__ __forceinline__ float add_swapped(float v) {
    const uint32_t u = __float_as_uint(v);
    uint32_t lo, hi;
    if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        lo = r[0]; hi = r[1];
    } else {
        static_assert(M == 32, "offset 16 or 32");
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        lo = r[0]; hi = r[1];
    }
    return __uint_as_float(lo) + __uint_as_float(hi);
}

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of the group
// ends with the group's sum, combined as the butterfly tree over xor offsets 1..G/2.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v = v + dpp<kDppXor1>(v);
    if constexpr (G >= 4) v = v + dpp<kDppXor2>(v);
    if constexpr (G >= 8) v = v + dpp<kDppHalfMirror>(v);
    if constexpr (G >= 16) v = v + dpp<kDppMirror>(v);
    if constexpr (G >= 32) v = add_swapped<16>(v);
    if constexpr (G >= 64) v = add_swapped<32>(v);
    return v;
}

// ---- group_sum of many values at once, transposed
// group_sum spends one exchange and one add per level on every value, and leaves each sum on
// every lane.  With N values per lane, level j of the transposed form instead splits the
// values between the two partner lanes: each keeps one half and adds the partner's copy of
// it, so the level costs N/2 adds and the sums end spread over the lanes.  The partners and
// the order of the levels are group_sum's, so every sum is the same tree of the same
// additions (fp addition is commutative): the bits equal group_sum's.
//
// Which half a lane keeps at level j is bit sel_j of its lane index l (l0 = bit 0, ...):
//   sel_0 = l0 ^ l2, sel_1 = l1 ^ l2, sel_2 = l2 ^ l3, sel_j = lj for j >= 3.
// A lane and its partner at level j (l ^ 1, l ^ 2, l ^ 7, l ^ 15, l ^ 16, l ^ 32) differ in
// sel_j and agree in every earlier sel, so they hold the same values when they split them.
template <int J>
__device__ __forceinline__ bool tr_sel(int lane) {
    if constexpr (J == 0) return ((lane ^ (lane >> 2)) & 1) != 0;
    else if constexpr (J == 1) return (((lane >> 1) ^ (lane >> 2)) & 1) != 0;
    else if constexpr (J == 2) return (((lane >> 2) ^ (lane >> 3)) & 1) != 0;
    else return ((lane >> J) & 1) != 0;
}

// level j of group_sum on one value
template <int J>
__device__ __forceinline__ float bf_level(float v) {
    if constexpr (J == 0) return v + dpp<kDppXor1>(v);
    else if constexpr (J == 1) return v + dpp<kDppXor2>(v);
    else if constexpr (J == 2) return v + dpp<kDppHalfMirror>(v);
    else if constexpr (J == 3) return v + dpp<kDppMirror>(v);
    else return add_swapped<(J == 4) ? 16 : 32>(v);
}

// level j, transposed: lo / hi are values i and i + C/2 of the lane's C; returns the
// level's sum of the one this lane keeps (lo where sel_j = 0, hi where sel_j = 1).  The
// cross-row levels take both halves in one v_permlane16/32_swap: with (lo, hi) as
// (vdst, vsrc), the rows of lanes with bit j = 0 end with lo of both partners, the others
// with hi of both.
template <int J>
__device__ __forceinline__ float tr_level(float lo, float hi, bool sel) {
    if constexpr (J <= 3) {
        const float keep = sel ? hi : lo, send = sel ? lo : hi;
        constexpr int kCtrl = J == 0 ? kDppXor1 : J == 1 ? kDppXor2
                            : J == 2 ? kDppHalfMirror : kDppMirror;
        return keep + dpp<kCtrl>(send);
    } else {
        const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
        uint32_t x, y;
        if constexpr (J == 4) {
            const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
            x = r[0]; y = r[1];
        } else {
            const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
            x = r[0]; y = r[1];
        }
        return __uint_as_float(x) + __uint_as_float(y);
    }
}

// Levels J .. log2(G) - 1 on v[0 .. C-1] (tuples of NM values that travel together):
// transposed while a lane holds more than one tuple, then group_sum's levels.
template <int G, int J, int C, int N, int NM>
__device__ __forceinline__ void tr_levels(float (&v)[N][NM], int lane) {
    if constexpr ((1 << J) < G) {
        if constexpr (C > 1) {
            constexpr int H = C / 2;
            const bool sel = tr_sel<J>(lane);
#pragma unroll
            for (int i = 0; i < H; ++i)
#pragma unroll
                for (int c = 0; c < NM; ++c) v[i][c] = tr_level<J>(v[i][c], v[i + H][c], sel);
            tr_levels<G, J + 1, H, N, NM>(v, lane);
        } else {
#pragma unroll
            for (int c = 0; c < NM; ++c) v[0][c] = bf_level<J>(v[0][c]);
            tr_levels<G, J + 1, 1, N, NM>(v, lane);
        }
    }
}

// Sums over aligned groups of G lanes (a power of two <= 64) of N tuples (N a power of two)
// of NM values each, each sum bit-identical to group_sum<G>.  On return the lane holds
// R = max(1, N / G) tuples in v[0 .. R-1]: v[r] is tuple tr_index(lane) * R + r.  When
// N < G, G / N lanes of the group hold each tuple; tr_writer picks one of them.
template <int G, int N, int NM>
__device__ __forceinline__ void group_sum_many(float (&v)[N][NM], int lane) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "G: a power of two <= 64");
    static_assert(N >= 1 && (N & (N - 1)) == 0, "N: a power of two");
    tr_levels<G, 0, N, N, NM>(v, lane);
}

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// the index of the tuples a lane holds after group_sum_many<G, N, ...>, divided by R
template <int G, int N>
__device__ __forceinline__ int tr_index(int lane) {
    constexpr int NT = ilog2(N < G ? N : G);           // transposed levels
    int idx = 0;
    if constexpr (NT > 0) idx = idx * 2 + (int)tr_sel<0>(lane);
    if constexpr (NT > 1) idx = idx * 2 + (int)tr_sel<1>(lane);
    if constexpr (NT > 2) idx = idx * 2 + (int)tr_sel<2>(lane);
    if constexpr (NT > 3) idx = idx * 2 + (int)tr_sel<3>(lane);
    if constexpr (NT > 4) idx = idx * 2 + (int)tr_sel<4>(lane);
    if constexpr (NT > 5) idx = idx * 2 + (int)tr_sel<5>(lane);
    return idx;
}

// one lane per distinct tuple: sel_j = 0 at every level that was not transposed
template <int G, int N>
__device__ __forceinline__ bool tr_writer(int lane) {
    constexpr int NT = ilog2(N < G ? N : G), L = ilog2(G);
    // no level transposed: every lane of the group holds the sums, the first one writes
    if constexpr (NT == 0) return (lane & (G - 1)) == 0;
    bool w = true;
    if constexpr (NT <= 0 && L > 0) w = w && !tr_sel<0>(lane);
    if constexpr (NT <= 1 && L > 1) w = w && !tr_sel<1>(lane);
    if constexpr (NT <= 2 && L > 2) w = w && !tr_sel<2>(lane);
    if constexpr (NT <= 3 && L > 3) w = w && !tr_sel<3>(lane);
    if constexpr (NT <= 4 && L > 4) w = w && !tr_sel<4>(lane);
    if constexpr (NT <= 5 && L > 5) w = w && !tr_sel<5>(lane);
    return w;
}

}  // namespace moe

// ---------------------------------------------------------------- launchers (host)
// Each returns hipSuccess or the first HIP error of its launches.  Arguments are already
// validated by the C entry points.
namespace moe {

// Workspace area that holds an arrival counter.  It must be zero before a workspace's
// first use; every call leaves it zero.
constexpr size_t kRouteCounterBytes = 256;

// Device error word (per device): bit 0 = expert id out of range.  Returns its device
// address for the current device.
int* device_error_flag();
hipError_t read_and_clear_device_error(int* flag);

// Tokens up to which the router with the fused pre-layer norm runs (one launch, GEMV).
constexpr int kRouteGemvMaxTokens = 16;
// moe_route: up to this many tokens one launch (the last block selects every token, four at a
// time); above, the logits kernel and then the selection kernel (one wave per token, all in
// parallel): 88.8 -> 82.3 us per 16-token layer step when this went from 16 to 4
constexpr int kRouteOneLaunchMaxTokens = 4;
// Tokens up to which it computes the logits by GEMV (one wave per expert row, token groups)
// and selects in a second kernel; above, the tiled GEMM (or the bounded form).  The bounded
// form's three launches cost more than the GEMV's repeated router reads (which the L2 and
// the cache below it serve) up to about 512 tokens: a layer call at 128 tokens 284 -> 250 us,
// at 512 tokens 430 -> 415 us when this went from 64 to 512.
constexpr int kRouteSplitMaxTokens = 512;
// decode layer / block: up to this many tokens the router writes logits only and every
// gate/up block selects its token's experts itself; above, the router's last block selects
constexpr int kDecodeSelectMaxTokens = 1;

hipError_t launch_route(const moe_router& r, const uint16_t* x, int T, int k, int32_t* ids,
                        float* weights, float* logits, unsigned* counter, hipStream_t s);
// Router logits only (fp32 [T][E], the same values launch_route computes), for
// T <= kRouteSplitMaxTokens.
hipError_t launch_route_logits(const moe_router& r, const uint16_t* x, int T, float* logits,
                               hipStream_t s);

// The pre-layer norm fused into the router, for the decode block (T <= kRouteGemvMaxTokens):
// the router runs on xn = RMSNorm(x) (gamma [d], eps), stores xn [T][d] and, if gw is not
// null, the residual-gate logits z [T].  T == 1: logits only (the decode gate/up kernel
// selects); T > 1: logits, ids and weights as launch_route.
hipError_t launch_route_norm(const moe_router& r, const uint16_t* x, int T, int k,
                             const float* gamma, float eps, const float* gw, float gb,
                             uint16_t* xn, float* z, int32_t* ids, float* weights,
                             float* logits, unsigned* counter, hipStream_t s);
// The norm alone (and the gate logits when gw is not null), one wave per token.
hipError_t launch_rmsnorm(const uint16_t* x, int T, int d, const float* gamma, float eps,
                          const float* gw, float gb, uint16_t* xn, float* z, hipStream_t s);

// Many tokens, logits not wanted: the bounded form.  launch_route_bounded_logits writes
// every logit to within 2^-11 (|x_t| nw[e] + |b_e|) of the fixed-order value (MFMA; planes
// is a workspace of route_bounded_planes_bytes, nw [E] the row norm bounds);
// launch_route_bounded_select recomputes in the fixed order the experts that bound cannot
// rule out and selects: ids and weights are those of launch_route, bit for bit.
size_t route_bounded_planes_bytes(int E, int d);
hipError_t launch_route_bounded_logits(const moe_router& r, const uint16_t* x, int T,
                                       uint16_t* planes, float* nw, float* lf, hipStream_t s);
hipError_t launch_route_bounded_select(const moe_router& r, const uint16_t* x, int T, int k,
                                       const float* nw, const float* lf, int32_t* ids,
                                       float* weights, hipStream_t s);

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* ws, hipStream_t s);
size_t permute_ws_bytes(int64_t P, int E);

// Weight-streaming GEMV, gate/up then down.  Up to kGemvMaxBallotRows pairs the positions
// come from ids alone (a ballot; ws = [h]); above, from the grouping (offsets, sorted_pairs;
// ws = gemv_sorted_ws_layout).  From kHybridMinRows pairs the call is split by expert: an
// expert with fewer than gemv_hot_rows(rows) pairs runs the GEMV in sorted mode, one with
// more the grouped MFMA GEMM (its weights streamed once per 256 pairs instead of once per
// chunk); at prefill sizes that leaves the GEMM only the experts worth a tile.  Dense mode
// (ids == nullptr): the token index, at most kGemvMaxBallotRows tokens.
constexpr int64_t kGemvMaxBallotRows = 64;
// Grouped calls leave the ballot for sorted mode above this many pairs: the ballot's slots
// stream the experts' weights at a lower rate than the sorted chunks once a call holds a few
// dozen pairs (four-call layer, top-10 of 512: 3 tokens 44.8 -> 39.6 us, 4 51.8 -> 43.2,
// 6 65.3 -> 50.7 in sorted mode; 2 tokens 35.6 -> 36.0).
constexpr int64_t kGemvMaxBallotPairs = 24;
constexpr int kGemvSortedMT = 3;    // pairs of one expert per pass over its weights
constexpr int64_t kHybridMinRows = 640;
constexpr int kMfmaTileRows = 256;  // pairs per entry of the grouped GEMM's work list
int gemv_hot_rows(int64_t rows);    // 0: no split
struct GemvSortedWs {
    size_t h, chunks, tiles, count, bytes;
    size_t tile_cap;       // entries of the MFMA work list (hot experts)
};
size_t gemv_sorted_chunk_capacity(int64_t rows, int E);
GemvSortedWs gemv_sorted_ws_layout(int64_t rows, int E, int F);
bool ffn_gemv_has_shape(int d_model, int d_ff);
hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, const int32_t* offsets, const int32_t* sorted,
                           uint16_t* y, void* ws, hipStream_t s);
// Large calls: grouped MFMA GEMM.  ws = [h][tile list].
hipError_t launch_ffn_mfma(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           void* ws, hipStream_t s);
size_t ffn_mfma_ws_bytes(int64_t rows, int E, int F);
// the grouped GEMM for the experts with at least min_rows pairs only, on caller-placed
// buffers: h [rows][d_ff], a work list of tile_cap entries (ffn_mfma_hot_tile_capacity) and
// its count
// (the list already built: entries (e, first sorted position, end of e's positions, 0) of
// at most kMfmaTileRows pairs, then the count)
size_t ffn_mfma_hot_tile_capacity(int64_t rows, int E, int min_rows);
hipError_t launch_ffn_mfma_hot(const moe_experts& ex, const uint16_t* x, int T, int k,
                               const int32_t* sorted_pairs, uint16_t* y, uint16_t* h,
                               const int4* tiles, const int* count, size_t tile_cap,
                               hipStream_t s);

// z: residual-gate logits [T] or null
hipError_t launch_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* w,
                          const uint16_t* y_shared, const uint16_t* residual, const float* z,
                          int T, int k, int d, uint16_t* out, hipStream_t s);

// Expert side of a decode step (routed + shared FFN and combine) in two launches, at most
// 64 pairs and S = T*k (+ T shared) slots whose h rows fit in kDecodeMaxLds bytes of LDS.
// Workspace: [h rows].
constexpr size_t kDecodeMaxLds = 128 * 1024;
struct DecodeWs {
    size_t h, bytes;
};
DecodeWs decode_ws_layout(int T, int k, int d_model, int d_ff);
bool decode_fits(int T, int k, int d_ff, bool shared);
// logits non-null: the selection runs inside (ids and weights are written); null: ids and
// weights are inputs.
// z: residual-gate logits [T] applied in the combine, or null.
hipError_t launch_decode_ffn(const moe_experts& routed, const moe_experts* shared,
                             const uint16_t* x, int T, int k, const float* logits,
                             int32_t* ids, float* weights, const uint16_t* residual,
                             const float* z, uint16_t* out, void* ws, hipStream_t s);

// The two expert paths' weight decoders over n_groups consecutive 32-code groups (form 0:
// fp32 out[n_groups][32], the GEMV arithmetic on one-hot activations; form 1: bf16
// out[n_groups][32], the grouped GEMM's operand conversion).
hipError_t launch_dequant_probe(int fmt, int form, const uint8_t* w, const uint16_t* s,
                                int64_t n_groups, void* out, hipStream_t st);

}  // namespace moe
