// ffn_gemv.hip -- expert FFN for few tokens (decode): stream the selected experts'
// packed weights once, dequantise in registers, reduce across the wavefront.
//
// Decode reads every active weight once per step and is bound by memory bandwidth
// [Halogen Flash Server配置與實測 (lcz.me), replies comparing decode with bandwidth];
// only the selected experts are touched, which is what sparse routing saves
// [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].
//
// The per-row arithmetic lives in gemv_common.h.  Two launches, gate/up + SwiGLU -> h (bf16)
// then down -> y (sorted mode adds the chunk list's launch before them).  In each, a block
// owns one slot and a block of rows and requests its activation rows and every weight load
// before any arithmetic.
//
// Grouped mode (at most kGemvMaxBallotPairs = 24 pairs): a slot is a pair p.  A block reads the whole ids vector
// with one load, so the expert e = ids[p] is known after one memory round trip and the
// weight loads start at once; the pairs routed to e form a ballot mask, every MT-th of
// them leads a chunk of MT pairs and the others return.  A pair's row is its
// expert-sorted position (valid pairs with a smaller id, plus earlier pairs with the same
// id), the same position moe_permute assigns.
// Dense mode (shared expert): a slot is a chunk of MT tokens.
// Sorted mode (more than 24 pairs): the grouping from moe_permute
// is read instead of a ballot; a small kernel lists, expert by expert, chunks of at most MT
// consecutive sorted positions with their tokens (sentinels fill the list to the grid's
// size), and a slot is one chunk.  Each expert's rows are streamed once per chunk, four
// rows per wave.  MT = kGemvSortedMT: larger chunks re-stream a hot expert's weights less
// often, smaller ones keep the wave's registers (each token's activations) low enough for
// more waves per SIMD and spread a hot expert over more blocks.  A pair's arithmetic is the
// same in every mode, so its output bits do not depend on the mode (or on the other pairs of
// the call).
#include "gemv_common.h"

namespace moe {
namespace {

// Chunk list of sorted mode: for every expert e with n pairs, ceil(n / MT) entries of two
// int4, (e, first sorted position q0, pairs in the chunk, 0) and the tokens of its pairs
// (the last repeated); entries from the list's end up to cap hold e = -1, so a block
// learns from its own entry alone whether it has work.  Split call (hot > 0): an expert with
// hot pairs or more gets no chunks but entries of the grouped GEMM's work list instead
// (kMfmaTileRows pairs each: (e, first position, end of e's positions, 0)) and the list's
// length goes to *tile_count.  One block, E <= 1024.
__global__ void __launch_bounds__(1024) build_chunks_kernel(const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ sorted,
                                                            int E, int k, int MT, int hot,
                                                            int cap, int4* __restrict__ chunks,
                                                            int4* __restrict__ tiles,
                                                            int* __restrict__ tile_count) {
    __shared__ int part[2][16];
    __shared__ int total;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int b = 0, n = 0, cnt = 0, tcnt = 0;
    if (tid < E) {
        b = offsets[tid];
        n = offsets[tid + 1] - b;
        if (hot > 0 && n >= hot)
            tcnt = (n + kMfmaTileRows - 1) / kMfmaTileRows;
        else
            cnt = (n + MT - 1) / MT;
    }
    int incl = cnt, tincl = tcnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64), to = __shfl_up(tincl, off, 64);
        if (lane >= off) {
            incl += o;
            tincl += to;
        }
    }
    if (lane == 63) {
        part[0][wv] = incl;
        part[1][wv] = tincl;
    }
    __syncthreads();
    if (tid < 2) {
        int run = 0;
        for (int i = 0; i < 16; ++i) {
            const int v = part[tid][i];
            part[tid][i] = run;
            run += v;
        }
        if (tid == 0) total = run;
        else if (tile_count) *tile_count = run;
    }
    __syncthreads();
    const int start = incl - cnt + part[0][wv];
    for (int i = 0; i < cnt; ++i) {
        const int q0 = b + i * MT, sn = min(MT, n - i * MT);
        int t[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) t[m] = sorted[q0 + min(m, sn - 1)] / k;
        chunks[2 * (start + i)] = make_int4(tid, q0, sn, 0);
        chunks[2 * (start + i) + 1] = make_int4(t[0], t[1], t[2], t[3]);
    }
    const int tstart = tincl - tcnt + part[1][wv];
    for (int i = 0; i < tcnt; ++i)
        tiles[tstart + i] = make_int4(tid, b + i * kMfmaTileRows, b + n, 0);
    for (int i = total + tid; i < cap; i += 1024) chunks[2 * i] = make_int4(-1, 0, 0, 0);
}

// Slot of sorted mode: entry blockIdx.y of the list, or false for an empty entry.
__device__ __forceinline__ bool sorted_slot(const int4* chunks, Slot& sl) {
    const int4 c = chunks[2 * blockIdx.y];
    if (c.x < 0) return false;
    const int4 t = chunks[2 * blockIdx.y + 1];
    sl.e = c.x;
    sl.members = 0;
    sl.seg0 = 0;
    sl.first = 0;
    sl.dense0 = sl.dense_n = 0;
    sl.q0 = c.y;
    sl.sn = c.z;
    sl.tok[0] = t.x; sl.tok[1] = t.y; sl.tok[2] = t.z; sl.tok[3] = t.w;
    return true;
}

// grid.x = row blocks, grid.y = slots
template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_gateup_kernel(
    const uint8_t* __restrict__ wg, const uint16_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint16_t* __restrict__ su,
    const uint16_t* __restrict__ x, int T, int k, const int32_t* __restrict__ ids, int E,
    uint16_t* __restrict__ h) {
    using GU = Shape<D>;   // gate/up rows have K = d_model
    Slot sl;
    if (!resolve_slot<MT>(blockIdx.y, T, k, ids, E, sl)) return;
    gemv_rows<FMT, kModeGateUp, GU::LPR, GU::GPL, GU::ITERS, MT>(wg, sg, wu, su, x, k, F,
                                                                blockIdx.x, sl, h);
}

template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_down_kernel(
    const uint8_t* __restrict__ wd, const uint16_t* __restrict__ sd,
    const uint16_t* __restrict__ h, int T, int k, const int32_t* __restrict__ ids, int E,
    uint16_t* __restrict__ y) {
    using DN = Shape<F>;   // down rows have K = d_ff
    Slot sl;
    if (!resolve_slot<MT>(blockIdx.y, T, k, ids, E, sl)) return;
    gemv_rows<FMT, kModeDown, DN::LPR, DN::GPL, DN::ITERS, MT>(wd, sd, nullptr, nullptr, h, k,
                                                              D, blockIdx.x, sl, y);
}

template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_gateup_sorted_kernel(
    const uint8_t* __restrict__ wg, const uint16_t* __restrict__ sg,
    const uint8_t* __restrict__ wu, const uint16_t* __restrict__ su,
    const uint16_t* __restrict__ x, int k, const int4* __restrict__ chunks,
    uint16_t* __restrict__ h) {
    using GU = SortedShape<D, FMT>;
    Slot sl;
    if (!sorted_slot(chunks, sl)) return;
    gemv_rows<FMT, kModeGateUp, GU::LPR, GU::GPL, GU::ITERS, MT>(wg, sg, wu, su, x, k, F,
                                                                blockIdx.x, sl, h);
}

template <int FMT, int D, int F, int MT>
__global__ void __launch_bounds__(256) ffn_down_sorted_kernel(
    const uint8_t* __restrict__ wd, const uint16_t* __restrict__ sd,
    const uint16_t* __restrict__ h, int k, const int4* __restrict__ chunks,
    uint16_t* __restrict__ y) {
    using DN = SortedShape<F, FMT>;
    Slot sl;
    if (!sorted_slot(chunks, sl)) return;
    gemv_rows<FMT, kModeDown, DN::LPR, DN::GPL, DN::ITERS, MT>(wd, sd, nullptr, nullptr, h, k,
                                                              D, blockIdx.x, sl, y);
}

template <int FMT, int D, int F, int MT>
hipError_t launch_sorted_mt(const moe_experts& ex, const uint16_t* x, int T, int k,
                            const int32_t* offsets, const int32_t* sorted, uint16_t* y,
                            void* ws, hipStream_t s) {
    const GemvSortedWs L = gemv_sorted_ws_layout((int64_t)T * k, ex.n_experts, F);
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(base + L.h);
    int4* chunks = reinterpret_cast<int4*>(base + L.chunks);
    const int cap = (int)gemv_sorted_chunk_capacity((int64_t)T * k, ex.n_experts);
    const int hot = gemv_hot_rows((int64_t)T * k);
    int4* tiles = reinterpret_cast<int4*>(base + L.tiles);
    int* tile_count = reinterpret_cast<int*>(base + L.count);
    build_chunks_kernel<<<1, 1024, 0, s>>>(offsets, sorted, ex.n_experts, k, MT, hot, cap,
                                           chunks, hot > 0 ? tiles : nullptr,
                                           hot > 0 ? tile_count : nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    constexpr int n_gu = (F + SortedShape<D, FMT>::RPB - 1) / SortedShape<D, FMT>::RPB;
    constexpr int n_dn = (D + SortedShape<F, FMT>::RPB - 1) / SortedShape<F, FMT>::RPB;
    // grid (row block, chunk): with the row block fastest and a multiple of 8 row blocks,
    // row block r always runs on XCD r % 8, so each XCD's L2 keeps its share of the rows of
    // an expert that several chunks stream
    ffn_gateup_sorted_kernel<FMT, D, F, MT><<<dim3(n_gu, cap), 256, 0, s>>>(
        ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x, k, chunks, h);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_down_sorted_kernel<FMT, D, F, MT><<<dim3(n_dn, cap), 256, 0, s>>>(
        ex.w_down, ex.s_down, h, k, chunks, y);
    err = hipGetLastError();
    if (err != hipSuccess || hot == 0) return err;
    // the experts with `hot` pairs or more: the grouped GEMM, on the same h and y
    return launch_ffn_mfma_hot(ex, x, T, k, sorted, y, h, tiles, tile_count, L.tile_cap, s);
}

template <int FMT, int D, int F, int MT>
hipError_t launch_mt(const moe_experts& ex, const uint16_t* x, int T, int k, const int32_t* ids,
                     uint16_t* y, uint16_t* h, hipStream_t s) {
    const int nslots = ids ? T * k : (T + MT - 1) / MT;
    constexpr int n_gu = (F + Shape<D>::RPB - 1) / Shape<D>::RPB;
    constexpr int n_dn = (D + Shape<F>::RPB - 1) / Shape<F>::RPB;
    // grid (row block, slot), the row block fastest: row block r on XCD r % 8, so slots
    // that stream the same expert (the dense mode's token chunks) find its rows in that L2
    ffn_gateup_kernel<FMT, D, F, MT><<<dim3(n_gu, nslots), 256, 0, s>>>(
        ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x, T, k, ids, ex.n_experts, h);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    ffn_down_kernel<FMT, D, F, MT><<<dim3(n_dn, nslots), 256, 0, s>>>(
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
                      const int32_t* ids, const int32_t* offsets, const int32_t* sorted,
                      uint16_t* y, void* ws, hipStream_t s) {
#define MOE_DEC(DV, FV)                                                                  \
    if (ex.d_model == DV && ex.d_ff == FV) {                                             \
        if (ids && (int64_t)T * k > kGemvMaxBallotPairs)                                 \
            return launch_sorted_mt<FMT, DV, FV, kGemvSortedMT>(ex, x, T, k, offsets,    \
                                                                sorted, y, ws, s);       \
        return launch_shape<FMT, DV, FV>(ex, x, T, k, ids, y, ws, s);                    \
    }
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

// Pairs from which an expert goes to the grouped GEMM (0: the whole call on the GEMV).  The
// GEMM's fixed cost per tile (a few microseconds of prologue and epilogue, and a launch
// after the GEMV's) pays off only when enough pairs share few experts: measured with spread
// and Zipf routing at 16 to 192 tokens of top-10 over 512 experts.
int gemv_hot_rows(int64_t rows) {
    if (rows < kHybridMinRows) return 0;
    return rows <= 1024 ? 8 : 4;
}

// chunks of the GEMV's experts: at most one per pair, one per kGemvSortedMT pairs plus one
// per expert, and (split call) ceil((hot - 1) / kGemvSortedMT) per expert
size_t gemv_sorted_chunk_capacity(int64_t rows, int E) {
    int64_t c = (rows + kGemvSortedMT - 1) / kGemvSortedMT + E;
    c = c < rows ? c : rows;
    const int hot = gemv_hot_rows(rows);
    if (hot > 0) {
        const int64_t per_e = (int64_t)E * ((hot - 1 + kGemvSortedMT - 1) / kGemvSortedMT);
        c = c < per_e ? c : per_e;
    }
    return (size_t)c;
}

GemvSortedWs gemv_sorted_ws_layout(int64_t rows, int E, int F) {
    auto al = [](size_t n) { return (n + 255) & ~size_t(255); };
    GemvSortedWs w;
    size_t off = 0;
    w.h = off; off += al((size_t)rows * F * 2);
    w.chunks = off; off += al(gemv_sorted_chunk_capacity(rows, E) * 2 * sizeof(int4));
    const int hot = gemv_hot_rows(rows);
    w.tile_cap = hot > 0 ? ffn_mfma_hot_tile_capacity(rows, E, hot) : 0;
    w.tiles = off; off += al(w.tile_cap * sizeof(int4));
    w.count = off; off += al(sizeof(int));
    w.bytes = off;
    return w;
}

hipError_t launch_ffn_gemv(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* ids, const int32_t* offsets, const int32_t* sorted,
                           uint16_t* y, void* ws, hipStream_t s) {
    switch (ex.fmt) {
        case MOE_FMT_INT4_G32:
            return launch_fmt<MOE_FMT_INT4_G32>(ex, x, T, k, ids, offsets, sorted, y, ws, s);
        case MOE_FMT_INT6_G32:
            return launch_fmt<MOE_FMT_INT6_G32>(ex, x, T, k, ids, offsets, sorted, y, ws, s);
        case MOE_FMT_INT3_G32:
            return launch_fmt<MOE_FMT_INT3_G32>(ex, x, T, k, ids, offsets, sorted, y, ws, s);
        case MOE_FMT_INT2_G32:
            return launch_fmt<MOE_FMT_INT2_G32>(ex, x, T, k, ids, offsets, sorted, y, ws, s);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace moe
