// decode.hip -- the expert side of a decode step in two launches: routed and shared
// expert FFN (gate/up + SwiGLU, then down) and the weighted combine, for at most 64
// (token, expert) pairs.
//
// Decode streams each selected expert's packed weights once per token and is bound by
// memory bandwidth and latency, not arithmetic [Halogen Flash Server配置與實測 (lcz.me),
// replies comparing decode with bandwidth].  The per-call path runs gate/up, down and the
// combine for the routed experts, and the shared expert beside them, as five launches on
// two streams.  Here the S = P + T_s slots (P routed pairs, then T_s shared-expert tokens)
// share two launches on one stream:
//   decode_gateup_kernel  one block per (slot, 4-row block): h rows of every slot;
//   decode_down_kernel    one block per 4 output rows: those rows of y for every slot
//                         (h of all slots staged in LDS), combined in registers into the
//                         output rows -- y never goes to memory.
// Handing h over at a kernel boundary costs less than any wait between blocks of one
// launch: blocks on different XCDs see each other's stores only through device-coherent
// memory, a round trip of about a microsecond each way.  The per-row arithmetic is that
// of gemv_rows (gemv_common.h) and the combine repeats combine8's operations
// (combine_common.h) on each element, so the result equals the per-call path bit for bit.
#include "combine_common.h"
#include "gemv_common.h"
#include "topk_common.h"

namespace moe {
namespace {

struct DecodeArgs {
    const uint8_t *rg, *ru, *rd;       // routed experts
    const uint16_t *rsg, *rsu, *rsd;
    int E;
    const uint8_t *sg, *su, *sd;       // shared expert (sg == nullptr: none)
    const uint16_t *ssg, *ssu, *ssd;
    const uint16_t* x;
    int T, k;
    const float* logits;                // [T][E] router logits, or null: ids / weights given
    int32_t* ids;                       // [T][k]; written by the gate/up kernel when logits
    float* weights;                     //   are given, read-only otherwise
    const uint16_t* residual;
    const float* z;                     // [T] residual-gate logits, or null
    uint16_t* out;
    uint16_t* h;                        // [S][F] bf16: pair rows, then shared-token rows
    int* err;
};

// gate/up: 4 waves per block, each with one load instruction per matrix (short chains of
// arithmetic per wave once the data is in).  Small blocks spread the rows evenly over the
// CUs (1 408 blocks for one token), which shortens the arithmetic tail after the loads,
// at the price of one selection per block of 4 waves (measured 12.4 -> 11.9 us per
// moe_experts_decode and 17.2 -> 16.65 us per decode step against blocks of 16 waves)
constexpr int GU_WAVES = 4;
template <int K>
struct GuShape {
    static constexpr int LPR = Shape<K>::LPR;
    static constexpr int GPL = Shape<K>::GPL;
    static constexpr int RPB = GU_WAVES * (64 / LPR);   // rows per block
};

// 8 activations (16 bytes) as the group dot products take them from LDS (int4 pairs
// elements p, p + 4; the other formats neighbours)
template <int FMT>
__device__ __forceinline__ uint4 paired(uint4 v) {
    if constexpr (FMT == MOE_FMT_INT4_G32) return nibble_pairs(v.x, v.y, v.z, v.w);
    return v;
}

// ---- down: 4 output rows per block for every slot, then their combine.  16 waves: wave w
// takes row w % 4 and every 4th wave load of that row (part w / 4).  A row's K = d_ff
// codes are read by LPR lanes exactly as in gemv_rows; the 64 / LPR lane groups of a wave
// take different slots of the same row.
constexpr int DN_WAVES = 16;
constexpr int DN_THREADS = DN_WAVES * 64;
template <int F>
struct DnShape {
    static constexpr int LPR = Shape<F>::LPR;
    static constexpr int GPL = Shape<F>::GPL;
    static constexpr int NG = 64 / LPR;          // slots per wave load
    static constexpr int ROWS = 4;               // rows per block
    static constexpr int SPLIT = DN_WAVES / ROWS;   // waves per row
    // wave loads per wave in registers at once: one when every slot fits in one load per
    // wave (a token with 10 experts and the shared one), else batches of 3 (four tokens
    // with 10 experts and the shared one: 44 slots, 11 wave loads per row, at most 3 per
    // wave, so one batch and no load beyond the last slot's)
    static constexpr int ITB_SMALL = 1;
    static constexpr int ITB_LARGE = 3;
};

template <int FMT, int D, int F, int ITB>
__device__ __forceinline__ void down_rows_combine(const DecodeArgs& a, int r0, int S,
                                                  uint8_t* lds) {
    using DS = DnShape<F>;
    constexpr int LPR = DS::LPR, GPL = DS::GPL, NG = DS::NG;
    constexpr int GB = Fmt<FMT>::kGroupBytes;
    constexpr size_t ROW_BYTES = (size_t)F / 32 * GB;
    constexpr int NGRP = F / 32;                 // groups per h row
    constexpr int SPLIT = DS::SPLIT;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rw = wave % DS::ROWS, part = wave / DS::ROWS;
    const int gp = lane % LPR, sub = lane / LPR;
    const int row = r0 + rw;                     // < D: D is a multiple of DS::ROWS
    const int P = a.T * a.k;
    // LDS: h rows [S][F] bf16 | group sums of h [S][NGRP] | y [S][ROWS] | gate weights [64]
    uint16_t* h_lds = reinterpret_cast<uint16_t*>(lds);
    float* sx_lds = reinterpret_cast<float*>(lds + (size_t)S * F * 2);
    float* y_lds = sx_lds + (size_t)S * NGRP;
    float* w_lds = y_lds + (size_t)S * DS::ROWS;

    // Loads that need nothing, all unconditional (clamped indexes) so that the compiler
    // can count them: every slot's expert (lane l: pair l; an id outside [0, E), never
    // produced by moe_route, reads expert 0), the gate weights, the residual of token
    // `lane` (combined by this lane), and the first kHPass h chunks of this thread.
    int my_e = a.ids[min(lane, P - 1)];
    const float gate_w = a.weights[min((int)threadIdx.x, P - 1)];
    const uint16_t* res_src = a.residual ? a.residual : a.x;   // x: same shape, unused
    const uint16_t res_bits = res_src[(size_t)min(lane, a.T - 1) * D + row];
    // chunks per thread requested up front: every chunk of h for the one-load-per-wave
    // shapes (at most 1 024 chunks), three for the larger ones (44 slots at d_ff 512 -- four
    // tokens with 10 experts and the shared one -- are 2 816 chunks), so that the staging
    // costs one round trip
    constexpr int kHPass = (ITB == DnShape<F>::ITB_SMALL) ? 1 : 3;
    const int n16 = S * F / 8;                    // 16-byte chunks of h
    // native 4-vectors: an array of HIP's uint4 struct is not kept in registers
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4* hsrc = reinterpret_cast<const u32x4*>(a.h);
    u32x4* hdst = reinterpret_cast<u32x4*>(h_lds);
    u32x4 hv[kHPass];
#pragma unroll
    for (int u = 0; u < kHPass; ++u)
        hv[u] = hsrc[min(u * DN_THREADS + (int)threadIdx.x, n16 - 1)];
    // all of the above in flight before the wait for the expert ids: left to itself the
    // scheduler may place that wait first and request the h chunks only after it
    __builtin_amdgcn_sched_barrier(0);
    my_e = (lane < P && my_e >= 0 && my_e < a.E) ? my_e : 0;

    GroupBits<FMT> wbits[ITB][GPL];
    uint16_t sbits[ITB][GPL];
    // this wave's loads l0 .. l0 + ITB - 1: wave load part + SPLIT * l of the row, slot
    // (part + SPLIT * l) * NG + sub (slots past S - 1 repeat slot S - 1, so every load is
    // unconditional and in bounds)
    auto load_batch = [&](int l0) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < ITB; ++q) {
            const int s = min((part + SPLIT * (l0 + q)) * NG + sub, S - 1);
            const int e = __shfl(my_e, s, 64);
            const uint8_t* wb;
            const uint16_t* sb;
            if (s < P) {
                const size_t mrow = (size_t)e * D + row;
                wb = a.rd + mrow * ROW_BYTES;
                sb = a.rsd + mrow * (F / 32);
            } else {
                wb = a.sd + (size_t)row * ROW_BYTES;
                sb = a.ssd + (size_t)row * (F / 32);
            }
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = gp + LPR * i;
                load_bits<FMT>(wb + (size_t)g * GB, wbits[q][i]);
                sbits[q][i] = load_scale(sb + g);
            }
        }
    };
    // the ITB dot products are independent chains: all of them first (one basic block,
    // so their latencies overlap), then the row sums and the stores
    auto compute_batch = [&](int l0) __attribute__((always_inline)) {
        float acc[ITB];
#pragma unroll
        for (int q = 0; q < ITB; ++q) {
            const int s = min((part + SPLIT * (l0 + q)) * NG + sub, S - 1);
            acc[q] = 0.0f;
#pragma unroll
            for (int i = 0; i < GPL; ++i) {
                const int g = gp + LPR * i;
                uint32_t xv[16];
                const uint4* src = reinterpret_cast<const uint4*>(h_lds + (size_t)s * F + 32 * g);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint4 t4 = src[v];
                    xv[4 * v] = t4.x; xv[4 * v + 1] = t4.y;
                    xv[4 * v + 2] = t4.z; xv[4 * v + 3] = t4.w;
                }
                const float sx = sx_lds[s * NGRP + g];
                const float sc = f16_to_f32(sbits[q][i]);
                if constexpr (kPairInRegisters<FMT>) pair_in_registers<FMT>(xv);
                const float raw = dot_bits<FMT>(wbits[q][i], xv);
                const float part = __builtin_fmaf(-Fmt<FMT>::kBias, sx, raw);
                acc[q] = __builtin_fmaf(sc, part, acc[q]);
            }
        }
        float yv[ITB];
#pragma unroll
        for (int q = 0; q < ITB; ++q) yv[q] = bf16_to_f32(f32_to_bf16(group_sum<LPR>(acc[q])));
#pragma unroll
        for (int q = 0; q < ITB; ++q) {
            const int s_raw = (part + SPLIT * (l0 + q)) * NG + sub;
            if (gp == 0 && s_raw < S) y_lds[s_raw * DS::ROWS + rw] = yv[q];
        }
    };

    // wave loads of this wave: part, part + SPLIT, ... below ceil(S / NG)
    const int n_l = ((S + NG - 1) / NG - part + SPLIT - 1) / SPLIT;
    load_batch(0);
    __builtin_amdgcn_sched_barrier(0);
    if (threadIdx.x < P) w_lds[threadIdx.x] = gate_w;
    // h rows -> LDS (int4: in nibble_pairs order).  An index past the end is clamped to the
    // last chunk, which then stores the same value twice: no branch, so no wait per chunk.
    auto to_lds = [&](int c, u32x4 v) __attribute__((always_inline)) {
        const uint4 p = paired<FMT>(make_uint4(v[0], v[1], v[2], v[3]));
        hdst[c] = u32x4{p.x, p.y, p.z, p.w};
    };
#pragma unroll
    for (int u = 0; u < kHPass; ++u) to_lds(min(u * DN_THREADS + (int)threadIdx.x, n16 - 1), hv[u]);
    for (int c0 = kHPass * DN_THREADS; c0 < n16; c0 += kHPass * DN_THREADS) {
        u32x4 hw[kHPass];
#pragma unroll
        for (int u = 0; u < kHPass; ++u)
            hw[u] = hsrc[min(c0 + u * DN_THREADS + (int)threadIdx.x, n16 - 1)];
#pragma unroll
        for (int u = 0; u < kHPass; ++u)
            to_lds(min(c0 + u * DN_THREADS + (int)threadIdx.x, n16 - 1), hw[u]);
    }
    __syncthreads();
    // group sums of h, once per (slot, group), in group_sum_x's order
    for (int i = threadIdx.x; i < S * NGRP; i += DN_THREADS)
        sx_lds[i] = group_sum_x(reinterpret_cast<const uint32_t*>(h_lds + (size_t)i * 32));
    __syncthreads();
    for (int l0 = 0; l0 < n_l; l0 += ITB) {
        if (l0 > 0) load_batch(l0);
        compute_batch(l0);
    }
    __syncthreads();

    // combine: lane t of the row's first wave, token t of the row, in combine8's order of
    // operations
    if (part != 0) return;
    const float* y = y_lds + rw;
    for (int t = lane; t < a.T; t += 64) {
        float acc = 0.0f;
        for (int j0 = 0; j0 < a.k; j0 += 8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int jj = min(j0 + j, a.k - 1);
                const float wj = (j0 + j < a.k) ? w_lds[t * a.k + jj] : 0.0f;
                acc = __builtin_fmaf(wj, y[(t * a.k + jj) * DS::ROWS], acc);
            }
        }
        if (a.sg) acc += y[(P + t) * DS::ROWS];
        if (a.z) acc = gate_value(a.z[t]) * acc;
        uint32_t o;
        if (a.residual) {
            const float r = bf16_to_f32(t == lane ? res_bits : a.residual[(size_t)t * D + row]);
            o = f32_to_bf16(r + bf16_to_f32(f32_to_bf16(acc)));
        } else {
            o = f32_to_bf16(acc);
        }
        a.out[(size_t)t * D + row] = (uint16_t)o;
    }
}

template <int F>
constexpr size_t dn_lds_bytes(int S) {
    return (size_t)S * F * 2 + (size_t)S * (F / 32) * 4 + (size_t)S * DnShape<F>::ROWS * 4 +
           64 * 4;
}

// NPL > 0: every block selects its token's experts from the logits itself (topk_wave, each
// wave redundantly, so no block waits for another) and the first row block of each
// token's first pair writes that token's ids and weights.  NPL = 0: ids are given.
template <int FMT, int D, int F, int NPL>
__global__ void __launch_bounds__(GU_WAVES * 64) decode_gateup_kernel(DecodeArgs a) {
    using GU = GuShape<D>;   // gate/up rows: K = d_model
    constexpr int n_gu = (F + GU::RPB - 1) / GU::RPB;
    const int P = a.T * a.k;
    const int s = blockIdx.x / n_gu, rb = blockIdx.x % n_gu;
    const bool pair = s < P;
    // the slot's activation row (token s / k, or s - P for the shared expert) goes to LDS
    // once per block, in 16-byte pieces: requested first and stored only after
    // the expert id (or the selection's logits) has been requested too, so that the two
    // round trips overlap instead of following each other
    constexpr int NT = GU_WAVES * 64;
    constexpr int XP = (D / 8 + NT - 1) / NT;            // 16-byte x pieces per thread
    __shared__ __attribute__((aligned(16))) uint16_t x_lds[D];
    const uint4* xsrc = reinterpret_cast<const uint4*>(a.x + (size_t)(pair ? s / a.k : s - P) * D);
    uint4 xq[XP];
#pragma unroll
    for (int p = 0; p < XP; ++p) xq[p] = xsrc[min((int)threadIdx.x + NT * p, D / 8 - 1)];
    auto store_x = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < XP; ++p) {
            const int xi = (int)threadIdx.x + NT * p;
            if (xi < D / 8) reinterpret_cast<uint4*>(x_lds)[xi] = paired<FMT>(xq[p]);
        }
    };
    // dense form of gemv_rows: one token, activation row 0 (x_lds), output row 0 of `out`
    Slot sl;
    sl.first = 0;
    sl.members = 0;
    sl.seg0 = 0;
    sl.dense0 = 0;
    sl.dense_n = 1;
    if (pair) {
        // h row s.  An id outside [0, E) (never produced by the selection) reads expert 0
        // and raises device error bit 0.
        int e;
        if constexpr (NPL > 0) {
            // wave 0 selects, the block reads its expert from LDS
            const int t = s / a.k, j = s - t * a.k;
            __shared__ int sel_lds;
            __shared__ uint64_t scratch[128];
            if (threadIdx.x < 64) {
                int sel_e;
                float sel_w;
                topk_wave<NPL, false>(a.logits + (size_t)t * a.E, a.E, a.k, scratch, sel_e,
                                      sel_w);
                if (threadIdx.x == j) sel_lds = sel_e;
                if (j == 0 && rb == 0 && threadIdx.x < a.k) {
                    a.ids[(size_t)t * a.k + threadIdx.x] = sel_e;
                    a.weights[(size_t)t * a.k + threadIdx.x] = sel_w;
                }
            }
            store_x();
            __syncthreads();
            e = sel_lds;
        } else {
            e = a.ids[s];
            store_x();
            __syncthreads();
        }
        sl.e = (e >= 0 && e < a.E) ? e : 0;
        if (sl.e != e && threadIdx.x == 0 && rb == 0) atomicOr(a.err, 1);
        gemv_rows<FMT, kModeGateUp, GU::LPR, GU::GPL, 1, 1, GU_WAVES, true>(
            a.rg, a.rsg, a.ru, a.rsu, x_lds, a.k, F, rb, sl, a.h + (size_t)s * F);
    } else {
        store_x();
        __syncthreads();
        sl.e = 0;
        gemv_rows<FMT, kModeGateUp, GU::LPR, GU::GPL, 1, 1, GU_WAVES, true>(
            a.sg, a.ssg, a.su, a.ssu, x_lds, a.k, F, rb, sl, a.h + (size_t)s * F);
    }
}

template <int FMT, int D, int F, int ITB>
__global__ void __launch_bounds__(DN_THREADS) decode_down_kernel(DecodeArgs a) {
    const int S = a.T * a.k + (a.sg ? a.T : 0);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    down_rows_combine<FMT, D, F, ITB>(a, blockIdx.x * DnShape<F>::ROWS, S, lds);
}

template <int FMT, int D, int F, int ITB>
hipError_t launch_itb(const DecodeArgs& a, hipStream_t s) {
    constexpr int n_gu = (F + GuShape<D>::RPB - 1) / GuShape<D>::RPB;
    constexpr int n_dn = D / DnShape<F>::ROWS;
    const int S = a.T * a.k + (a.sg ? a.T : 0);
    const size_t lds = dn_lds_bytes<F>(S);
    if (lds > 64 * 1024) {   // opt in to more than 64 KiB of LDS, once per device
        constexpr int kMaxDev = 64;
        static bool attr_set[kMaxDev] = {};
        int dev = 0;
        hipError_t err = hipGetDevice(&dev);
        if (err != hipSuccess) return err;
        if (dev >= kMaxDev || !attr_set[dev]) {
            err = hipFuncSetAttribute(
                reinterpret_cast<const void*>(&decode_down_kernel<FMT, D, F, ITB>),
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)kDecodeMaxLds);
            if (err != hipSuccess) return err;
            if (dev < kMaxDev) attr_set[dev] = true;
        }
    }
    if (!a.logits)
        decode_gateup_kernel<FMT, D, F, 0><<<S * n_gu, GU_WAVES * 64, 0, s>>>(a);
    else if (a.E <= 64 * 8)
        decode_gateup_kernel<FMT, D, F, 8><<<S * n_gu, GU_WAVES * 64, 0, s>>>(a);
    else
        decode_gateup_kernel<FMT, D, F, 16><<<S * n_gu, GU_WAVES * 64, 0, s>>>(a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    decode_down_kernel<FMT, D, F, ITB><<<n_dn, DN_THREADS, lds, s>>>(a);
    return hipGetLastError();
}

template <int FMT, int D, int F>
hipError_t launch_shape(const DecodeArgs& a, hipStream_t s) {
    using DS = DnShape<F>;
    const int S = a.T * a.k + (a.sg ? a.T : 0);
    if (S <= DS::SPLIT * DS::NG) return launch_itb<FMT, D, F, DS::ITB_SMALL>(a, s);
    return launch_itb<FMT, D, F, DS::ITB_LARGE>(a, s);
}

template <int FMT>
hipError_t launch_fmt(const DecodeArgs& a, int d, int F, hipStream_t s) {
#define MOE_DEC(DV, FV) \
    if (d == DV && F == FV) return launch_shape<FMT, DV, FV>(a, s);
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

DecodeWs decode_ws_layout(int T, int k, int d, int F) {
    (void)d;
    auto al = [](size_t n) { return (n + 255) & ~size_t(255); };
    const int S = T * k + T;   // room for the shared expert's rows
    DecodeWs w;
    size_t off = 0;
    w.h = off; off += al((size_t)S * F * 2);
    w.bytes = off;
    return w;
}

bool decode_fits(int T, int k, int F, bool shared) {
    const int S = T * k + (shared ? T : 0);
    // h rows and the y rows of one down block (at most 64 rows per block)
    return T * k <= 64 && (size_t)S * F * 2 + (size_t)S * (F / 32) * 4 + (size_t)S * 16 +
                              256 <= kDecodeMaxLds;
}

hipError_t launch_decode_ffn(const moe_experts& routed, const moe_experts* shared,
                             const uint16_t* x, int T, int k, const float* logits,
                             int32_t* ids, float* weights, const uint16_t* residual,
                             const float* z, uint16_t* out, void* ws, hipStream_t s) {
    const int d = routed.d_model, F = routed.d_ff;
    const DecodeWs L = decode_ws_layout(T, k, d, F);
    uint8_t* base = static_cast<uint8_t*>(ws);
    DecodeArgs a;
    a.rg = routed.w_gate; a.ru = routed.w_up; a.rd = routed.w_down;
    a.rsg = routed.s_gate; a.rsu = routed.s_up; a.rsd = routed.s_down;
    a.E = routed.n_experts;
    a.sg = shared ? shared->w_gate : nullptr;
    a.su = shared ? shared->w_up : nullptr;
    a.sd = shared ? shared->w_down : nullptr;
    a.ssg = shared ? shared->s_gate : nullptr;
    a.ssu = shared ? shared->s_up : nullptr;
    a.ssd = shared ? shared->s_down : nullptr;
    a.x = x; a.T = T; a.k = k; a.logits = logits; a.ids = ids; a.weights = weights;
    a.residual = residual; a.z = z; a.out = out;
    a.h = reinterpret_cast<uint16_t*>(base + L.h);
    a.err = device_error_flag();
    switch (routed.fmt) {
        case MOE_FMT_INT4_G32: return launch_fmt<MOE_FMT_INT4_G32>(a, d, F, s);
        case MOE_FMT_INT6_G32: return launch_fmt<MOE_FMT_INT6_G32>(a, d, F, s);
        case MOE_FMT_INT3_G32: return launch_fmt<MOE_FMT_INT3_G32>(a, d, F, s);
        case MOE_FMT_INT2_G32: return launch_fmt<MOE_FMT_INT2_G32>(a, d, F, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace moe
