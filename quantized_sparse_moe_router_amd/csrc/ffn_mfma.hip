// ffn_mfma.hip -- expert FFN for many tokens (prefill): grouped GEMM on gfx950 MFMA.
//
// Prefill pushes large batches of tokens through each expert [Strata 与
// Qwen3.8-Flash-Next (telli.sh), section GPU、RAM 和 SSD 各司其职], so per expert the FFN
// is a dense contraction: [M_e x d] x [d x 2F] (gate and up), SwiGLU, then
// [M_e x F] x [F x d] (down).  That is the one place the layer maps onto the matrix
// cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation.
//
// Work list: one entry per (expert, BM-row tile of that expert's pairs), built on the
// device from the offsets (no host round trip).  The grid covers the largest possible
// list; blocks past its end return at once.
//
// Block = 4 waves, one per SIMD, tile BM = 256 rows x BN = 256 output columns; wave w owns
// columns [64 w, 64 w + 64) for all 256 rows (8 x 2 MFMA blocks of 32 x 32, 256 fp32
// accumulators in AGPRs).  All waves share the tile's rows, so a partial tile (an
// expert's last rows) shrinks every wave's MFMA work alike.
//
// Data movement per k-step of 64:
//   - activations: global -> LDS directly (global_load_lds_dwordx4, no register round
//     trip), 256 rows x 128 bytes, XOR-swizzled 16-byte chunks so the MFMA operand reads
//     are free of bank conflicts;
//   - weight codes and fp16 scales: global -> LDS directly, into a region private to the
//     wave that uses them; each lane later reads back exactly the 16 (int4), 24 (int6),
//     12 (int3) or 8 (int2) bytes of the one 32-code group it dequantises;
//   - dequantisation happens in registers straight into the MFMA B operand (no LDS
//     round trip for bf16 weights);
//   - the bf16 output tile is staged through LDS so global stores are full rows.  The MFMA k order inside a step is permuted so that
//     lane half h of every operand covers the 32-code group h: codes and scales of one
//     group serve four MFMA sub-steps.
// Three LDS stages: loads for step ks + 2 are issued at the start of step ks, so each
// has about two k-steps to land.  Loads are counted by hand (s_waitcnt vmcnt) because the
// compiler does not track LDS written by these loads.
#include "mfma_common.h"

#include <algorithm>
#include <type_traits>

namespace moe {
namespace {

constexpr int BM = kMfmaTileRows;   // rows (pairs) per tile
constexpr int BN = 256;          // output columns per tile (gate/up: 128 f x 2)
constexpr int NW = 4;            // waves per block
constexpr int NT = 64 * NW;      // threads per block
constexpr int TN = BN / NW;      // columns per wave
constexpr int NI = TN / 32;      // 32-column MFMA blocks per wave (2)
constexpr int MI = BM / 32;      // 32-row MFMA blocks per tile (8)
constexpr int BK = 64;           // reduction step
constexpr int kStages = 3;       // LDS pipeline stages
constexpr int kXcds = 8;         // MI355X: 8 XCDs of 32 CUs, each with its own L2

// entries of the work list: at most ceil(rows / BM) + E tiles, rounded up to whole XCD groups
// so that every block of the grid can read its entry before checking the count
size_t tile_capacity(int64_t rows, int E) {
    const size_t n = (size_t)((rows + BM - 1) / BM + E);
    return (n + kXcds - 1) / kXcds * kXcds;
}

// -------------------------------------------------------------- work list
__global__ void __launch_bounds__(1024) build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                           int E, int4* __restrict__ tiles,
                                                           int* __restrict__ count) {
    __shared__ int part[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int b = 0, n = 0, cnt = 0;
    if (tid < E) {
        b = offsets[tid];
        n = offsets[tid + 1] - b;
        cnt = (n + BM - 1) / BM;
    }
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) part[wv] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < 16; ++i) {
            const int v = part[i];
            part[i] = run;
            run += v;
        }
        *count = run;
    }
    __syncthreads();
    const int start = incl - cnt + part[wv];
    for (int i = 0; i < cnt; ++i) tiles[start + i] = make_int4(tid, b + i * BM, b + n, 0);
}

enum { kGateUp = 0, kDown = 1 };

// LDS bytes of one pipeline stage
template <int FMT>
struct StageLayout {
    // bytes per group; loads per group (int4 one dwordx4, int6 two dwordx3, int3 one
    // dwordx3, int2 two dword) and the LDS bytes one load gives each lane
    static constexpr int GB = FMT == MOE_FMT_INT4_G32 ? 16 : FMT == MOE_FMT_INT6_G32 ? 24
                              : FMT == MOE_FMT_INT3_G32 ? 12 : 8;
    static constexpr int DMA_B = (FMT == MOE_FMT_INT6_G32 || FMT == MOE_FMT_INT2_G32) ? 2 : 1;
    static constexpr int DMA_STRIDE = FMT == MOE_FMT_INT2_G32 ? 4 : 16;
    static constexpr int A = BM * BK * 2;                             // activations
    static constexpr int B_WJ = DMA_B * 64 * DMA_STRIDE;              // codes of (wave, j)
    static constexpr int B = NW * NI * B_WJ;
    static constexpr int S_WJ = 64 * 4;                               // scales of (wave, j)
    static constexpr int S = NW * NI * S_WJ;
    static constexpr int BYTES = A + B + S;
};
template <int FMT>
constexpr int kGemmLds = kStages * StageLayout<FMT>::BYTES;
static_assert(kStages * StageLayout<MOE_FMT_INT6_G32>::BYTES <= 160 * 1024, "LDS");

// -------------------------------------------------------------- grouped GEMM
//   kGateUp: K = d; block column tile ny covers f in [128 ny, 128 ny + 128); wave w's
//            MFMA block j = 0 holds the gate rows, j = 1 the up rows of the same 32 f's,
//            so a lane holds g and u of the same (row, f); epilogue h = silu(g) * u ->
//            bf16 [rows][F].
//   kDown  : K = F; wave w's blocks hold W_down rows 256 ny + 64 w + 32 j + (0..31);
//            epilogue y -> bf16 [rows][d].
// dense (sorted_pairs == nullptr): one expert, rows are tokens 0..T-1.
// MB = 32-row MFMA blocks of the tile that hold rows (1..8); rows past the tile's end
// repeat its last row (loads stay in bounds) and are never stored.
struct GemmArgs {
    const uint8_t* wa;
    const uint16_t* sa;
    const uint8_t* wb;
    const uint16_t* sb;
    const uint16_t* act;
    int K, n_out, topk;
    const int32_t* sorted_pairs;
    uint16_t* out;
};

template <int FMT, int MODE, int MB>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int e, int m0, int m1, int ny,
                                          uint8_t* smem) {
    using L = StageLayout<FMT>;
    constexpr int GB = L::GB;
    constexpr int NG = MB + NI * L::DMA_B + NI;   // global loads per wave per k-step
    static_assert(NG <= 16, "one load every third slot of sub-steps 0..2");
    constexpr int kIssuedBySs2 = NG < 11 ? NG : 11;   // loads issued in slots 0..31
    const int K = g.K;
    const int nk = K / BK;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;                  // lane half: 32-code group h of the k-step
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

    // ---- activation rows this lane loads: row r = 32 i + 8 wave + lane / 8 of the tile
    // into LDS chunk position lane % 8 of that row.  Position p of row r holds logical
    // 16-byte chunk p ^ ((r / 2) % 8): the 16 rows an MFMA operand read touches per LDS
    // cycle then cover all 64 banks.
    // Addresses: a wave-uniform base per source (SGPRs, advanced per k-step) plus a per-lane
    // 32-bit byte offset (activations: at most T * K * 2 bytes; weights: within one
    // expert's rows).
    const uint16_t* a_base = uniform_ptr(g.act);
    uint32_t a_off[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int r = 32 * i + 8 * wave + (lane >> 3);
        const int pos = min(m0 + r, m1 - 1);
        uint32_t arow;
        if (MODE == kGateUp && g.sorted_pairs)
            arow = (uint32_t)(g.sorted_pairs[pos] / g.topk);
        else
            arow = (uint32_t)pos;
        a_off[i] = (arow * (uint32_t)K + 8u * (uint32_t)((lane & 7) ^ ((r >> 1) & 7))) * 2u;
    }
    // ---- weight rows of this lane's two MFMA columns (column lane % 32 of block j): the
    // wave's first row of block j as the base, lane % 32 rows further as the offset
    const uint8_t* b_base[NI];
    const uint16_t* s_base[NI];
    const uint32_t row_bytes = (uint32_t)(K / 32 * GB);
    const uint32_t b_off = (uint32_t)(lane & 31) * row_bytes + (uint32_t)(h * GB);
    const uint32_t s_off = ((uint32_t)(lane & 31) * (uint32_t)(K / 32) + (uint32_t)h) * 2u;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        size_t grow0;
        const uint8_t* wm;
        const uint16_t* sm;
        if (MODE == kGateUp) {
            grow0 = (size_t)e * g.n_out + ny * (BN / 2) + 32 * wave;
            wm = j == 0 ? g.wa : g.wb;
            sm = j == 0 ? g.sa : g.sb;
        } else {
            grow0 = (size_t)e * g.n_out + ny * BN + TN * wave + 32 * j;
            wm = g.wa;
            sm = g.sa;
        }
        b_base[j] = uniform_ptr(wm + grow0 * row_bytes);
        s_base[j] = uniform_ptr(sm + grow0 * (size_t)(K / 32));
    }

    f32x16_t acc[MB][NI];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // stage byte offsets (relative to smem / absolute LDS addresses)
    const uint32_t a_rd = (uint32_t)(lane & 31) * 128;   // + 4096 i + swizzled chunk
    const uint32_t own_b = (uint32_t)(wave * NI) * L::B_WJ + lane * L::DMA_STRIDE;
    const uint32_t own_s = (uint32_t)(wave * NI) * L::S_WJ + lane * 4;

    // load number q (0..NG-1) of k-step `step` into stage st
    auto issue = [&](int q, int step, int st) __attribute__((always_inline)) {
        const int kk = step;
        const uint32_t base = lds0 + st * L::BYTES;
        if (q < MB) {
            dma16s(a_base + kk * BK, a_off[q], base + (32 * q + 8 * wave) * 128);
        } else if (q < MB + NI * L::DMA_B) {
            const int j = (q - MB) / L::DMA_B, part = (q - MB) % L::DMA_B;
            const uint8_t* src = b_base[j] + kk * 2 * GB;
            const uint32_t dst = base + L::A + (wave * NI + j) * L::B_WJ;
            if constexpr (FMT == MOE_FMT_INT4_G32)
                dma16s(src, b_off, dst);
            else if constexpr (FMT == MOE_FMT_INT6_G32)
                dma12s(src, b_off + 12 * part, dst + 1024 * part);
            else if constexpr (FMT == MOE_FMT_INT3_G32)
                dma12s(src, b_off, dst);
            else
                dma4s(src, b_off + 4 * part, dst + 256 * part);
        } else {
            const int j = q - MB - NI * L::DMA_B;
            dma2s(s_base[j] + kk * 2, s_off, base + L::A + L::B + (wave * NI + j) * L::S_WJ);
        }
    };
    // this lane's group codes and scale of MFMA column block j, from stage st
    auto read_codes = [&](int st, int j, GroupCodes<FMT>& c, float& s)
        __attribute__((always_inline)) {
        const uint8_t* base = smem + st * L::BYTES;
        const uint8_t* p = base + L::A + own_b + j * L::B_WJ;
        if constexpr (FMT == MOE_FMT_INT4_G32) {
            c.a = *reinterpret_cast<const u32x4_t*>(p);
        } else if constexpr (FMT == MOE_FMT_INT6_G32) {
            const u32x4_t q0 = *reinterpret_cast<const u32x4_t*>(p);          // bytes 0..11
            const u32x4_t q1 = *reinterpret_cast<const u32x4_t*>(p + 1024);   // bytes 12..23
            c.a = u32x4_t{q0.x, q0.y, q0.z, q1.x};
            c.b = u32x2_t{q1.y, q1.z};
        } else if constexpr (FMT == MOE_FMT_INT3_G32) {
            const u32x4_t q0 = *reinterpret_cast<const u32x4_t*>(p);          // bytes 0..11
            c.a = u32x4_t{q0.x, q0.y, q0.z, 0u};
        } else {
            c.a = u32x4_t{*reinterpret_cast<const uint32_t*>(p),               // bytes 0..3
                          *reinterpret_cast<const uint32_t*>(p + 256), 0u, 0u};   // 4..7
        }
        s = f16_to_f32(*reinterpret_cast<const uint16_t*>(base + L::A + L::B + own_s +
                                                          j * L::S_WJ));
    };
    // A operand of MFMA row block i, sub-step ss: logical chunk 4 h + ss of row 32 i +
    // lane % 32 (k = 32 h + 8 ss .. + 7 of the step)
    auto read_a = [&](int st, int i, int ss) __attribute__((always_inline)) {
        const uint32_t chunk = (uint32_t)((4 * h + ss) ^ ((lane >> 1) & 7));
        return *reinterpret_cast<const bf16x8_t*>(smem + st * L::BYTES + a_rd + 4096 * i +
                                                  (chunk << 4));
    };

    // codes/scales of the current k-step (codes, zc = -zero_point * scale) and of the next
    GroupCodes<FMT> codes[NI], codes_n[NI];
    float scale[NI], scale_n[NI];
    bf16x8_t fa[2][MB], fb[2][NI];
    uint32_t lo = 0, hi = 0;
    float e0 = 0.0f, e1 = 0.0f;
    constexpr float kZero = kZeroPoint<FMT>;

    // Half H of B operand pair b (codes 8 ss + 2b, +1) of column block j for sub-step ss,
    // into fb[F][j]: half 0 converts the two codes to float, half 1 scales and packs them.
    auto dequant_half = [&](const GroupCodes<FMT>* cd, const float* sc, int F, int j, int ss,
                            int b, int half) __attribute__((always_inline)) {
        if (half == 0) {
            if (b == 0) chunk_codes<FMT>(cd[j], ss, lo, hi);
            e0 = (float)((lo >> (8 * b)) & 0xffu);
            e1 = (float)((hi >> (8 * b)) & 0xffu);
        } else {
            const float s = sc[j], zc = -kZero * s;
            u32x4_t v = __builtin_bit_cast(u32x4_t, fb[F][j]);
            v[b] = pack_bf16(__builtin_fmaf(e0, s, zc), __builtin_fmaf(e1, s, zc));
            fb[F][j] = __builtin_bit_cast(bf16x8_t, v);
        }
    };
    // The product is formed transposed, D^T = B^T A^T (weights as the first operand): the
    // two operand layouts are mirror images, and the transposed result leaves each lane
    // one row of the tile with runs of 4 adjacent output columns.
    auto mfma = [&](int F, int t) __attribute__((always_inline)) {
        const int i = t / NI, j = t % NI;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[F][j], fa[F][i], acc[i][j],
                                                            0, 0, 0);
    };

    // ---- prologue: steps 0 and 1 in flight, step 0's operands of sub-step 0 ready
#pragma unroll
    for (int q = 0; q < NG; ++q) issue(q, 0, 0);
#pragma unroll
    for (int q = 0; q < NG; ++q) issue(q, 1, 1);
    MOE_WAIT_VMCNT(NG);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NI; ++j) read_codes(0, j, codes[j], scale[j]);
#pragma unroll
    for (int i = 0; i < MB; ++i) fa[0][i] = read_a(0, i, 0);
#pragma unroll
    for (int p = 0; p < 8 * NI; ++p) dequant_half(codes, scale, 0, p / 8, 0, (p / 2) % 4, p % 2);

    // ---- main loop.  One k-step is an explicit issue order of 4 x 16 slots.  A slot holds
    // at most one MFMA and after it about four issue cycles of other work: a global load of
    // step ks + 2, an A operand read, or half of one packed bf16 B pair (2-3 VALU ops) for
    // the next sub-step.  A 32x32x16 MFMA leaves its wave free to issue for about 16 of its
    // 32 cycles, so this keeps the matrix pipe fed; sched_barrier keeps the compiler from
    // regrouping the slots.
    // One k-step; PF: the loads of step ks + 2 are issued (every step but the last two,
    // which wait for everything outstanding instead).
    int st = 0;                                   // stage of step ks
    auto kstep = [&](int ks, auto pf) __attribute__((always_inline)) {
        constexpr bool PF = decltype(pf)::value;
        const int st1 = st == kStages - 1 ? 0 : st + 1;
        const int st2 = st1 == kStages - 1 ? 0 : st1 + 1;
#pragma unroll
        for (int u = 0; u < 48; ++u) {            // sub-steps 0..2
            const int ss = u / 16, t = u % 16, F = ss & 1;
            if (t < MB * NI) mfma(F, t);
            // the loads of step ks + 2 are spread over the first 48 slots, one every third:
            // issued in one burst they queue in the address path and the waves fall out
            // of step, which the barrier then pays for
            if (PF && u % 3 == 0 && u / 3 < NG) issue(u / 3, ks + 2, st2);
            if (t % 2 == 0 && t / 2 < MB) fa[F ^ 1][t / 2] = read_a(st, t / 2, ss + 1);
            dequant_half(codes, scale, F ^ 1, t / 8, ss + 1, (t / 2) % 4, t % 2);
            // this wave's loads of step ks + 1 are done (the loads of step ks + 2 issued so
            // far, slots 0, 3, .., 30, may still be in flight); its codes are private to the
            // wave
            if (ss == 2 && t == 0) {
                if constexpr (PF) MOE_WAIT_VMCNT(kIssuedBySs2);
                else MOE_WAIT_VMCNT(0);
            }
            if (ss == 2 && (t == 1 || t == 3)) read_codes(st1, t / 2, codes_n[t / 2], scale_n[t / 2]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // every wave's loads of step ks + 1 have landed once all pass the barrier; stage st
        // is not read after it
        if constexpr (PF) MOE_WAIT_VMCNT_LDS(NG);
        else MOE_WAIT_VMCNT_LDS(0);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 16; ++t) {            // sub-step 3, and step ks + 1's sub-step 0
            if (t < MB * NI) mfma(1, t);
            if (t % 2 == 0 && t / 2 < MB) fa[0][t / 2] = read_a(st1, t / 2, 0);
            dequant_half(codes_n, scale_n, 0, t / 8, 0, (t / 2) % 4, t % 2);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            codes[j] = codes_n[j];
            scale[j] = scale_n[j];
        }
        st = st1;
    };
    for (int ks = 0; ks + 2 < nk; ++ks) kstep(ks, std::true_type{});
    for (int ks = nk - 2; ks < nk; ++ks) kstep(ks, std::false_type{});
    // nothing is in flight; after the barrier no wave reads the stages and LDS holds the
    // output tile
    __syncthreads();

    // ---- epilogue: accumulator r of lane l in block (i, j) is tile row 32 i + l % 32 and
    // column 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 of the wave's 64 columns.  The bf16
    // tile goes through LDS (row pitch padded against bank conflicts) so that global
    // stores are whole 16-byte chunks of contiguous rows.
    constexpr int OCOLS = MODE == kGateUp ? BN / 2 : BN;   // output columns of the block
    constexpr int OP = OCOLS * 2 + 16;                      // LDS row pitch in bytes
    constexpr int RP = MODE == kGateUp ? BM : BM / 2;       // rows per pass
    static_assert(RP * OP <= kStages * L::BYTES, "output tile fits in LDS");
    const int col0 = ny * OCOLS;
#pragma unroll
    for (int pass = 0; pass < BM / RP; ++pass) {
        if (32 * MB <= pass * RP) break;                    // no rows in this pass
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            if ((32 * i) / RP != pass) continue;
            uint8_t* lrow = smem + (32 * i - pass * RP + (lane & 31)) * OP;
            if constexpr (MODE == kGateUp) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    float hv[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float gt = acc[i][0][4 * rb + c], u = acc[i][1][4 * rb + c];
                        // silu(g) * u = g * u / (1 + 2^(-g log2 e))
                        const float den =
                            1.0f + __builtin_amdgcn_exp2f(-gt * 1.4426950408889634f);
                        hv[c] = gt * u * __builtin_amdgcn_rcpf(den);
                    }
                    *reinterpret_cast<u32x2_t*>(lrow + 2 * (32 * wave + 8 * rb + 4 * h)) =
                        u32x2_t{pack_bf16(hv[0], hv[1]), pack_bf16(hv[2], hv[3])};
                }
            } else {
#pragma unroll
                for (int j = 0; j < NI; ++j)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb)
                        *reinterpret_cast<u32x2_t*>(lrow +
                                                    2 * (TN * wave + 32 * j + 8 * rb + 4 * h)) =
                            u32x2_t{pack_bf16(acc[i][j][4 * rb], acc[i][j][4 * rb + 1]),
                                    pack_bf16(acc[i][j][4 * rb + 2], acc[i][j][4 * rb + 3])};
            }
        }
        __syncthreads();
        constexpr int CPR = OCOLS / 8;                      // 16-byte chunks per row
#pragma unroll
        for (int n = 0; n < RP * CPR / NT; ++n) {
            const int qd = tid + NT * n, r = qd / CPR, c = qd % CPR;
            const int grow = m0 + pass * RP + r;
            if (r < 32 * MB - pass * RP && grow < m1) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + r * OP + 16 * c);
                u32x4_t* dst =
                    reinterpret_cast<u32x4_t*>(g.out + (size_t)grow * g.n_out + col0 + 8 * c);
                // y (down) is read once, by the combine after this launch: stored
                // non-temporal so that it does not displace the expert weights that the
                // next tiles of the same expert read again (8192 tokens: 2.3 % off the
                // layer); h (gate/up) is read straight back by the down GEMM
                if constexpr (MODE == kDown)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
        }
        if (pass + 1 < BM / RP) __syncthreads();
    }
}

template <int FMT, int MODE>
__global__ void __launch_bounds__(NT, 1) grouped_gemm_kernel(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const uint16_t* __restrict__ act, int K, int n_out, int topk,
    const int32_t* __restrict__ sorted_pairs, const int4* __restrict__ tiles,
    const int* __restrict__ tile_count, int T_dense, int n_ny, uint16_t* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // XCD-aware order: workgroups go round-robin to the 8 XCDs, so XCD x runs blocks
    // x, x + 8, x + 16, ...; give each XCD whole row tiles, all n_ny column blocks of a tile
    // back to back, so the tile's activation rows are fetched into that XCD's L2 once.
    const int xcd = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
    const int tile = (q / n_ny) * kXcds + xcd, ny = q % n_ny;
    int e, m0, m1;
    if (tiles) {
        // the entry (in bounds for every block of the grid) and the count load together
        const int4 t = tiles[tile];
        if (tile >= *tile_count) return;
        e = t.x; m0 = t.y; m1 = t.z;
    } else {
        e = 0;
        m0 = tile * BM;
        if (m0 >= T_dense) return;
        m1 = T_dense;
    }
    const GemmArgs g{wa, sa, wb, sb, act, K, n_out, topk, sorted_pairs, out};
    const int mb = min(MI, (m1 - m0 + 31) / 32);   // >= 1, block-uniform
    static_assert(MI == 8, "row-block dispatch below assumes 8 blocks per tile");
    switch (mb) {
        case 8: gemm_tile<FMT, MODE, 8>(g, e, m0, m1, ny, smem); break;
        case 7: gemm_tile<FMT, MODE, 7>(g, e, m0, m1, ny, smem); break;
        case 6: gemm_tile<FMT, MODE, 6>(g, e, m0, m1, ny, smem); break;
        case 5: gemm_tile<FMT, MODE, 5>(g, e, m0, m1, ny, smem); break;
        case 4: gemm_tile<FMT, MODE, 4>(g, e, m0, m1, ny, smem); break;
        case 3: gemm_tile<FMT, MODE, 3>(g, e, m0, m1, ny, smem); break;
        case 2: gemm_tile<FMT, MODE, 2>(g, e, m0, m1, ny, smem); break;
        default: gemm_tile<FMT, MODE, 1>(g, e, m0, m1, ny, smem); break;
    }
}

// grouped: tiles / count hold the work list (capacity tile_cap, a multiple of kXcds; built
// here from offsets when offsets is given); dense: tiles == nullptr
template <int FMT>
hipError_t launch_gemm_fmt(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           uint16_t* h, const int4* tiles, const int* count, size_t tile_cap,
                           hipStream_t s) {
    const int d = ex.d_model, F = ex.d_ff, E = ex.n_experts;
    int gx;
    if (tiles) {
        if (offsets)
            build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, const_cast<int4*>(tiles),
                                                  const_cast<int*>(count));
        gx = (int)tile_cap;
    } else {
        gx = (T + BM - 1) / BM;
    }
    // opt in to more than 64 KiB of LDS, once per device
    constexpr int kMaxDev = 64;
    static bool attr_set[kMaxDev] = {};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev >= kMaxDev || !attr_set[dev]) {
        err = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&grouped_gemm_kernel<FMT, kGateUp>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds<FMT>);
        if (err != hipSuccess) return err;
        err = hipFuncSetAttribute(
            reinterpret_cast<const void*>(&grouped_gemm_kernel<FMT, kDown>),
            hipFuncAttributeMaxDynamicSharedMemorySize, kGemmLds<FMT>);
        if (err != hipSuccess) return err;
        if (dev < kMaxDev) attr_set[dev] = true;
    }
    const int gx8 = (gx + kXcds - 1) / kXcds * kXcds;   // whole tiles per XCD
    const int ny_gu = F / (BN / 2), ny_dn = d / BN;
    grouped_gemm_kernel<FMT, kGateUp><<<gx8 * ny_gu, NT, kGemmLds<FMT>, s>>>(
        ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x, d, F, k, sorted_pairs, tiles, count, T, ny_gu,
        h);
    grouped_gemm_kernel<FMT, kDown><<<gx8 * ny_dn, NT, kGemmLds<FMT>, s>>>(
        ex.w_down, ex.s_down, nullptr, nullptr, h, F, d, k, sorted_pairs, tiles, count, T, ny_dn,
        y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(const moe_experts& ex, const uint16_t* x, int T, int k,
                      const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                      void* ws, hipStream_t s) {
    const int E = ex.n_experts, F = ex.d_ff;
    const bool grouped = offsets != nullptr;
    const int64_t rows = grouped ? (int64_t)T * k : (int64_t)T;
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(base);
    size_t off = ((size_t)rows * F * 2 + 255) & ~size_t(255);
    int4* tiles = nullptr;
    int* count = nullptr;
    if (grouped) {
        tiles = reinterpret_cast<int4*>(base + off);
        off += (tile_capacity(rows, E) * sizeof(int4) + 255) & ~size_t(255);
        count = reinterpret_cast<int*>(base + off);
    }
    return launch_gemm_fmt<FMT>(ex, x, T, k, offsets, sorted_pairs, y, h, tiles, count,
                                grouped ? tile_capacity(rows, E) : 0, s);
}

}  // namespace

// tiles of the experts with at least min_rows >= 1 of rows pairs: at most ceil(rows / BM)
// plus one per such expert, rounded up to whole XCD groups
size_t ffn_mfma_hot_tile_capacity(int64_t rows, int E, int min_rows) {
    const int64_t experts = std::min<int64_t>(E, rows / std::max(min_rows, 1));
    const size_t n = (size_t)((rows + BM - 1) / BM + experts);
    return (n + kXcds - 1) / kXcds * kXcds;
}

hipError_t launch_ffn_mfma_hot(const moe_experts& ex, const uint16_t* x, int T, int k,
                               const int32_t* sorted_pairs, uint16_t* y, uint16_t* h,
                               const int4* tiles, const int* count, size_t tile_cap,
                               hipStream_t s) {
    switch (ex.fmt) {
#define MOE_HOT(F)                                                                        \
        case F:                                                                           \
            return launch_gemm_fmt<F>(ex, x, T, k, nullptr, sorted_pairs, y, h, tiles,     \
                                      count, tile_cap, s);
        MOE_HOT(MOE_FMT_INT4_G32)
        MOE_HOT(MOE_FMT_INT6_G32)
        MOE_HOT(MOE_FMT_INT3_G32)
        MOE_HOT(MOE_FMT_INT2_G32)
#undef MOE_HOT
        default:
            return hipErrorNotSupported;
    }
}

size_t ffn_mfma_ws_bytes(int64_t rows, int E, int F) {
    size_t n = ((size_t)rows * F * 2 + 255) & ~size_t(255);
    n += (tile_capacity(rows, E) * sizeof(int4) + 255) & ~size_t(255);
    n += 256;
    return n;
}

hipError_t launch_ffn_mfma(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           void* ws, hipStream_t s) {
    switch (ex.fmt) {
        case MOE_FMT_INT4_G32:
            return launch_fmt<MOE_FMT_INT4_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
        case MOE_FMT_INT6_G32:
            return launch_fmt<MOE_FMT_INT6_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
        case MOE_FMT_INT3_G32:
            return launch_fmt<MOE_FMT_INT3_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
        case MOE_FMT_INT2_G32:
            return launch_fmt<MOE_FMT_INT2_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
        default:
            return hipErrorNotSupported;
    }
}

}  // namespace moe
