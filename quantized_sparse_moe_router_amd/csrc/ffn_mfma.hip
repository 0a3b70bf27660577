// ffn_mfma.hip -- expert FFN for many tokens (prefill): grouped GEMM on gfx950 MFMA.
//
// Prefill pushes large batches of tokens through each expert [Strata 与
// Qwen3.8-Flash-Next (telli.sh), section GPU、RAM 和 SSD 各司其职], so per expert the FFN
// is a dense contraction: [M_e x d] x [d x 2F] (gate and up), SwiGLU, then
// [M_e x F] x [F x d] (down).  That is the one place the layer maps onto the matrix
// cores.  Weight tiles are dequantised to bf16 once per block and k-step into LDS;
// activation rows are gathered by the sorted pair list into LDS; both feed
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// Work list: one entry per (expert, 128-row tile of that expert's pairs), built on the
// device from the offsets (no host round trip).  The grid covers the largest possible
// list; blocks past its end return at once.
#include "moe_common.h"

namespace moe {
namespace {

constexpr int BM = 128;          // rows (pairs) per tile
constexpr int BN = 128;          // output columns per tile (gate/up: 64 f x 2)
constexpr int BK = 64;           // reduction step
constexpr int LDP = BK + 8;      // LDS row pitch in bf16 (padding against bank conflicts)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct TileList {
    int4* tiles;     // {expert, row begin, row end (segment end), 0}
    int* count;
};

size_t tile_capacity(int64_t rows, int E) { return (size_t)((rows + BM - 1) / BM + E); }

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

// -------------------------------------------------------------- dequantisation
// 32 codes of one group (one row, one scale) -> 32 bf16 (16 packed pairs).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2_t p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ void dequant_int4(const uint4 w, float s, uint32_t* out) {
    const float c = -8.0f * s;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t lo = wd[q] & 0x0f0f0f0fu, hi = (wd[q] >> 4) & 0x0f0f0f0fu;
        // keep the nibbles byte-aligned so each converts with one byte-to-float op
        asm volatile("" : "+v"(lo), "+v"(hi));
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float e0 = (float)((lo >> (8 * b)) & 0xffu);
            const float e1 = (float)((hi >> (8 * b)) & 0xffu);
            out[4 * q + b] = pack_bf16(__builtin_fmaf(e0, s, c), __builtin_fmaf(e1, s, c));
        }
    }
}

__device__ __forceinline__ void dequant_int6(const uint32_t* w6, float s, uint32_t* out) {
    const float c = -32.0f * s;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint64_t lo64 = (uint64_t)w6[3 * half] | ((uint64_t)w6[3 * half + 1] << 32);
        const uint64_t hi32 = w6[3 * half + 2];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            float v[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int bit = 6 * (2 * p + t);
                uint32_t u;
                if (bit + 6 <= 64)
                    u = (uint32_t)(lo64 >> bit);
                else if (bit >= 64)
                    u = (uint32_t)(hi32 >> (bit - 64));
                else
                    u = (uint32_t)(lo64 >> bit) | (uint32_t)(hi32 << (64 - bit));
                v[t] = __builtin_fmaf((float)(u & 63u), s, c);
            }
            out[8 * half + p] = pack_bf16(v[0], v[1]);
        }
    }
}

template <int FMT>
struct GroupLoad {
    uint4 a;
    uint2 b;   // int6 tail
};

template <int FMT>
__device__ __forceinline__ void load_group(const uint8_t* p, GroupLoad<FMT>& g) {
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
__device__ __forceinline__ void dequant_group(const GroupLoad<FMT>& g, float s, uint32_t* out) {
    if constexpr (FMT == MOE_FMT_INT4_G32) {
        dequant_int4(g.a, s, out);
    } else {
        const uint32_t w6[6] = {g.a.x, g.a.y, g.a.z, g.a.w, g.b.x, g.b.y};
        dequant_int6(w6, s, out);
    }
}

enum { kGateUp = 0, kDown = 1 };

// -------------------------------------------------------------- grouped GEMM
// 256 threads = 4 waves in a 2 x 2 layout, each wave a 64 x 64 sub-tile made of 4 x 4
// MFMA 16x16x32 blocks.
//   kGateUp: K = d, B rows = 64 gate rows and the 64 up rows of the same f; the LDS B
//            tile is ordered [gate f0..+31 | up f0..+31 | gate f0+32..+63 | up f0+32..+63]
//            so each lane holds the gate and up outputs of the same (row, f); epilogue
//            h = silu(g) * u -> bf16 [rows][F].
//   kDown  : K = F, B rows = 128 rows of W_down; epilogue y -> bf16 [rows][d].
// dense (sorted_pairs == nullptr): one expert, rows are tokens 0..T-1.
template <int FMT, int MODE>
__global__ void __launch_bounds__(256) grouped_gemm_kernel(
    const uint8_t* __restrict__ wa, const uint16_t* __restrict__ sa,
    const uint8_t* __restrict__ wb, const uint16_t* __restrict__ sb,
    const uint16_t* __restrict__ act, int K, int n_out, int topk,
    const int32_t* __restrict__ sorted_pairs, const int4* __restrict__ tiles,
    const int* __restrict__ tile_count, int T_dense, uint16_t* __restrict__ out) {
    constexpr int GB = (FMT == MOE_FMT_INT4_G32) ? 16 : 24;   // bytes per 32-code group
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDP];

    // ---- which tile
    int e, m0, m1;
    if (tiles) {
        if ((int)blockIdx.x >= *tile_count) return;
        const int4 t = tiles[blockIdx.x];
        e = t.x; m0 = t.y; m1 = t.z;
    } else {
        e = 0;
        m0 = blockIdx.x * BM;
        if (m0 >= T_dense) return;
        m1 = T_dense;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- A rows this thread stages: rows r = tid/8 + 32 i, 16-byte column tid%8
    const int a_col = (tid & 7) * 8;
    const uint16_t* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int pos = m0 + r;
        if (pos < m1) {
            size_t arow;
            if (MODE == kGateUp && sorted_pairs)
                arow = (size_t)(sorted_pairs[pos] / topk);
            else
                arow = (size_t)pos;
            a_src[i] = act + arow * K + a_col;
        } else {
            a_src[i] = nullptr;
        }
    }
    // ---- B row this thread dequantises: LDS row nn = tid/2, group half = tid%2
    const int nn = tid >> 1, bhalf = tid & 1;
    const uint8_t* b_w;
    const uint16_t* b_s;
    {
        const size_t rows_per_expert = (MODE == kGateUp) ? (size_t)(n_out) : (size_t)n_out;
        int mat = 0, r;
        if (MODE == kGateUp) {
            const int f0 = blockIdx.y * (BN / 2);
            const int blk = nn >> 5;                  // 0..3
            mat = blk & 1;                            // 0 gate, 1 up
            r = f0 + 32 * (blk >> 1) + (nn & 31);
        } else {
            r = blockIdx.y * BN + nn;
        }
        const size_t grow = (size_t)e * rows_per_expert + r;
        const size_t row_bytes = (size_t)K / 32 * GB;
        b_w = ((mat == 0) ? wa : wb) + grow * row_bytes + (size_t)bhalf * GB;
        b_s = ((mat == 0) ? sa : sb) + grow * (K / 32) + bhalf;
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 a_reg[4];
    GroupLoad<FMT> b_reg;
    float b_scale;

    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a_reg[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0)
                                : make_uint4(0u, 0u, 0u, 0u);
        load_group<FMT>(b_w + (size_t)(k0 / 32) * GB, b_reg);
        b_scale = f16_to_f32(b_s[k0 / 32]);
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(&As[buf][(tid >> 3) + 32 * i][a_col]) = a_reg[i];
        uint32_t deq[16];
        dequant_group<FMT>(b_reg, b_scale, deq);
        uint4* dst = reinterpret_cast<uint4*>(&Bs[buf][nn][32 * bhalf]);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            dst[v] = make_uint4(deq[4 * v], deq[4 * v + 1], deq[4 * v + 2], deq[4 * v + 3]);
    };

    const int nk = K / BK;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) load_global((ks + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8_t a[4], b[4];
            const int kc = kk + 8 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                a[i] = *reinterpret_cast<const bf16x8_t*>(
                    &As[buf][wm * 64 + i * 16 + (lane & 15)][kc]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = *reinterpret_cast<const bf16x8_t*>(
                    &Bs[buf][wn * 64 + j * 16 + (lane & 15)][kc]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (ks + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    const int col = lane & 15, rq = 4 * (lane >> 4);
    if constexpr (MODE == kGateUp) {
        const int F = n_out;
        const int fbase = blockIdx.y * (BN / 2) + wn * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm * 64 + i * 16 + rq + r;
                    if (row < m1) {
                        const float g = acc[i][j][r], u = acc[i][j + 2][r];
                        const float h = g / (1.0f + expf(-g)) * u;
                        out[(size_t)row * F + fbase + j * 16 + col] = (uint16_t)f32_to_bf16(h);
                    }
                }
    } else {
        const int nbase = blockIdx.y * BN + wn * 64;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = m0 + wm * 64 + i * 16 + rq + r;
                    if (row < m1)
                        out[(size_t)row * n_out + nbase + j * 16 + col] =
                            (uint16_t)f32_to_bf16(acc[i][j][r]);
                }
    }
}

template <int FMT>
hipError_t launch_fmt(const moe_experts& ex, const uint16_t* x, int T, int k,
                      const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                      void* ws, hipStream_t s) {
    const int d = ex.d_model, F = ex.d_ff, E = ex.n_experts;
    const bool grouped = offsets != nullptr;
    const int64_t rows = grouped ? (int64_t)T * k : (int64_t)T;
    uint8_t* base = static_cast<uint8_t*>(ws);
    uint16_t* h = reinterpret_cast<uint16_t*>(base);
    size_t off = ((size_t)rows * F * 2 + 255) & ~size_t(255);
    int4* tiles = nullptr;
    int* count = nullptr;
    int gx;
    if (grouped) {
        tiles = reinterpret_cast<int4*>(base + off);
        off += (tile_capacity(rows, E) * sizeof(int4) + 255) & ~size_t(255);
        count = reinterpret_cast<int*>(base + off);
        build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, tiles, count);
        gx = (int)tile_capacity(rows, E);
    } else {
        gx = (T + BM - 1) / BM;
    }
    grouped_gemm_kernel<FMT, kGateUp><<<dim3(gx, F / (BN / 2)), 256, 0, s>>>(
        ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, x, d, F, k, sorted_pairs, tiles, count, T, h);
    grouped_gemm_kernel<FMT, kDown><<<dim3(gx, d / BN), 256, 0, s>>>(
        ex.w_down, ex.s_down, nullptr, nullptr, h, F, d, k, sorted_pairs, tiles, count, T, y);
    return hipGetLastError();
}

}  // namespace

size_t ffn_mfma_ws_bytes(int64_t rows, int E, int F) {
    size_t n = ((size_t)rows * F * 2 + 255) & ~size_t(255);
    n += (tile_capacity(rows, E) * sizeof(int4) + 255) & ~size_t(255);
    n += 256;
    return n;
}

hipError_t launch_ffn_mfma(const moe_experts& ex, const uint16_t* x, int T, int k,
                           const int32_t* offsets, const int32_t* sorted_pairs, uint16_t* y,
                           void* ws, hipStream_t s) {
    if (ex.fmt == MOE_FMT_INT4_G32)
        return launch_fmt<MOE_FMT_INT4_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
    return launch_fmt<MOE_FMT_INT6_G32>(ex, x, T, k, offsets, sorted_pairs, y, ws, s);
}

}  // namespace moe
