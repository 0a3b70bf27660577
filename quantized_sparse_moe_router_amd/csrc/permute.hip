// permute.hip -- stable grouping of (token, slot) pairs by expert on gfx950.
//
// Prefill runs many tokens per expert in one batch [Strata 与 Qwen3.8-Flash-Next
// (telli.sh), section GPU、RAM 和 SSD 各司其职]; the grouped GEMM needs each expert's
// pairs contiguous.  The order inside an expert's segment is by pair index p = t*k + j
// (a stable counting sort), so the result is a function of the ids alone.
//
// Work is cut into chunks of kChunk consecutive pairs:
//   1. per-chunk histograms (LDS integer atomics: the counts do not depend on order);
//   2. per expert, an exclusive scan of the chunk counts (blocks of 64 experts, 16 waves
//      each over a slice of the chunks) and the expert's total;
//   3. per chunk (16 waves of 64 pairs): the scan of the totals over experts gives the
//      offsets; each wave ranks its pairs among equal ids (ballot match on the id bits),
//      waves before it in the chunk add their counts, and the pairs are scattered.
// A call with at most 2 kChunk pairs runs all three steps in one block, one or two pairs per
// thread (the several-token decode GEMV reads this grouping too); at most 64 pairs, in one
// wave.
#include "moe_common.h"

namespace moe {

// Device error word: bit 0 is raised by any kernel that meets an expert id outside
// [0, E).
static __device__ int g_bad_id_flag;

namespace {

constexpr int kChunk = 1024;     // pairs per chunk
constexpr int kMaxE = 1024;

// Exclusive scan of cnt[0..E) into out[0..E], out[E] = total; blockDim.x = 1024.
__device__ void block_exclusive_scan(const int* cnt, int* out, int E) {
    __shared__ int part[1024 / 64];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int v = (tid < E) ? cnt[tid] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) part[wv] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int i = 0; i < 1024 / 64; ++i) {
            const int pv = part[i];
            part[i] = run;
            run += pv;
        }
    }
    __syncthreads();
    const int excl = incl - v + part[wv];
    if (tid < E) out[tid] = excl;
    if (tid == E - 1) out[E] = excl + v;
    __syncthreads();
}

// Decode-sized calls (P <= 64): one wave.  Histogram in LDS, a wave-wide exclusive scan
// gives offsets; a pair's sorted position is offsets[id] plus the number of earlier pairs
// with the same id.
__global__ void __launch_bounds__(64) permute_wave_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
    __shared__ int hist[kMaxE];
    const int lane = threadIdx.x;
    const int id = (lane < P) ? ids[lane] : -1;
    const bool valid = lane < P && id >= 0 && id < E;
    for (int e = lane; e < E; e += 64) hist[e] = 0;
    __syncthreads();
    if (lane < P && !valid) {
        pair_pos[lane] = -1;
        atomicOr(&g_bad_id_flag, 1);
    }
    if (valid) atomicAdd(&hist[id], 1);
    __syncthreads();
    // lane owns entries [lane*C, lane*C + C)
    const int C = (E + 63) / 64;
    int local = 0;
    for (int j = 0; j < C; ++j) {
        const int e = lane * C + j;
        if (e < E) local += hist[e];
    }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    int run = incl - local;
    __syncthreads();
    for (int j = 0; j < C; ++j) {
        const int e = lane * C + j;
        if (e < E) {
            const int c = hist[e];
            hist[e] = run;                 // now the exclusive prefix (start of e)
            offsets[e] = run;
            run += c;
        }
    }
    if (lane == 63) offsets[E] = incl;     // total of valid pairs
    __syncthreads();
    int rank = 0;
    for (int q = 0; q < P; ++q) {          // uniform loop: readlane needs a uniform lane
        const int oid = __builtin_amdgcn_readlane(id, q);
        rank += (q < lane && oid == id) ? 1 : 0;
    }
    if (valid) {
        const int pos = hist[id] + rank;
        sorted_pairs[pos] = lane;
        pair_pos[lane] = pos;
    }
}

// Step 1: chunk histograms -> hist[chunk][E].
__global__ void __launch_bounds__(256) chunk_hist_kernel(const int32_t* __restrict__ ids,
                                                         int64_t P, int E,
                                                         int* __restrict__ hist) {
    __shared__ int h[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int64_t p0 = (int64_t)blockIdx.x * kChunk;
    const int64_t p1 = min(P, p0 + kChunk);
    for (int64_t p = p0 + tid; p < p1; p += 256) {
        const int id = ids[p];
        if (id >= 0 && id < E) atomicAdd(&h[id], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = h[e];
}

// Step 2: for experts 64 b .. 64 b + 63, the chunk table becomes each chunk's count of
// earlier pairs of that expert (exclusive scan over chunks), and tot[e] the expert's
// total.  Wave g of the 16 takes chunks [g L, g L + L); lane = expert.
__global__ void __launch_bounds__(1024) chunk_scan_kernel(int* __restrict__ hist, int nchunk,
                                                          int E, int* __restrict__ tot) {
    __shared__ int part[16][64];
    const int lane = threadIdx.x & 63, g = threadIdx.x >> 6;
    const int e = blockIdx.x * 64 + lane;
    const int L = (nchunk + 15) / 16;
    const int c0 = g * L, c1 = min(nchunk, c0 + L);
    int sum = 0;
    if (e < E)
        for (int c = c0; c < c1; ++c) sum += hist[(size_t)c * E + e];
    part[g][lane] = sum;
    __syncthreads();
    int run = 0;
    for (int i = 0; i < g; ++i) run += part[i][lane];
    if (e < E) {
        for (int c = c0; c < c1; ++c) {
            const int v = hist[(size_t)c * E + e];
            hist[(size_t)c * E + e] = run;
            run += v;
        }
        if (g == 15) tot[e] = run;
    }
}

// Lanes of the wave holding the same id as this lane (valid lanes only): a ballot per id
// bit, kept where the lane's bit agrees.
__device__ __forceinline__ uint64_t match_id(int id, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (id >> b) & 1;
        const uint64_t bb = __ballot(bit);
        m &= bit ? bb : ~bb;
    }
    return m;
}

// Step 3: chunk blockIdx.x, 16 waves of 64 consecutive pairs.  Block 0 also writes the
// offsets.
__global__ void __launch_bounds__(1024) chunk_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t P, int E, int nbits,
    const int* __restrict__ start, const int* __restrict__ tot,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
    int32_t* __restrict__ pair_pos) {
    __shared__ int off[kMaxE + 1];
    __shared__ int tl[kMaxE];
    __shared__ __attribute__((aligned(16))) uint8_t wcnt[16][kMaxE];   // pairs of wave w with id e (<= 64)
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid < E) tl[tid] = tot[tid];
    for (int i = tid; i < 16 * kMaxE / 4; i += 1024) reinterpret_cast<uint32_t*>(wcnt)[i] = 0;
    const int64_t p = (int64_t)blockIdx.x * kChunk + tid;
    const bool inrange = p < P;
    const int id = inrange ? ids[p] : -1;
    const bool valid = inrange && id >= 0 && id < E;
    if (inrange && !valid) {
        pair_pos[p] = -1;
        atomicOr(&g_bad_id_flag, 1);
    }
    __syncthreads();
    block_exclusive_scan(tl, off, E);     // ends with a barrier
    if (blockIdx.x == 0)
        for (int e = tid; e <= E; e += 1024) offsets[e] = off[e];
    const uint64_t m = match_id(id, valid, nbits);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (valid && rank == 0) wcnt[w][id] = (uint8_t)__popcll(m);
    __syncthreads();
    if (valid) {
        int pos = off[id] + start[(size_t)blockIdx.x * E + id] + rank;
        for (int i = 0; i < w; ++i) pos += wcnt[i][id];
        sorted_pairs[pos] = (int32_t)p;
        pair_pos[p] = pos;
    }
}

// All three steps in one block (P <= R * kChunk), R pairs per thread: pair p = r * kChunk +
// tid is handled in round r by wave 16 r + (tid >> 6) of R * 16 virtual waves, so virtual
// waves come in pair order.  The histogram (LDS atomics), the scan of the counts gives the
// offsets, and a pair's position is its expert's offset + the pairs of that expert in
// earlier virtual waves + its rank in its own (ballot match on the id bits).
// blockDim.x = 1024.  R = 2 replaces the three chunked launches from 1025 to 2048 pairs
// (128 tokens x top-10: 14.4 -> one launch).
template <int R>
__global__ void __launch_bounds__(1024) permute_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int nbits, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_pos) {
    __shared__ int hist[kMaxE];
    __shared__ int base[kMaxE + 1];
    // pairs of virtual wave v with id e (<= 64)
    __shared__ __attribute__((aligned(16))) uint8_t wcnt[16 * R][kMaxE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (tid < E) hist[tid] = 0;
    for (int i = tid; i < 16 * R * kMaxE / 4; i += 1024)
        reinterpret_cast<uint32_t*>(wcnt)[i] = 0;
    int id[R], rank[R];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int p = r * kChunk + tid;
        const bool inrange = p < P;
        id[r] = inrange ? ids[p] : -1;
        valid[r] = inrange && id[r] >= 0 && id[r] < E;
        if (inrange && !valid[r]) {
            pair_pos[p] = -1;
            atomicOr(&g_bad_id_flag, 1);
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (valid[r]) atomicAdd(&hist[id[r]], 1);
        const uint64_t m = match_id(id[r], valid[r], nbits);
        rank[r] = __popcll(m & ((1ull << lane) - 1ull));
        if (valid[r] && rank[r] == 0) wcnt[r * 16 + w][id[r]] = (uint8_t)__popcll(m);
    }
    __syncthreads();
    block_exclusive_scan(hist, base, E);     // ends with a barrier
    for (int e = tid; e <= E; e += 1024) offsets[e] = base[e];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (valid[r]) {
            const int p = r * kChunk + tid;
            int pos = base[id[r]] + rank[r];
            for (int i = 0; i < r * 16 + w; ++i) pos += wcnt[i][id[r]];
            sorted_pairs[pos] = p;
            pair_pos[p] = pos;
        }
    }
}

}  // namespace

// workspace: [chunk table nchunk x E][expert totals E]; none for the one-block form
size_t permute_ws_bytes(int64_t P, int E) {
    if (P <= 2 * kChunk) return 0;
    const int64_t nchunk = (P + kChunk - 1) / kChunk;
    return (size_t)(nchunk + 1) * (size_t)E * sizeof(int);
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_pos, void* ws, hipStream_t s) {
    const int64_t P = (int64_t)T * k;
    if (P <= 64) {
        permute_wave_kernel<<<1, 64, 0, s>>>(ids, (int)P, E, offsets, sorted_pairs, pair_pos);
        return hipGetLastError();
    }
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    if (P <= kChunk) {
        permute_small_kernel<1><<<1, 1024, 0, s>>>(ids, (int)P, E, nbits, offsets,
                                                   sorted_pairs, pair_pos);
        return hipGetLastError();
    }
    if (P <= 2 * kChunk) {
        permute_small_kernel<2><<<1, 1024, 0, s>>>(ids, (int)P, E, nbits, offsets,
                                                   sorted_pairs, pair_pos);
        return hipGetLastError();
    }
    const int nchunk = (int)((P + kChunk - 1) / kChunk);
    int* hist = static_cast<int*>(ws);
    int* tot = hist + (size_t)nchunk * E;
    chunk_hist_kernel<<<nchunk, 256, 0, s>>>(ids, P, E, hist);
    chunk_scan_kernel<<<(E + 63) / 64, 1024, 0, s>>>(hist, nchunk, E, tot);
    chunk_scatter_kernel<<<nchunk, 1024, 0, s>>>(ids, P, E, nbits, hist, tot, offsets,
                                                 sorted_pairs, pair_pos);
    return hipGetLastError();
}

int* device_error_flag() {
    static int* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!addr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad_id_flag)) == hipSuccess)
            addr[dev] = static_cast<int*>(p);
    }
    return addr[dev];
}

hipError_t read_and_clear_device_error(int* flag) {
    int zero = 0;
    hipError_t e = hipMemcpyFromSymbol(flag, HIP_SYMBOL(g_bad_id_flag), sizeof(int), 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    return hipMemcpyToSymbol(HIP_SYMBOL(g_bad_id_flag), &zero, sizeof(int), 0,
                             hipMemcpyHostToDevice);
}

}  // namespace moe
