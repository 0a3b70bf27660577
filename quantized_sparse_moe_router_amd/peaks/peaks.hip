// peaks.hip -- measurement helpers for bench.py, not part of the MoE layer: what this GPU
// reaches on plain work (a stream read from HBM, a loop of bf16 MFMAs), so that the
// layer's rates can be put next to measured ceilings as well as the spec peaks.  Built into
// libmoe_peaks.so, separate from the layer's library.  Declarations: include/moe_peaks.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStreamBlocks = 4096;
constexpr int kThreads = 256;

// Grid-stride read of n16 16-byte words, four loads in flight per thread; the XOR of what a
// block read goes to sink[block] so the loads are not removed.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const u32x4* __restrict__ src,
                                                               size_t n16,
                                                               uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * kThreads;
    size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride],
                    d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int m = 32; m >= 1; m >>= 1) v ^= __shfl_xor(v, m, 64);
    __shared__ uint32_t part[kThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Every wave: `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 chains, operands
// alternating between two register sets of lane-dependent bit patterns (so the inputs change
// from one instruction to the next, as in a GEMM).  Wave 0 of each block records the shader
// clock (s_memtime) and the 100 MHz reference clock (s_memrealtime) around its loop.
__global__ void __launch_bounds__(kThreads) mfma_loop_kernel(int iters, float* __restrict__ sink,
                                                             uint64_t* __restrict__ clk) {
    const int lane = threadIdx.x & 63;
    uint32_t seed = (uint32_t)(lane * 2654435761u) ^ (uint32_t)(blockIdx.x * 40503u);
    auto nxt = [&]() {
        seed = seed * 1664525u + 1013904223u;
        // bf16 pair with exponent near 1 (values in [1, 2) and [-2, -1]), varied mantissas
        return ((seed >> 9) & 0x807f807fu) | 0x3f803f80u;
    };
    u32x4 ra0 = {nxt(), nxt(), nxt(), nxt()}, rb0 = {nxt(), nxt(), nxt(), nxt()};
    u32x4 ra1 = {nxt(), nxt(), nxt(), nxt()}, rb1 = {nxt(), nxt(), nxt(), nxt()};
    const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra0), b0 = __builtin_bit_cast(bf16x8, rb0);
    const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra1), b1 = __builtin_bit_cast(bf16x8, rb1);
    f32x16 acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[c][r] = 0.0f;
    uint64_t t0 = 0, r0 = 0;
    if (threadIdx.x == 0) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 8; ++c)
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((c & 1) ? a1 : a0,
                                                            (c & 2) ? b1 : b0, acc[c], 0, 0, 0);
    }
    if (threadIdx.x == 0) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        clk[2 * blockIdx.x] = t1 - t0;
        clk[2 * blockIdx.x + 1] = r1 - r0;
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    if (lane == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

extern "C" {

int moe_peaks_stream_blocks(void) { return kStreamBlocks; }

int moe_peaks_stream_read(const void* src, size_t n_bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || (n_bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
        return (int)hipErrorInvalidValue;
    stream_read_kernel<<<kStreamBlocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4*>(src), n_bytes / 16, sink);
    return (int)hipGetLastError();
}

int moe_peaks_mfma_loop(int blocks, int iters, float* sink, uint64_t* clk, void* stream) {
    if (blocks < 1 || iters < 1 || !sink || !clk) return (int)hipErrorInvalidValue;
    mfma_loop_kernel<<<blocks, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, sink,
                                                                               clk);
    return (int)hipGetLastError();
}

}  // extern "C"
