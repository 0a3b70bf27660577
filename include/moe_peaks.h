/*
 * moe_peaks.h -- measurement helpers used by bench.py (libmoe_peaks.so), not part of the
 * MoE layer: kernels that show what this GPU reaches on plain work, reported next to the
 * spec peaks.  Each call enqueues one kernel on `stream` (a hipStream_t as void*, NULL = the
 * default stream) and returns a hipError_t value (0 = success); arguments are checked on the
 * host first (hipErrorInvalidValue).  Pointers are device pointers owned by the caller.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of blocks of moe_peaks_stream_read (the length of its sink). */
int moe_peaks_stream_blocks(void);

/* Reads n_bytes (a multiple of 16; src 16-byte aligned) with 16-byte loads, four in flight
 * per thread, grid-stride over moe_peaks_stream_blocks() blocks of 256 threads; writes one
 * 32-bit XOR of what each block read to sink[block]. */
int moe_peaks_stream_read(const void* src, size_t n_bytes, uint32_t* sink, void* stream);

/* `blocks` blocks of 256 threads; every wave runs `iters` rounds of 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands that change from one
 * instruction to the next.  sink: float [blocks * 4] (a sum per wave); clk: uint64
 * [2 * blocks], for each block the shader-clock and 100 MHz reference-clock counts of its
 * first wave's loop. */
int moe_peaks_mfma_loop(int blocks, int iters, float* sink, uint64_t* clk, void* stream);

#ifdef __cplusplus
}
#endif

#endif
