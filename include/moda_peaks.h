/*
 * moda_peaks.h - attained-peak microbenchmarks (libmoda_peaks.so), measurement
 * tools only: they give the rates this MI355X actually reaches on the two
 * resources the MoDA forward is bound by, the HBM stream of the depth slots and
 * the bf16 matrix-core products of the sequence loop (MoDA deck, slide "Depth
 * compute still accumulates quadratically in depth": the sequence part grows
 * with T^2 d and the depth part with T S d). They compute nothing of the operator.
 *
 * Both launch asynchronously on `stream` (a hipStream_t, NULL = default stream),
 * allocate nothing and return 0, 1 for invalid arguments (nothing launched) or 2
 * for a failed launch. All pointers are device memory owned by the caller.
 */
#ifndef MODA_PEAKS_H
#define MODA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16, >= 16) of `buf` (16-byte aligned) once with
 * 16-byte non-temporal loads, `workgroups` workgroups of 256 lanes in a grid-stride
 * loop, and writes one 32-bit XOR per workgroup to sink[0 .. workgroups). */
int moda_peak_stream_read(const void* buf, int64_t bytes, void* sink, int32_t workgroups, void* stream);

/* `workgroups` workgroups of 4 waves; every wave runs `iters` iterations of four
 * independent v_mfma_f32_32x32x16_bf16 on register operands. sink holds at least
 * `workgroups` floats (practically never written: it keeps the products live). */
int moda_peak_mfma_bf16(int32_t iters, void* sink, int32_t workgroups, void* stream);

/* Floating-point operations of one moda_peak_mfma_bf16 launch. */
double moda_peak_mfma_flops_per_launch(int32_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MODA_PEAKS_H */
