/*
 * attn_probe.h - measurement kernels that give the practical ceilings of the
 * device the attention library runs on (not part of the attention path).
 *
 * The attention kernels' rates are reported against the published MI355X
 * peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s) and against these measured
 * ceilings: what a plain streaming read reaches, and what back-to-back matrix
 * instructions reach at the clock the part sustains under that load.
 * Both calls only enqueue work on `stream` (a hipStream_t as void*, NULL = the
 * default stream); every pointer is device memory owned by the caller.
 */
#ifndef ATTN_PROBE_H
#define ATTN_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_PROBE_INVALID (-1) /* NULL pointer, misalignment or a size out of range */
#define ATTN_PROBE_LAUNCH (-5)  /* the HIP runtime refused the launch */

/*
 * Streaming read: `grid` work-groups of 256 threads read the `bytes` bytes at
 * `buf` once (16-byte nontemporal loads, eight in flight per thread, in a
 * grid-stride order) and write one 32-bit XOR fold per thread to `out`
 * (grid * 256 words). bytes must be a positive multiple of 16 and `buf`
 * 16-byte aligned. Rate = bytes / kernel time.
 */
int attn_probe_stream_read(const void *buf, size_t bytes, unsigned *out, int grid, void *stream);

/*
 * Matrix-core loop: `grid` work-groups of four waves; each wave issues
 * `iters` rounds of four independent v_mfma_f32_32x32x16_bf16 (32768 flop
 * each) on register operands, then writes one float per thread to `out`
 * (grid * 256 floats). clk[0..3] receive, from the first wave, the shader
 * clock counter at its start and end and the 100 MHz constant counter at its
 * start and end, so clock = (clk[1] - clk[0]) / (clk[3] - clk[2]) * 100 MHz.
 * Rate = grid * 4 * iters * 4 * 32768 flop / kernel time.
 */
int attn_probe_mfma_bf16(float *out, int grid, int iters, unsigned long long *clk, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H */
