/*
 * mxq_measure.h -- C ABI of libmxq_measure.so: measurement references for
 * the benchmark of the MXNorm library (include/mxnorm.h).  These are not
 * steps of the method ([P1] "MXNorm: Reusing MXFP block scales for efficient
 * tensor normalisation", gist.science summary, "Resumen tecnico" §4 prices
 * the fused norm by memory traffic; these kernels give the practical HBM
 * ceiling of its traffic on the chip).
 *
 * Each pattern moves exactly the bytes of an E4M3 mxnorm_fwd call: it reads
 * x [rows, hidden] bf16 and writes rows x hidden code bytes, rows x hidden/32
 * scale bytes and one fp32 value per row, with non-temporal 16-byte loads and
 * non-temporal code stores, and does no arithmetic beyond XOR.  Outputs
 * (identical for every layout): F = XOR of every 32-bit word of the row; the
 * 8 code bytes of the row's 16-byte input chunk (w0, w1, w2, w3) are the words
 * (w0 ^ w1 ^ F, w2 ^ w3); every scale dword of the row is F; the row's fp32
 * value has the bits of F.  No store of a row leaves before the whole row has
 * arrived (F needs it), as in the forward.
 */
#ifndef MXQ_MEASURE_H
#define MXQ_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Lane layouts; "one wave" / "two waves" is the number of waves per row. */
enum {
    MXQ_PATTERN_ONE_WAVE_CHUNK8 = 0,   /* lane: 8-element chunks s*64 + lane; 8-byte code stores */
    MXQ_PATTERN_TWO_WAVES_CHUNK8 = 1,  /* as the 16384 x 4096 forward: each wave a contiguous half */
    MXQ_PATTERN_ONE_WAVE_LANE16 = 2,   /* lane: 16 consecutive elements (loads 16 B apart), 16-byte stores */
    MXQ_PATTERN_ONE_WAVE_LANE16X = 3,  /* contiguous loads, a DPP swap of halves, 16-byte stores */
    MXQ_PATTERN_TWO_WAVES_LANE16 = 4,  /* two waves, 16 consecutive elements per lane */
    MXQ_PATTERN_TWO_WAVES_LANE16X = 5, /* two waves, each a contiguous half; loads and stores as 3 */
    MXQ_PATTERN_COUNT = 6
};

/* mxq_pattern_supported -- host: 1 if `layout` covers rows of `hidden`
 * (hidden = waves * 512 * {1, 2, 4, 8, 16}; the 16-element layouts need at
 * least 2 chunks per lane), else 0. */
int mxq_pattern_supported(int layout, int64_t hidden);

/* mxq_measure_pattern -- enqueue one pattern pass on `stream` (a HIP stream,
 * 0 = null stream).  x, codes: 16-byte aligned device pointers; scales,
 * rrms: 4-byte aligned.  Returns 0 on success, -1 bad argument, -2
 * misaligned pointer, -3 unsupported layout/shape, -4 launch failure.
 * rows == 0 is a no-op. */
int mxq_measure_pattern(int layout, const void *x, int64_t rows, int64_t hidden, uint8_t *codes,
                        uint8_t *scales, float *rrms, void *stream);

/*
 * The backward's byte pattern: the bytes of an mxnorm_bwd call without a
 * gain ([P1] "Resumen tecnico" §2, gradients item of "Implementacion": the
 * straight-through backward reads x and dy and writes dx), 16-byte
 * non-temporal loads of x [rows, hidden] and dy [rows, hidden] (bf16) and
 * non-temporal 16-byte stores of dx [rows, hidden] (bf16), no arithmetic
 * beyond XOR.  Output: F = XOR of every 32-bit word of the row's x and dy;
 * every 32-bit word of dx is the matching x word ^ dy word ^ F.  `waves`
 * waves own a row (2: two rows per 256-thread workgroup; 8: one row per
 * 512-thread workgroup), with the backward's lane layout.
 */

/* mxq_bwd_pattern_supported -- host: 1 if waves is 2 or 8 and hidden =
 * waves * 512 * {1, 2, 4, 8}, else 0. */
int mxq_bwd_pattern_supported(int waves, int64_t hidden);

/* mxq_measure_bwd_pattern -- enqueue one backward pattern pass on `stream`.
 * x, dy, dx: 16-byte aligned device pointers.  Returns 0 on success, -1 bad
 * argument, -2 misaligned pointer, -3 unsupported waves/shape, -4 launch
 * failure.  rows == 0 is a no-op. */
int mxq_measure_bwd_pattern(int waves, const void *x, const void *dy, int64_t rows,
                            int64_t hidden, void *dx, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_MEASURE_H */
