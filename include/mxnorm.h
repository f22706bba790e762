/*
 * mxnorm.h -- C ABI of the MI355X (gfx950) MXNorm library, libmxnorm.so.
 *
 * MXNorm is a drop-in replacement for RMSNorm that emits the row already cast
 * to an MX format and estimates the row's inverse RMS from the E8M0 block
 * scales of that cast.  Sources, cited by page title and section:
 *   [P1] "MXNorm: Reusing MXFP block scales for efficient tensor
 *        normalisation", gist.science summary (Spanish), "Resumen tecnico".
 *   [P2] the same paper, gptget.net summary (Chinese) with the authors'
 *        English abstract.
 *   [P3] summary of the MXFP4 pre-training study on AMD MI355X,
 *        gist.science (Spanish), "Metodologia" and "Hallazgos" 2.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates and frees nothing, keeps no global state, never synchronises
 *     the stream, and may be called from several host threads at once.
 *   - Matrices are row-major with contiguous rows (row stride = hidden).
 *     bf16 data is passed as raw 16-bit patterns.
 *   - Block size is 32 elements along the hidden dimension; hidden must be a
 *     multiple of 32 and at most MXQ_MAX_HIDDEN.
 *   - Outputs of an MX cast (the "MX tensor"):
 *       codes : E4M3 -> rows*hidden bytes, one OCP E4M3 ("FN") code per
 *               element; E2M1 -> rows*hidden/2 bytes, two OCP E2M1 codes per
 *               byte, element 2j in the low nibble of byte j.
 *       scales: rows*(hidden/32) bytes, E8M0 (value 2^(byte-127)); 0xFF is
 *               the NaN scale, used for any block holding NaN or Inf.
 *     Element rule (OCP MX): scale exponent e = floor(log2(block absmax))
 *     - emax (emax 8 for E4M3, 2 for E2M1), clamped to [-127, 127]; an
 *     all-zero block takes e = -127.  Each element is value / 2^e rounded to
 *     the nearest code, ties to the even code, saturating at +-448 (E4M3) or
 *     +-6 (E2M1); the sign of zero is kept.  Codes under a 0xFF scale are
 *     unspecified.
 *   - Alignment: x, codes and any bf16 workspace must be 16-byte aligned;
 *     gamma 16-byte aligned; scales and rrms/rstd need natural alignment only.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns
 *     immediately.  A device fault surfaces at the caller's next
 *     synchronisation, as usual for HIP.
 *   - Errors are reported before anything is launched; rows == 0 is a valid
 *     no-op.
 */
#ifndef MXNORM_H
#define MXNORM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque HIP stream handle (hipStream_t); 0 selects the null stream. */
typedef void *mxq_stream_t;

typedef enum {
    MXQ_OK = 0,
    MXQ_EINVAL = -1,        /* bad shape, NULL pointer, bad p / c / eps / had */
    MXQ_EALIGN = -2,        /* a pointer is not aligned as required above */
    MXQ_EUNSUPPORTED = -3,  /* valid arguments outside what the library supports */
    MXQ_EHIP = -4,          /* the HIP runtime refused the launch */
    MXQ_STATUS_MIN_ = -2147483647 - 1,  /* not statuses: the type spans int */
    MXQ_STATUS_MAX_ = 2147483647
} mxq_status;

/* The argument enums below span the whole int range (the _MIN_ / _MAX_
 * enumerators are not values of the type): a caller may pass any int, and the
 * library rejects values outside the listed ones with MXQ_EINVAL. */
typedef enum {
    MXQ_E4M3 = 0,           /* MXFP8: E4M3 elements, 1 byte each */
    MXQ_E2M1 = 1,           /* MXFP4: E2M1 elements, 2 per byte */
    MXQ_ELEM_MIN_ = -2147483647 - 1,
    MXQ_ELEM_MAX_ = 2147483647
} mxq_elem;

/* Which block magnitude enters the MXNorm power mean. */
typedef enum {
    MXQ_SRC_SCALES = 0,     /* 2^(e_k + emax): the E8M0 scale of block k as a power of two */
    MXQ_SRC_ABSMAX = 1,     /* the exact block absmax max_i |x_i| */
    MXQ_SRC_MIN_ = -2147483647 - 1,
    MXQ_SRC_MAX_ = 2147483647
} mxq_source;

/* Element type of a matrix-product output. */
typedef enum {
    MXQ_OUT_F32 = 0,        /* fp32 */
    MXQ_OUT_BF16 = 1,       /* bf16: the fp32 result rounded to nearest even */
    MXQ_OUT_MIN_ = -2147483647 - 1,
    MXQ_OUT_MAX_ = 2147483647
} mxq_out;

#define MXQ_BLOCK 32
#define MXQ_MAX_HIDDEN 32768

/*
 * mx_quant -- MXCast of a bf16 matrix [rows, hidden] into an MX tensor.
 * The stand-alone cast that follows RMSNorm in the unfused pipeline
 * ([P1] §1; [P2] abstract: block scales computed by the MXFP8 cast).
 *   x      : device bf16 [rows, hidden]
 *   codes  : device out, layout above
 *   scales : device out, [rows, hidden/32]
 */
mxq_status mx_quant(const void *x, int64_t rows, int64_t hidden, mxq_elem elem,
                    uint8_t *codes, uint8_t *scales, mxq_stream_t stream);

/*
 * mxnorm_fwd -- MXNorm forward, one pass over x ([P1] §2 "Implementacion":
 * block absmax, RMS estimate, scaling and quantisation scales fused; [P1] §2
 * "Formula" for the estimate; [P1] §3 for the 32x smaller reduction).
 *   Per row: mt_k = 2^(e_k + emax) with e_k the E8M0 exponent the MX cast of
 *   x gives block k; E = max_k (e_k + emax);
 *   S = sum_k 2^(40 - p (E - e_k - emax)) over the terms with exponent >= 0
 *   (an exact integer); rho = fl(c / r) * 2^(40/p - E) with
 *   r = fl(fl(S)/K) (p = 1) or fl(sqrt(fl(fl(S)/K))) (p = 2), all fp32
 *   correctly rounded; this is c * ((1/K) sum mt_k^p)^(-1/p).
 *   y_i = fl(x_i * rho), then fl(y_i * gamma_i) if gamma is given; y is then
 *   MX-cast with scales taken from y.  A row holding NaN/Inf gets rho = NaN
 *   and all-0xFF scales.
 *   gamma  : device bf16 [hidden], or NULL (the MXNormLinear mode of [P1] §2,
 *            where the gain is folded into the next linear layer)
 *   p      : 1 (arithmetic mean) or 2 (quadratic mean)
 *   c      : correction constant c(p, 32) > 0; 0 selects mxnorm_default_c(p)
 *   rrms   : device fp32 [rows] receiving rho (the inverse-RMS estimate kept
 *            for the straight-through backward of [P1] §2), or NULL
 */
mxq_status mxnorm_fwd(const void *x, const void *gamma, int64_t rows, int64_t hidden,
                      int p, float c, mxq_elem elem, uint8_t *codes, uint8_t *scales,
                      float *rrms, mxq_stream_t stream);

/*
 * mxnorm_hadamard_fwd -- mxnorm_fwd followed, before the cast, by a fixed
 * normalised Sylvester Hadamard rotation of every group of `had` consecutive
 * elements ([P3] "Metodologia" and "Hallazgos" 2: deterministic H16 / H32
 * rotation before MXFP4 quantisation).  rho is the same as mxnorm_fwd's
 * (taken from the unrotated input).  The rotation is a fast Walsh-Hadamard
 * transform in fp32 with butterfly distances 1, 2, 4, ... (each butterfly
 * (a, b) -> (a + b, a - b)), then multiplied by fl(1/sqrt(had)) (0.25 for 16).
 *   had    : 16 or 32
 *   other arguments as mxnorm_fwd
 */
mxq_status mxnorm_hadamard_fwd(const void *x, const void *gamma, int64_t rows,
                               int64_t hidden, int p, float c, int had, mxq_elem elem,
                               uint8_t *codes, uint8_t *scales, float *rrms,
                               mxq_stream_t stream);

/*
 * mxnorm_fwd_ex -- mxnorm_fwd / mxnorm_hadamard_fwd with a choice of block
 * magnitude.  [P2]'s abstract has MXNorm use only the block scales of the
 * cast (MXQ_SRC_SCALES, what mxnorm_fwd computes); [P1] §2 "Formula" writes
 * the estimate over the block absmax itself (MXQ_SRC_ABSMAX):
 *   mt_k = m_k = max_i |x_i| of block k, exactly.  With
 *   E_k = max(floor(log2 m_k), -126) (-126 for a zero block), the 8-bit
 *   integer M_k = m_k 2^(7 - E_k) and E = max_k E_k,
 *   S = sum_k M_k^p 2^(24 - p (E - E_k)) over the terms with
 *   p (E - E_k) <= 24 (an exact integer), and
 *   rho = fl(c / r) * 2^(24/p + 7 - E), r = fl(fl(S)/K) (p = 1) or
 *   fl(sqrt(fl(fl(S)/K))) (p = 2); this is c ((1/K) sum m_k^p)^(-1/p).
 *   An all-zero row has no RMS to estimate: rho = +Inf, and its y (0 * Inf)
 *   is NaN, so all its scales are 0xFF.  NaN/Inf rows as in mxnorm_fwd.
 *   source : MXQ_SRC_SCALES or MXQ_SRC_ABSMAX
 *   c      : 0 selects mxnorm_default_c_for(p, source)
 *   had    : 0 (no rotation), 16 or 32 (as mxnorm_hadamard_fwd)
 *   other arguments as mxnorm_fwd
 */
mxq_status mxnorm_fwd_ex(const void *x, const void *gamma, int64_t rows, int64_t hidden,
                         int p, float c, mxq_source source, int had, mxq_elem elem,
                         uint8_t *codes, uint8_t *scales, float *rrms, mxq_stream_t stream);

/*
 * rmsnorm_mxquant_fwd -- the two-pass pipeline MXNorm replaces ([P1] §1:
 * RMSNorm and the MX cast as separate operations; [P1] §3: the
 * high-precision intermediate makes a round trip through memory).
 *   pass 1: rstd = 1/sqrt(mean(x^2) + eps) (fp32 accumulation),
 *           y = bf16(fl(fl(x * rstd) * gamma)) written to y_workspace;
 *   pass 2: mx_quant(y_workspace).
 *   y_workspace : device bf16 [rows, hidden], caller-owned scratch that
 *                 holds y on return
 *   rstd        : device fp32 [rows], or NULL
 *   eps         : >= 0, finite
 */
mxq_status rmsnorm_mxquant_fwd(const void *x, const void *gamma, int64_t rows,
                               int64_t hidden, float eps, mxq_elem elem,
                               void *y_workspace, uint8_t *codes, uint8_t *scales,
                               float *rstd, mxq_stream_t stream);

/*
 * mx_quant_gain -- MX cast of a weight with a gain folded in ([P1] §2
 * "Implementacion", MXNormLinear: the RMSNorm gain is folded into the
 * weights of the following linear layer).  Casts W'[o, d] = fl32(W[o, d] *
 * gamma[d]) (a product of two bf16 values, exact) row by row exactly as
 * mx_quant casts a matrix.
 *   w      : device bf16 [rows, hidden] (rows = output features of the layer)
 *   gamma  : device bf16 [hidden], 16-byte aligned
 *   codes, scales : as mx_quant
 */
mxq_status mx_quant_gain(const void *w, const void *gamma, int64_t rows, int64_t hidden,
                         mxq_elem elem, uint8_t *codes, uint8_t *scales, mxq_stream_t stream);

/*
 * mx_matmul -- C = A B^T for two MXFP8 matrices (E4M3 codes, one E8M0 scale
 * per 32 consecutive k): C[m, n] = sum_k A[m, k] B[n, k], in fp32, on the
 * gfx950 scaled matrix instructions (the MXFP8 linear layer that consumes the
 * MX tensor, [P1] §2 MXNormLinear; [P2] abstract).
 *   a_codes  : device [M, K] E4M3, 16-byte aligned;  a_scales : [M, K/32]
 *   b_codes  : device [N, K] E4M3, 16-byte aligned;  b_scales : [N, K/32]
 *              (scales 4-byte aligned)
 *   c        : device [M, N] out, fp32 or bf16 (c_type, mxq_out), 4-byte
 *              aligned; bf16 is the fp32 result rounded to nearest even
 * K must be a multiple of 128 (MXQ_EUNSUPPORTED otherwise; MXQ_EINVAL if not
 * a multiple of 32).  A 0xFF scale makes the outputs that use its block NaN.
 * Numerics: each 64-element slice of k is summed by the matrix unit, which
 * aligns the products to the largest one with a short window (measured error
 * up to 2^-11.9 of the largest product of the slice), and the slices are
 * accumulated in fp32.
 */
mxq_status mx_matmul(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                     const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c,
                     mxq_out c_type, mxq_stream_t stream);

/*
 * mxnorm_linear_fwd -- the MXNormLinear forward of [P1] §2: mxnorm_fwd with no
 * gain (E4M3 elements, E8M0-scale reading) into x_codes / x_scales, then
 * out = mx_matmul(x, W') with W' the gain-folded MXFP8 weight from
 * mx_quant_gain.  Two launches.
 *   x        : device bf16 [rows, hidden]; hidden a multiple of 128
 *   w_codes, w_scales : device [out_features, hidden], [out_features, hidden/32]
 *   x_codes, x_scales : device scratch/outputs [rows, hidden], [rows, hidden/32]
 *   rrms     : device fp32 [rows] or NULL
 *   out      : device [rows, out_features], fp32 or bf16 (out_type), as
 *              mx_matmul's c
 */
mxq_status mxnorm_linear_fwd(const void *x, int64_t rows, int64_t hidden, int p, float c,
                             const uint8_t *w_codes, const uint8_t *w_scales,
                             int64_t out_features, uint8_t *x_codes, uint8_t *x_scales,
                             float *rrms, void *out, mxq_out out_type, mxq_stream_t stream);

/*
 * mxnorm_bwd -- straight-through MXNorm backward ([P1] §2 "Implementacion",
 * the gradients item: RMSNorm's gradient logic reused, nothing stored beyond
 * what RMSNorm keeps).  Reading: the MX cast passes the gradient straight
 * through (dy is taken as the gradient of the unquantised y = x*rho*gamma)
 * and the forward's rho takes the place of RMSNorm's rstd.  With
 * g = dy * gamma (g = dy without a gain), per row:
 *     dx_j     = rho * g_j - rho^3 * x_j * (1/hidden) * sum_k x_k g_k
 *     dgamma_j = sum over rows of dy_j * x_j * rho
 * computed in fp32 as dx_j = rho * (g_j - y_j * m) with y = fl(rho * x) and
 * m = (1/hidden) * sum_k y_k g_k (the same value; no intermediate overflows
 * unless dx does), and dx rounded to bf16 (nearest even); dgamma_j
 * accumulates fma(dy_j, y_j, .).  dgamma is summed in an order that
 * depends only on (rows, hidden): results are bit-reproducible run to run.
 *   x, dy     : device bf16 [rows, hidden] (the forward's input and the
 *               gradient of its output), 16-byte aligned
 *   gamma     : device bf16 [hidden], 16-byte aligned, or NULL
 *   rrms      : device fp32 [rows], rho as written by mxnorm_fwd
 *   dx        : device bf16 [rows, hidden] out, 16-byte aligned
 *   dgamma    : device fp32 [hidden] out; required iff gamma != NULL (rows
 *               == 0 writes zeros); ignored without a gain
 *   workspace : device scratch of mxnorm_bwd_workspace_bytes(rows, hidden)
 *               bytes, 16-byte aligned, caller-owned; required iff gamma !=
 *               NULL and rows > 0; its contents on entry do not matter
 * hidden must be a multiple of 32 and at most MXQ_MAX_HIDDEN (MXQ_EUNSUPPORTED
 * above).  The sum over a row of y.g: per lane, eight fused multiply-add
 * chains (one per position in the lane's 8-element chunks, over the chunks in
 * order) added in a fixed tree, then a fixed tree over the wave, and where
 * a row is split over several waves (2 to 8, rows wider than 2048; the
 * count depends only on rows and hidden) the wave sums added in wave order.
 * Two launches with a gain (rows, then the dgamma column sums), one without.
 */
mxq_status mxnorm_bwd(const void *x, const void *dy, const void *gamma, const float *rrms,
                      int64_t rows, int64_t hidden, void *dx, float *dgamma,
                      float *workspace, mxq_stream_t stream);

/*
 * mxnorm_bwd_workspace_bytes -- host function: bytes of the workspace
 * mxnorm_bwd needs with a gain (0 for rows == 0 or unsupported shapes).
 */
size_t mxnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden);

/*
 * mxnorm_bwd_noalloc -- mxnorm_bwd for callers that cannot allocate device
 * memory (work under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, kernels and results as mxnorm_bwd
 * (bit-identical), without the workspace argument: the dgamma partial rows
 * go to a static device array of mxnorm_bwd_noalloc_scratch_bytes() bytes
 * (32 MiB) that each GPU the library runs on holds until the process ends.
 * The call allocates and frees nothing.
 *   - Shapes whose workspace (mxnorm_bwd_workspace_bytes) would exceed the
 *     array return MXQ_EUNSUPPORTED (no supported shape does at present).
 *   - `stream` must belong to the current device (MXQ_EINVAL otherwise);
 *     the first call with a gain on a device looks up the array's device
 *     address (MXQ_EHIP if that fails).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap
 *     on a GPU (other streams, other host threads) race and give wrong
 *     dgamma.  Calls ordered on one stream are safe; nothing needs clearing
 *     between them (every partial row is written before it is read).
 */
mxq_status mxnorm_bwd_noalloc(const void *x, const void *dy, const void *gamma,
                              const float *rrms, int64_t rows, int64_t hidden, void *dx,
                              float *dgamma, mxq_stream_t stream);

/* mxnorm_bwd_noalloc_scratch_bytes -- host function: size of the static
 * scratch array of mxnorm_bwd_noalloc, per GPU, in bytes. */
size_t mxnorm_bwd_noalloc_scratch_bytes(void);

/*
 * mxnorm_default_c -- host function.  Default c(p, 32) for power-of-two block
 * magnitudes and Gaussian activations with a log-uniform row scale (the
 * pages call the constant precalculated but print no value; [P1] §2
 * "Fundamentos Teoricos").  Returns 0 for p outside {1, 2}.
 */
float mxnorm_default_c(int p);

/*
 * mxnorm_default_c_for -- host function.  Default c for either block
 * magnitude: mxnorm_default_c(p) for MXQ_SRC_SCALES; for MXQ_SRC_ABSMAX,
 * c = E[M^p]^(1/p) with M the max of 32 i.i.d. |N(0,1)| (2.3470793 for p = 1,
 * 2.3894572 for p = 2), which makes c E[m^p]^(-1/p) = 1/RMS for Gaussian
 * rows.  Returns 0 for p or source out of range.
 */
float mxnorm_default_c_for(int p, mxq_source source);

/* mxq_status_str -- host function: a static, human-readable status name. */
const char *mxq_status_str(mxq_status s);

/* mxq_version -- host function: library version string. */
const char *mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXNORM_H */
