/*
 * mx_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, deliberately obvious CPU reference for the MXNorm forward
 * path, its straight-through backward, and their companions.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product library never calls
 * it, and it shares no code, header, table or constant with the GPU path.
 *
 * Sources (cited by page title and section; no other numbering is used):
 *   [P1] "MXNorm: Reusing MXFP block scales for efficient tensor
 *        normalisation" -- gist.science summary (Spanish), "Resumen tecnico".
 *   [P2] The same paper -- gptget.net summary (Chinese) with the authors'
 *        English abstract.
 *   [P3] Summary of the MXFP4 pre-training study on AMD MI355X --
 *        gist.science (Spanish), "Metodologia" and "Hallazgos" sections.
 *
 * The pages state the method but not its bit-level rules; each reading taken
 * here is listed next to the step that uses it.  Number formats follow the
 * OCP Microscaling (MX) definitions: E8M0 shared scale per block of 32,
 * E4M3 (OCP "FN": bias 7, no infinities, max 448) or E2M1 (bias 1, max 6)
 * elements.
 *
 * Precision.  Values that decide an integer output (a code or a scale) are
 * computed in IEEE fp32, the precision the GPU path computes in, with
 * correctly rounded operations; everything else is exact (double holds every
 * quantity below without rounding) or, for the RMSNorm baseline statistic,
 * in fp64 as its plain definition.  Build with -O2 -ffp-contract=off and no
 * fast-math so that C float arithmetic is IEEE single precision.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define MXO_OK 0
#define MXO_EINVAL (-1)

#define MXO_E4M3 0
#define MXO_E2M1 1

/* Which block magnitude enters the power mean (see mxo_row_stat and
 * mxo_row_stat_absmax). */
#define MXO_SRC_SCALES 0
#define MXO_SRC_ABSMAX 1

/* Block size of the MX formats (P2 abstract: reduction 32x smaller; P1 §3). */
#define MXO_BLOCK 32

/* ------------------------------------------------------------------------
 * bf16: sign, 8-bit exponent (bias 127), 7-bit fraction.
 * Decoded from its definition, not by bit reinterpretation.
 * ---------------------------------------------------------------------- */
double mxo_bf16_decode(uint16_t b)
{
    int s = b >> 15;
    int e = (b >> 7) & 0xFF;
    int m = b & 0x7F;
    double mag;
    if (e == 0xFF)
        mag = (m == 0) ? INFINITY : NAN;
    else if (e == 0)
        mag = ldexp((double)m, -126 - 7); /* subnormal: m/128 * 2^-126 */
    else
        mag = ldexp(1.0 + m / 128.0, e - 127);
    return s ? -mag : mag;
}

/* fp32 -> bf16, round to nearest, ties to the even fraction.  The two bf16
 * neighbours of |f| are the truncation t and t+1 (next magnitude); the one
 * closer to |f| wins, and on a tie the one with an even code. */
uint16_t mxo_bf16_encode_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000);
    if (isnan(f))
        return (uint16_t)(sign | 0x7FC0);
    if (isinf(f))
        return (uint16_t)(sign | 0x7F80);
    double a = fabs((double)f);
    uint16_t lo = (uint16_t)((u >> 16) & 0x7FFF); /* truncation, magnitude */
    double vlo = mxo_bf16_decode(lo);
    if (vlo == a)
        return (uint16_t)(sign | lo);
    uint16_t hi = (uint16_t)(lo + 1);
    /* when lo is the largest finite bf16, the next step up is 2^128 (Inf) */
    double vhi = (hi == 0x7F80) ? ldexp(1.0, 128) : mxo_bf16_decode(hi);
    double dlo = a - vlo, dhi = vhi - a;
    uint16_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = (lo & 1) ? hi : lo;
    return (uint16_t)(sign | pick);
}

/* ------------------------------------------------------------------------
 * MX element formats, decoded from the bit fields (OCP MX).
 * ---------------------------------------------------------------------- */
double mxo_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
    double mag;
    if (e == 15 && m == 7)
        mag = NAN;
    else if (e == 0)
        mag = ldexp((double)m, -9); /* m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

double mxo_e2m1_decode(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + m / 2.0, e - 1);
    return s ? -mag : mag;
}

/* Nearest representable magnitude by search over the sorted table of the
 * format's non-negative finite values (their codes are the table indices),
 * ties to the even code, saturating at the largest value.  This is the
 * "round to nearest even, saturate" conversion chosen for MX elements. */
static uint8_t nearest_even_code(double a, const double *tab, int n)
{
    if (!(a < tab[n - 1]))
        return (uint8_t)(n - 1); /* saturate (also a >= max exactly) */
    int lo = 0, hi = n - 1;      /* invariant: tab[lo] <= a < tab[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (tab[mid] <= a)
            lo = mid;
        else
            hi = mid;
    }
    double dlo = a - tab[lo], dhi = tab[hi] - a;
    if (dlo < dhi)
        return (uint8_t)lo;
    if (dhi < dlo)
        return (uint8_t)hi;
    return (uint8_t)((lo & 1) ? hi : lo);
}

static double e4m3_tab[127]; /* codes 0x00..0x7E */
static double e2m1_tab[8];   /* codes 0x0..0x7 */
static int tabs_ready = 0;

static void build_tables(void)
{
    if (tabs_ready)
        return;
    for (int c = 0; c < 127; c++)
        e4m3_tab[c] = mxo_e4m3_decode((uint8_t)c);
    for (int c = 0; c < 8; c++)
        e2m1_tab[c] = mxo_e2m1_decode((uint8_t)c);
    tabs_ready = 1;
}

uint8_t mxo_e4m3_encode(double v)
{
    build_tables();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    return (uint8_t)(sign | nearest_even_code(fabs(v), e4m3_tab, 127));
}

uint8_t mxo_e2m1_encode(double v)
{
    build_tables();
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    if (isnan(v)) /* E2M1 has no NaN; only ever under an 0xFF scale */
        return (uint8_t)(sign | 0x7);
    return (uint8_t)(sign | nearest_even_code(fabs(v), e2m1_tab, 8));
}

/* emax of the element format: exponent of its largest power of two. */
static int elem_emax(int elem) { return elem == MXO_E4M3 ? 8 : 2; }

/* ------------------------------------------------------------------------
 * E8M0 shared scale (OCP MX): X = 2^e with e = floor(log2(amax)) - emax,
 * clamped to the E8M0 range [-127, 127]; amax == 0 takes the smallest scale.
 * floor(log2) is taken exactly from frexp.  Returns 128 for a non-finite
 * amax (the E8M0 NaN byte 0xFF = 128 + 127).
 * ---------------------------------------------------------------------- */
int mxo_scale_exponent(double amax, int emax)
{
    if (!isfinite(amax))
        return 128;
    if (amax == 0.0)
        return -127;
    int k;
    (void)frexp(amax, &k); /* amax = f * 2^k, f in [0.5, 1) */
    int e = (k - 1) - emax;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e;
}

/* Quantise one block of n values (already in their final fp32 form) into
 * codes and one scale byte.  A block holding NaN or Inf gets scale 0xFF. */
static void quantise_block(const float *v, int n, int elem, uint8_t *codes_row,
                           int first, uint8_t *scale_out)
{
    int emax = elem_emax(elem);
    double amax = 0.0;
    int nonfinite = 0;
    for (int i = 0; i < n; i++) {
        if (!isfinite(v[i]))
            nonfinite = 1;
        else if (fabs((double)v[i]) > amax)
            amax = fabs((double)v[i]);
    }
    int e = nonfinite ? 128 : mxo_scale_exponent(amax, emax);
    *scale_out = (uint8_t)(e + 127);
    for (int i = 0; i < n; i++) {
        /* dividing by the power-of-two scale is exact in double */
        double q = nonfinite ? (double)NAN : ldexp((double)v[i], -e);
        int idx = first + i;
        if (elem == MXO_E4M3) {
            codes_row[idx] = mxo_e4m3_encode(q);
        } else {
            uint8_t c = mxo_e2m1_encode(q);
            uint8_t *byte = &codes_row[idx / 2];
            if ((idx & 1) == 0)
                *byte = (uint8_t)((*byte & 0xF0) | c); /* even element: low nibble */
            else
                *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
        }
    }
}

static int64_t codes_per_row(int64_t hidden, int elem)
{
    return elem == MXO_E4M3 ? hidden : hidden / 2;
}

static int check_shape(int64_t rows, int64_t hidden, int elem)
{
    if (rows < 0 || hidden <= 0 || hidden % MXO_BLOCK != 0)
        return MXO_EINVAL;
    if (elem != MXO_E4M3 && elem != MXO_E2M1)
        return MXO_EINVAL;
    return MXO_OK;
}

/* ------------------------------------------------------------------------
 * MXCast of a bf16 matrix [rows, hidden] (P1 §1: the cast to MXFP that
 * RMSNorm's output goes through; P2 abstract: block scales of the cast).
 * ---------------------------------------------------------------------- */
int mxo_mx_quant(const uint16_t *x, int64_t rows, int64_t hidden, int elem,
                 uint8_t *codes, uint8_t *scales)
{
    if (check_shape(rows, hidden, elem) != MXO_OK)
        return MXO_EINVAL;
    build_tables();
    const int64_t K = hidden / MXO_BLOCK, cpr = codes_per_row(hidden, elem);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float v[MXO_BLOCK];
        for (int64_t k = 0; k < K; k++) {
            for (int i = 0; i < MXO_BLOCK; i++)
                v[i] = (float)mxo_bf16_decode(x[r * hidden + k * MXO_BLOCK + i]);
            quantise_block(v, MXO_BLOCK, elem, codes + r * cpr, (int)(k * MXO_BLOCK),
                           &scales[r * K + k]);
        }
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------------
 * The MXNorm row statistic.
 *
 * P1 §2 "Fórmula": the inverse RMS is estimated as
 *     rho = c(p,B) * ( (1/K) * sum_k mt_k^p )^(-1/p),   K = hidden / B,
 * from per-block magnitudes mt_k (P1 §2 "Fundamentos Teóricos", Theorem 1:
 * the power mean of block absmax tracks the RMS up to a constant).  P2's
 * abstract says only the block scales of the MXFP8 cast are used, so mt_k is
 * the E8M0 scale of block k re-expressed as a power-of-two absmax:
 *     mt_k = 2^(e_k + emax),  e_k = the block's E8M0 exponent for the cast of x.
 *
 * Exact evaluation of the sum: with E = max_k (e_k + emax) and
 * t_k = p*(E - e_k - emax), (1/K) sum mt_k^p = 2^(pE) * 2^-40 * S / K where
 *     S = sum_k [t_k <= 40] * 2^(40 - t_k)
 * is an integer (terms below 2^-40 of the largest are dropped).  S is summed
 * exactly in uint64 (S < 2^53 whenever K < 2^13).
 *
 * Returns the row maximum E (or 1000 if the row holds NaN/Inf) and S.
 * ---------------------------------------------------------------------- */
int mxo_row_stat(const uint16_t *xrow, int64_t hidden, int p, int emax,
                 int *E_out, uint64_t *S_out)
{
    const int64_t K = hidden / MXO_BLOCK;
    int E = -100000, nonfinite = 0;
    for (int64_t k = 0; k < K; k++) {
        double amax = 0.0;
        for (int i = 0; i < MXO_BLOCK; i++) {
            double v = mxo_bf16_decode(xrow[k * MXO_BLOCK + i]);
            if (!isfinite(v))
                nonfinite = 1;
            else if (fabs(v) > amax)
                amax = fabs(v);
        }
        int eh = mxo_scale_exponent(amax, emax) + emax;
        if (eh > E)
            E = eh;
    }
    if (nonfinite) {
        *E_out = 1000;
        *S_out = 0;
        return MXO_OK;
    }
    uint64_t S = 0;
    for (int64_t k = 0; k < K; k++) {
        double amax = 0.0;
        for (int i = 0; i < MXO_BLOCK; i++) {
            double v = fabs(mxo_bf16_decode(xrow[k * MXO_BLOCK + i]));
            if (v > amax)
                amax = v;
        }
        int eh = mxo_scale_exponent(amax, emax) + emax;
        int t = p * (E - eh);
        if (t <= 40)
            S += (uint64_t)1 << (40 - t);
    }
    *E_out = E;
    *S_out = S;
    return MXO_OK;
}

/* rho from (E, S) in correctly rounded fp32 steps:
 *   mu = fl(fl(S) / K);  r = mu (p = 1) or fl(sqrt(mu)) (p = 2);
 *   rho = fl(c / r) * 2^(40/p - E)   (the power of two is exact unless the
 *   result leaves the normal range, where ldexpf rounds once). */
float mxo_rho(int E, uint64_t S, int64_t K, int p, float c)
{
    if (E == 1000)
        return NAN;
    float Sf = (float)S;
    float mu = Sf / (float)K;
    float r = (p == 1) ? mu : sqrtf(mu);
    float q = c / r;
    return ldexpf(q, 40 / p - E);
}

/* ------------------------------------------------------------------------
 * The other reading of the block magnitude: P1 §2 "Formula" writes the
 * estimate over the block absmax itself, mt_k = m_k = max_i |x_i| (exact),
 * rather than its power-of-two E8M0 scale.
 *
 * Exact evaluation: a bf16 absmax has 8 significant bits, so with
 *     E_k = max(floor(log2 m_k), -126)   (-126 for a zero block)
 *     M_k = m_k * 2^(7 - E_k)            (an integer in [0, 255])
 * and E = max_k E_k,
 *     (1/K) sum m_k^p = 2^(p (E - 7) - 24) * S / K,
 *     S = sum_k [p (E - E_k) <= 24] * M_k^p * 2^(24 - p (E - E_k)),
 * an integer below 2^50 for K <= 1024 (terms whose exponent is more than
 * 24 / p below the largest are dropped).  E = 1000 marks a row with NaN/Inf.
 * ---------------------------------------------------------------------- */
static void block_absmax_parts(double m, int *E_k, uint64_t *M_k)
{
    if (m == 0.0) {
        *E_k = -126;
        *M_k = 0;
        return;
    }
    int ex;
    (void)frexp(m, &ex); /* m = f * 2^ex, f in [0.5, 1): floor(log2 m) = ex - 1 */
    int e = ex - 1;
    if (e < -126)
        e = -126;
    *E_k = e;
    *M_k = (uint64_t)ldexp(m, 7 - e); /* exact: 8 significant bits */
}

int mxo_row_stat_absmax(const uint16_t *xrow, int64_t hidden, int p, int *E_out,
                        uint64_t *S_out)
{
    const int64_t K = hidden / MXO_BLOCK;
    int E = -100000, nonfinite = 0;
    for (int64_t k = 0; k < K; k++) {
        double amax = 0.0;
        for (int i = 0; i < MXO_BLOCK; i++) {
            double v = mxo_bf16_decode(xrow[k * MXO_BLOCK + i]);
            if (!isfinite(v))
                nonfinite = 1;
            else if (fabs(v) > amax)
                amax = fabs(v);
        }
        int ek;
        uint64_t mk;
        block_absmax_parts(amax, &ek, &mk);
        if (ek > E)
            E = ek;
    }
    if (nonfinite) {
        *E_out = 1000;
        *S_out = 0;
        return MXO_OK;
    }
    uint64_t S = 0;
    for (int64_t k = 0; k < K; k++) {
        double amax = 0.0;
        for (int i = 0; i < MXO_BLOCK; i++) {
            double v = fabs(mxo_bf16_decode(xrow[k * MXO_BLOCK + i]));
            if (v > amax)
                amax = v;
        }
        int ek;
        uint64_t mk;
        block_absmax_parts(amax, &ek, &mk);
        int t = p * (E - ek);
        if (t <= 24) {
            uint64_t mp = (p == 1) ? mk : mk * mk;
            S += mp << (24 - t);
        }
    }
    *E_out = E;
    *S_out = S;
    return MXO_OK;
}

/* rho for the absmax reading: mu = fl(fl(S) / K); r = mu (p = 1) or
 * fl(sqrt(mu)) (p = 2); rho = fl(c / r) * 2^(24/p + 7 - E).  An all-zero row
 * has S = 0 and no RMS to estimate: rho = +Inf. */
float mxo_rho_absmax(int E, uint64_t S, int64_t K, int p, float c)
{
    if (E == 1000)
        return NAN;
    float Sf = (float)S;
    float mu = Sf / (float)K;
    float r = (p == 1) ? mu : sqrtf(mu);
    float q = c / r;
    return ldexpf(q, 24 / p + 7 - E);
}

/* In-place fast Walsh-Hadamard transform of each group of `had` values
 * (had = 16 or 32), natural (Sylvester) order, in fp32, butterfly distance
 * h = 1, 2, 4, ...; each butterfly maps (a, b) -> (a + b, a - b); then the
 * group is multiplied by the normalisation 1/sqrt(had) rounded to fp32
 * (0.25 exactly for had = 16).  P3 "Metodología": a fixed, deterministic
 * 16x16 (H16) or 32x32 (H32) Hadamard rotation before MXFP4 quantisation. */
void mxo_fwht_f32(float *y, int64_t n, int had)
{
    const float norm = (had == 16) ? 0.25f : (float)(1.0 / sqrt((double)had));
    for (int64_t g = 0; g + had <= n; g += had) {
        for (int h = 1; h < had; h *= 2)
            for (int j = 0; j < had; j++)
                if ((j % (2 * h)) < h) {
                    float a = y[g + j], b = y[g + j + h];
                    y[g + j] = a + b;
                    y[g + j + h] = a - b;
                }
        for (int j = 0; j < had; j++)
            y[g + j] = y[g + j] * norm;
    }
}

/* ------------------------------------------------------------------------
 * MXNorm forward (P1 §2 "Implementación", fusion: block absmax -> RMS
 * estimate -> scale the values -> quantisation scales, one pass; P2
 * abstract: drop-in for RMSNorm emitting the MXFP8 tensor).
 *   y_i = fl(x_i * rho), then fl(y_i * gamma_i) when gamma is given (NULL is
 *   the MXNormLinear mode of P1 §2, gain folded into the next linear layer);
 *   optional Hadamard rotation (had = 16 / 32, P3); then MXCast of y with
 *   scales re-derived from y.  rrms (optional) receives rho per row.
 * ---------------------------------------------------------------------- */
static int mxnorm_common(const uint16_t *x, const uint16_t *gamma, int64_t rows,
                         int64_t hidden, int p, float c, int source, int had, int elem,
                         uint8_t *codes, uint8_t *scales, float *rrms)
{
    if (source != MXO_SRC_SCALES && source != MXO_SRC_ABSMAX)
        return MXO_EINVAL;
    if (check_shape(rows, hidden, elem) != MXO_OK)
        return MXO_EINVAL;
    if (p != 1 && p != 2)
        return MXO_EINVAL;
    if (!(c > 0.0f) || !isfinite(c))
        return MXO_EINVAL;
    if (had != 0 && had != 16 && had != 32)
        return MXO_EINVAL;
    if (hidden / MXO_BLOCK >= (1 << 13))
        return MXO_EINVAL;
    build_tables();
    const int emax = elem_emax(elem);
    const int64_t K = hidden / MXO_BLOCK, cpr = codes_per_row(hidden, elem);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *xr = x + r * hidden;
        int E;
        uint64_t S;
        float rho;
        if (source == MXO_SRC_SCALES) {
            mxo_row_stat(xr, hidden, p, emax, &E, &S);
            rho = mxo_rho(E, S, K, p, c);
        } else {
            mxo_row_stat_absmax(xr, hidden, p, &E, &S);
            rho = mxo_rho_absmax(E, S, K, p, c);
        }
        if (rrms)
            rrms[r] = rho;
        float y[MXO_BLOCK];
        for (int64_t k = 0; k < K; k++) {
            for (int i = 0; i < MXO_BLOCK; i++) {
                int64_t col = k * MXO_BLOCK + i;
                float xi = (float)mxo_bf16_decode(xr[col]);
                float yi = xi * rho;
                if (gamma)
                    yi = yi * (float)mxo_bf16_decode(gamma[col]);
                y[i] = yi;
            }
            if (had)
                mxo_fwht_f32(y, MXO_BLOCK, had);
            quantise_block(y, MXO_BLOCK, elem, codes + r * cpr, (int)(k * MXO_BLOCK),
                           &scales[r * K + k]);
        }
    }
    return MXO_OK;
}

int mxo_mxnorm_fwd(const uint16_t *x, const uint16_t *gamma, int64_t rows, int64_t hidden,
                   int p, float c, int elem, uint8_t *codes, uint8_t *scales, float *rrms)
{
    return mxnorm_common(x, gamma, rows, hidden, p, c, MXO_SRC_SCALES, 0, elem, codes, scales,
                         rrms);
}

/* Both readings of the block magnitude and the optional rotation in one call. */
int mxo_mxnorm_fwd_ex(const uint16_t *x, const uint16_t *gamma, int64_t rows, int64_t hidden,
                      int p, float c, int source, int had, int elem, uint8_t *codes,
                      uint8_t *scales, float *rrms)
{
    return mxnorm_common(x, gamma, rows, hidden, p, c, source, had, elem, codes, scales, rrms);
}

int mxo_mxnorm_hadamard_fwd(const uint16_t *x, const uint16_t *gamma, int64_t rows,
                            int64_t hidden, int p, float c, int had, int elem,
                            uint8_t *codes, uint8_t *scales, float *rrms)
{
    if (had != 16 && had != 32)
        return MXO_EINVAL;
    return mxnorm_common(x, gamma, rows, hidden, p, c, MXO_SRC_SCALES, had, elem, codes, scales,
                         rrms);
}

/* ------------------------------------------------------------------------
 * The two-pass baseline MXNorm replaces (P1 §1: RMSNorm and the MXCast run
 * as separate operations; P1 §3: the high-precision intermediate goes
 * through memory):
 *   pass 1: rstd = 1 / sqrt(mean_i x_i^2 + eps), mean in fp64, rounded once
 *           to fp32; y_i = bf16_rne(fl(fl(x_i * rstd) * gamma_i));
 *   pass 2: MXCast of the bf16 y.
 * ---------------------------------------------------------------------- */
int mxo_rmsnorm_mxquant_fwd(const uint16_t *x, const uint16_t *gamma, int64_t rows,
                            int64_t hidden, float eps, int elem, uint16_t *y_out,
                            uint8_t *codes, uint8_t *scales, float *rstd)
{
    if (check_shape(rows, hidden, elem) != MXO_OK)
        return MXO_EINVAL;
    if (!(eps >= 0.0f) || !isfinite(eps))
        return MXO_EINVAL;
    build_tables();
    const int64_t K = hidden / MXO_BLOCK, cpr = codes_per_row(hidden, elem);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *xr = x + r * hidden;
        double ss = 0.0;
        for (int64_t i = 0; i < hidden; i++) {
            double v = mxo_bf16_decode(xr[i]);
            ss += v * v;
        }
        float rs = (float)(1.0 / sqrt(ss / (double)hidden + (double)eps));
        if (rstd)
            rstd[r] = rs;
        float v[MXO_BLOCK];
        for (int64_t k = 0; k < K; k++) {
            for (int i = 0; i < MXO_BLOCK; i++) {
                int64_t col = k * MXO_BLOCK + i;
                float yi = (float)mxo_bf16_decode(xr[col]) * rs;
                if (gamma)
                    yi = yi * (float)mxo_bf16_decode(gamma[col]);
                uint16_t yb = mxo_bf16_encode_rne(yi);
                if (y_out)
                    y_out[r * hidden + col] = yb;
                v[i] = (float)mxo_bf16_decode(yb);
            }
            quantise_block(v, MXO_BLOCK, elem, codes + r * cpr, (int)(k * MXO_BLOCK),
                           &scales[r * K + k]);
        }
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------------
 * MXNorm backward (P1 §2 "Implementacion", the gradients item: a
 * straight-through estimator that reuses the standard RMSNorm gradient, with
 * no extra memory beyond what RMSNorm keeps).
 *
 * Reading taken (the pages give no formula):
 *   - the MX cast is passed straight through: dy is the gradient with respect
 *     to the unquantised y = x * rho * gamma;
 *   - rho, the forward's per-row estimate saved like RMSNorm's rstd, takes
 *     the place of rstd in RMSNorm's gradient.  With g = dy * gamma:
 *         dx_j     = rho * g_j - rho^3 * x_j * (1/D) * sum_k x_k g_k
 *         dgamma_j = sum over rows of dy_j * x_j * rho
 *     (gamma == NULL: g = dy and no dgamma).
 * The pages fix no precision; everything is evaluated in fp64 and returned
 * unrounded.
 * ---------------------------------------------------------------------- */
int mxo_mxnorm_bwd(const uint16_t *x, const uint16_t *dy, const uint16_t *gamma,
                   const float *rho, int64_t rows, int64_t hidden, double *dx,
                   double *dgamma)
{
    if (rows < 0 || hidden <= 0)
        return MXO_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        const uint16_t *xr = x + r * hidden, *dyr = dy + r * hidden;
        const double rh = (double)rho[r];
        double dot = 0.0; /* sum_k x_k g_k */
        for (int64_t k = 0; k < hidden; k++) {
            double gk = mxo_bf16_decode(dyr[k]);
            if (gamma)
                gk *= mxo_bf16_decode(gamma[k]);
            dot += mxo_bf16_decode(xr[k]) * gk;
        }
        const double corr = rh * rh * rh * dot / (double)hidden;
        for (int64_t j = 0; j < hidden; j++) {
            double gj = mxo_bf16_decode(dyr[j]);
            if (gamma)
                gj *= mxo_bf16_decode(gamma[j]);
            dx[r * hidden + j] = rh * gj - corr * mxo_bf16_decode(xr[j]);
        }
    }
    if (gamma && dgamma) {
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < hidden; j++) {
            double acc = 0.0;
            for (int64_t r = 0; r < rows; r++)
                acc += mxo_bf16_decode(dy[r * hidden + j]) * mxo_bf16_decode(x[r * hidden + j]) *
                       (double)rho[r];
            dgamma[j] = acc;
        }
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------------
 * MXNormLinear (P1 §2 "Implementacion", MXNormLinear item: the gain is folded
 * into the weights of the following linear layer, and that layer consumes
 * the MX tensor MXNorm emits).
 *
 * mxo_mx_quant_gain: the folded weight W'[o, d] = W[o, d] * gamma[d] (a
 * product of two bf16 values, exact in fp32), MX-cast along d exactly as
 * mxo_mx_quant casts a matrix (scales per 32 consecutive d).
 * ---------------------------------------------------------------------- */
int mxo_mx_quant_gain(const uint16_t *w, const uint16_t *gamma, int64_t rows, int64_t hidden,
                      int elem, uint8_t *codes, uint8_t *scales)
{
    if (check_shape(rows, hidden, elem) != MXO_OK || gamma == NULL)
        return MXO_EINVAL;
    build_tables();
    const int64_t K = hidden / MXO_BLOCK, cpr = codes_per_row(hidden, elem);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; r++) {
        float v[MXO_BLOCK];
        for (int64_t k = 0; k < K; k++) {
            for (int i = 0; i < MXO_BLOCK; i++) {
                int64_t col = k * MXO_BLOCK + i;
                v[i] = (float)mxo_bf16_decode(w[r * hidden + col]) *
                       (float)mxo_bf16_decode(gamma[col]);
            }
            quantise_block(v, MXO_BLOCK, elem, codes + r * cpr, (int)(k * MXO_BLOCK),
                           &scales[r * K + k]);
        }
    }
    return MXO_OK;
}

/* Value of element k of an MXFP8 (E4M3) row: code * 2^(scale - 127); a 0xFF
 * scale is NaN. */
static double mx_e4m3_value(const uint8_t *codes, const uint8_t *scales, int64_t k)
{
    uint8_t s = scales[k / MXO_BLOCK];
    if (s == 0xFF)
        return NAN;
    return ldexp(mxo_e4m3_decode(codes[k]), (int)s - 127);
}

/* Dot product of two MXFP8 rows of length K, in fp64 in index order. */
double mxo_mx_dot(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                  const uint8_t *b_scales, int64_t K)
{
    build_tables();
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++)
        acc += mx_e4m3_value(a_codes, a_scales, k) * mx_e4m3_value(b_codes, b_scales, k);
    return acc;
}

/* C[m, n] = sum_k A[m, k] B[n, k] for MXFP8 A [M, K] and B [N, K] (both
 * K-contiguous with scales [*, K/32]), in fp64. */
int mxo_mx_matmul(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                  const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, double *c)
{
    if (M < 0 || N < 0 || K <= 0 || K % MXO_BLOCK != 0)
        return MXO_EINVAL;
    build_tables();
    const int64_t KB = K / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            c[m * N + n] = mxo_mx_dot(a_codes + m * K, a_scales + m * KB, b_codes + n * K,
                                      b_scales + n * KB, K);
    return MXO_OK;
}

/* The same for a list of (m, n) pairs only (large shapes, sampled outputs). */
int mxo_mx_matmul_sampled(const uint8_t *a_codes, const uint8_t *a_scales,
                          const uint8_t *b_codes, const uint8_t *b_scales, int64_t K,
                          const int64_t *mn, int64_t count, double *out)
{
    if (K <= 0 || K % MXO_BLOCK != 0)
        return MXO_EINVAL;
    build_tables();
    const int64_t KB = K / MXO_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; t++) {
        int64_t m = mn[2 * t], n = mn[2 * t + 1];
        out[t] = mxo_mx_dot(a_codes + m * K, a_scales + m * KB, b_codes + n * K,
                            b_scales + n * KB, K);
    }
    return MXO_OK;
}

/* ------------------------------------------------------------------------
 * Bulk helpers used by the tests to pin the scalar routines over large sets.
 * ---------------------------------------------------------------------- */
void mxo_bf16_encode_array(const float *f, int64_t n, uint16_t *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = mxo_bf16_encode_rne(f[i]);
}

void mxo_encode_array(const double *v, int64_t n, int elem, uint8_t *out)
{
    build_tables();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        out[i] = elem == MXO_E4M3 ? mxo_e4m3_encode(v[i]) : mxo_e2m1_encode(v[i]);
}

int mxo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the OpenMP loops (timing of the CPU baseline only). */
void mxo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
