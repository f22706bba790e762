/*
 * check_mxnorm.c -- the C ABI of libmxnorm.so used from plain C, with no
 * Python in the process: device buffers from the HIP runtime, mx_quant and
 * mxnorm_fwd (with and without a gain, p = 1 and 2, E4M3 and E2M1) on the
 * default stream, results compared with the CPU oracle (liboracle_mx.so, test
 * infrastructure) on the same inputs: codes, scales and rho must be
 * identical.  Exit status 0 when every case matches.
 *
 * Inputs: bf16 rows from a SplitMix64 stream (Gaussian-like: sum of four
 * uniforms minus two, times a per-row power-of-two scale in 2^-8 .. 2^8),
 * rounded to bf16 to nearest even.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mxnorm.h"

/* the oracle's entry points (oracle/mx_oracle.c) */
int mxo_mx_quant(const uint16_t *x, int64_t rows, int64_t hidden, int elem, uint8_t *codes,
                 uint8_t *scales);
int mxo_mxnorm_fwd(const uint16_t *x, const uint16_t *gamma, int64_t rows, int64_t hidden,
                   int p, float c, int elem, uint8_t *codes, uint8_t *scales, float *rrms);

static uint64_t sm_state;
static uint64_t splitmix64(void)
{
    uint64_t z = (sm_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static double uniform01(void) { return (double)(splitmix64() >> 11) * 0x1.0p-53; }

static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u); /* finite inputs only */
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(e)                                                                     \
    do {                                                                                 \
        hipError_t err_ = (e);                                                           \
        if (err_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)err_, __FILE__, __LINE__);  \
            exit(2);                                                                     \
        }                                                                                \
    } while (0)

static int run_case(int64_t rows, int64_t hidden, int p, int elem, int with_gamma, int quant)
{
    const int64_t n = rows * hidden, K = hidden / 32;
    const int64_t cbytes = elem == MXQ_E4M3 ? n : n / 2;
    uint16_t *x = malloc(n * 2), *g = malloc(hidden * 2);
    uint8_t *codes = malloc(cbytes), *scales = malloc(rows * K);
    uint8_t *ocodes = malloc(cbytes), *oscales = malloc(rows * K);
    float *rho = malloc(rows * 4), *orho = malloc(rows * 4);
    for (int64_t r = 0; r < rows; r++) {
        const float s = (float)(1 << (splitmix64() % 17)) / 256.0f;
        for (int64_t j = 0; j < hidden; j++) {
            const double v = uniform01() + uniform01() + uniform01() + uniform01() - 2.0;
            x[r * hidden + j] = to_bf16((float)v * s);
        }
    }
    for (int64_t j = 0; j < hidden; j++) g[j] = to_bf16((float)(0.75 + 0.5 * uniform01()));

    void *dx, *dg, *dc, *ds, *dr;
    CHECK_HIP(hipMalloc(&dx, n * 2));
    CHECK_HIP(hipMalloc(&dg, hidden * 2));
    CHECK_HIP(hipMalloc(&dc, cbytes));
    CHECK_HIP(hipMalloc(&ds, rows * K));
    CHECK_HIP(hipMalloc(&dr, rows * 4));
    CHECK_HIP(hipMemcpy(dx, x, n * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dg, g, hidden * 2, hipMemcpyHostToDevice));

    const float c = p == 1 ? mxnorm_default_c(1) : mxnorm_default_c(2);
    mxq_status st;
    int orc;
    if (quant) {
        st = mx_quant(dx, rows, hidden, (mxq_elem)elem, dc, ds, NULL);
        orc = mxo_mx_quant(x, rows, hidden, elem, ocodes, oscales);
    } else {
        st = mxnorm_fwd(dx, with_gamma ? dg : NULL, rows, hidden, p, c, (mxq_elem)elem, dc, ds,
                        dr, NULL);
        orc = mxo_mxnorm_fwd(x, with_gamma ? g : NULL, rows, hidden, p, c, elem, ocodes,
                             oscales, orho);
    }
    if (st != MXQ_OK || orc != 0) {
        fprintf(stderr, "call failed: %s (oracle %d)\n", mxq_status_str(st), orc);
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(codes, dc, cbytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(scales, ds, rows * K, hipMemcpyDeviceToHost));
    int bad = memcmp(codes, ocodes, cbytes) != 0 || memcmp(scales, oscales, rows * K) != 0;
    if (!quant) {
        CHECK_HIP(hipMemcpy(rho, dr, rows * 4, hipMemcpyDeviceToHost));
        bad |= memcmp(rho, orho, rows * 4) != 0;
    }
    printf("%-10s rows=%lld hidden=%lld p=%d elem=%d gamma=%d: %s\n",
           quant ? "mx_quant" : "mxnorm_fwd", (long long)rows, (long long)hidden, p, elem,
           with_gamma, bad ? "MISMATCH" : "identical");
    hipFree(dx); hipFree(dg); hipFree(dc); hipFree(ds); hipFree(dr);
    free(x); free(g); free(codes); free(scales); free(ocodes); free(oscales); free(rho);
    free(orho);
    return bad;
}

int main(void)
{
    sm_state = 20261202u;
    printf("%s\n", mxq_version());
    int bad = 0;
    bad |= run_case(300, 4096, 2, MXQ_E4M3, 1, 0);
    bad |= run_case(300, 4096, 1, MXQ_E4M3, 0, 0);
    bad |= run_case(77, 1056, 2, MXQ_E2M1, 1, 0);
    bad |= run_case(5, 8192, 2, MXQ_E4M3, 1, 0);
    bad |= run_case(129, 2048, 0, MXQ_E4M3, 0, 1);
    bad |= run_case(129, 2048, 0, MXQ_E2M1, 0, 1);
    printf(bad ? "c-abi check FAILED\n" : "c-abi check ok\n");
    return bad ? 1 : 0;
}
