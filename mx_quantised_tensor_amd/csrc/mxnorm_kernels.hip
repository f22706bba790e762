// mxnorm_kernels.hip -- gfx950 kernels of the MXNorm library and their launchers.
//
// Sources (by page title and section):
//   [P1] "MXNorm: Reusing MXFP block scales for efficient tensor
//        normalisation" (gist.science summary), "Resumen tecnico" §1-§3.
//   [P2] the same paper (gptget.net summary) with the authors' abstract.
//   [P3] MXFP4 pre-training on AMD MI355X (gist.science summary),
//        "Metodologia", "Hallazgos" 2 (deterministic H16 / H32 rotation).
//
// All kernels are HBM-bandwidth bound streaming codecs: no MFMA (no dense
// contraction exists on this path), 16-byte loads and stores per lane, a
// row held in VGPRs between its statistic and its cast, and workgroups
// assigned to XCDs in contiguous row ranges.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "mx_device.h"

namespace mxq {

constexpr int kThreads = 256;             // 4 waves per workgroup
constexpr int kNegExp = -100000;          // exponent of a block outside the row
constexpr int kNonFinite = 1000;          // exponent marking a NaN/Inf block

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so that each
// XCD (and its L2) works through one contiguous range of rows.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t n) {
  const int64_t x = b & 7, i = b >> 3, per = n >> 3, rem = n & 7;
  return x < rem ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

template <int ELEM>
struct Elem;
template <>
struct Elem<0> {  // E4M3: largest power of two 2^8 (448 = 1.75 * 2^8)
  static constexpr int kEmax = 8;
  static constexpr int kCodeBytesPerLane = 8;
};
template <>
struct Elem<1> {  // E2M1: largest power of two 2^2 (6 = 1.5 * 2^2)
  static constexpr int kEmax = 2;
  static constexpr int kCodeBytesPerLane = 4;
};

template <int ELEM>
__device__ __forceinline__ void store_codes(uint8_t* __restrict__ dst, const float (&y)[8],
                                            uint32_t e8m0) {
  if constexpr (ELEM == 0)
    *reinterpret_cast<uint2*>(dst) = encode8_e4m3(y, e8m0);
  else
    *reinterpret_cast<uint32_t*>(dst) = encode8_e2m1(y, e8m0);
}

// ----------------------------------------------------------------------------------
// MXNorm forward ([P1] §2 "Implementacion": absmax per block -> RMS estimate ->
// scale the values -> quantisation scales, one pass; [P1] §2 "Formula").
//
// A row is owned by W waves (4/W rows per workgroup).  Lane `lane` of wave
// `wir` owns chunk (s*W + wir)*64 + lane of the row at step s (8 bf16 each).
// Phase 1 keeps the row in VGPRs and reduces the E8M0 exponents of its
// blocks; phase 2 normalises, rotates (HAD), re-derives the output scales
// and casts.
// ----------------------------------------------------------------------------------
template <int ELEM, bool GAMMA, int HAD, int W, int STEPS>
__global__ __launch_bounds__(kThreads) void k_mxnorm(
    const uint4* __restrict__ x, const uint4* __restrict__ gamma, int64_t rows, int hidden,
    int p, float c, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    float* __restrict__ rrms) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  constexpr int RPW = 4 / W;
  static_assert(W == 1 || W == 2 || W == 4, "waves per row");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rslot = wave / W;
  const int wir = wave % W;
  const int64_t row = xcd_remap(blockIdx.x, gridDim.x) * RPW + rslot;
  const bool row_ok = row < rows;
  const int nchunk = hidden >> 3;
  const int K = hidden >> 5;

  // ---- load the row (16 B per lane per step) --------------------------------------
  uint4 v[STEPS];
  bool act[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = (s * W + wir) * kWave + lane;
    act[s] = row_ok && ch < nchunk;  // uniform over each quad: nchunk % 4 == 0
    v[s] = act[s] ? x[row * nchunk + ch] : make_uint4(0, 0, 0, 0);
  }

  // ---- block exponents e_k + emax, from the bf16 exponent field ------------------
  int eh[STEPS];
  int emx = kNegExp;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const uint32_t m = quad_max_u32(absmax8_bf16_bits(v[s]));
    const int e = m >= 0x7F80u ? kNonFinite : max((int)(m >> 7) - 127 - EMAX, -127) + EMAX;
    eh[s] = act[s] ? e : kNegExp;
    emx = max(emx, eh[s]);
  }
  emx = wave_max_quads(emx);
  __shared__ int s_max[4];
  __shared__ double s_sum[4];
  if constexpr (W > 1) {
    if (lane == 0) s_max[wave] = emx;
    __syncthreads();
    emx = s_max[rslot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) emx = max(emx, s_max[rslot * W + w]);
  }
  const int E = emx;

  // ---- power sum S = sum 2^(40 - p (E - eh)), exact in fp64 ---------------------
  double S = 0.0;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int t = p * (E - eh[s]);
    if (t <= 40) S += __longlong_as_double((int64_t)(1023 + 40 - t) << 52);
  }
  S = wave_sum_quads_f64(S);
  if constexpr (W > 1) {
    if (lane == 0) s_sum[wave] = S;
    __syncthreads();
    S = s_sum[rslot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) S += s_sum[rslot * W + w];
  }

  // ---- rho = fl(c / r) * 2^(40/p - E) -------------------------------------------
  // Each step is one correctly rounded fp32 operation.  It is evaluated in
  // fp64 and rounded once to fp32, which gives the same value: for +, /, sqrt
  // a double result rounded to float is the correctly rounded float result
  // (53 >= 2*24 + 2).
  float rho;
  if (E >= kNonFinite) {
    rho = __uint_as_float(0x7FC00000u);
  } else {
    const float Sf = (float)S;  // S < 2^53 is exact in fp64; one rounding here
    const float mu = (float)((double)Sf / (double)K);
    const float r = p == 1 ? mu : (float)sqrt((double)mu);
    const float q = (float)((double)c / (double)r);
    rho = (float)ldexp((double)q, 40 / p - E);
  }
  if (rrms != nullptr && row_ok && wir == 0 && lane == 0) rrms[row] = rho;

  // ---- normalise, rotate, re-derive scales, cast --------------------------------
  const int64_t crow = row * (int64_t)(ELEM == 0 ? hidden : hidden / 2);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!act[s]) continue;  // quad-uniform; DPP below stays inside the quad
    const int ch = (s * W + wir) * kWave + lane;
    float y[8];
    widen8(v[s], y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = y[i] * rho;
    if constexpr (GAMMA) {
      float g[8];
      widen8(gamma[ch], g);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = y[i] * g[i];
    }
    if constexpr (HAD != 0) {
      fwht8_inlane(y);
      fwht8_crosslane<kDppQuadSwap1>(y, (lane & 1) != 0);
      if constexpr (HAD == 32) fwht8_crosslane<kDppQuadSwap2>(y, (lane & 2) != 0);
      constexpr float norm = HAD == 16 ? 0.25f : 0x1.6a09e6p-3f;  // fl32(1/sqrt(32))
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = y[i] * norm;
    }
    const uint32_t mb = quad_max_u32(absmax8_f32_bits(y));
    const uint32_t sb = e8m0_from_expfield<EMAX>(mb >> 23);
    store_codes<ELEM>(codes + crow + (int64_t)ch * Elem<ELEM>::kCodeBytesPerLane, y, sb);
    if ((lane & 3) == 0) scales[row * K + (ch >> 2)] = (uint8_t)sb;
  }
}

// ----------------------------------------------------------------------------------
// MXCast of bf16 data ([P1] §1 and [P2] abstract: the cast whose block scales
// MXNorm reuses).  Flat over 8-element chunks; a quad owns a block.
// ----------------------------------------------------------------------------------
template <int ELEM>
__global__ __launch_bounds__(kThreads) void k_mx_quant(const uint4* __restrict__ x,
                                                        int64_t nchunks,
                                                        uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ scales) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  const int64_t nwg = gridDim.x;
  const int64_t ch = xcd_remap(blockIdx.x, nwg) * kThreads + threadIdx.x;
  if (ch >= nchunks) return;  // nchunks % 4 == 0: quads stay whole
  const uint4 v = x[ch];
  const uint32_t m = quad_max_u32(absmax8_bf16_bits(v));
  const uint32_t sb = e8m0_from_expfield<EMAX>(m >> 7);
  float y[8];
  widen8(v, y);
  store_codes<ELEM>(codes + ch * Elem<ELEM>::kCodeBytesPerLane, y, sb);
  if ((threadIdx.x & 3) == 0) scales[ch >> 2] = (uint8_t)sb;
}

// ----------------------------------------------------------------------------------
// RMSNorm, pass 1 of the two-pass baseline ([P1] §1): full-width fp32 sum of
// squares, rstd = 1/sqrt(mean + eps), bf16 y written to memory.
// ----------------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // RNE
}

template <bool GAMMA, int W, int STEPS>
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const uint4* __restrict__ x,
                                                       const uint4* __restrict__ gamma,
                                                       int64_t rows, int hidden, float eps,
                                                       uint4* __restrict__ y,
                                                       float* __restrict__ rstd) {
  constexpr int RPW = 4 / W;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rslot = wave / W;
  const int wir = wave % W;
  const int64_t row = xcd_remap(blockIdx.x, gridDim.x) * RPW + rslot;
  const bool row_ok = row < rows;
  const int nchunk = hidden >> 3;

  uint4 v[STEPS];
  bool act[STEPS];
  float ss = 0.0f;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = (s * W + wir) * kWave + lane;
    act[s] = row_ok && ch < nchunk;
    v[s] = act[s] ? x[row * nchunk + ch] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    float f[8];
    widen8(v[s], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(f[i], f[i], ss);
  }
  ss = wave_sum_f32(ss);
  __shared__ float s_sum[4];
  if constexpr (W > 1) {
    if (lane == 0) s_sum[wave] = ss;
    __syncthreads();
    ss = s_sum[rslot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) ss += s_sum[rslot * W + w];
  }
  const float rs = 1.0f / __builtin_sqrtf(ss / (float)hidden + eps);
  if (rstd != nullptr && row_ok && wir == 0 && lane == 0) rstd[row] = rs;

#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!act[s]) continue;
    const int ch = (s * W + wir) * kWave + lane;
    float f[8];
    widen8(v[s], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] * rs;
    if constexpr (GAMMA) {
      float g[8];
      widen8(gamma[ch], g);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * g[i];
    }
    y[row * nchunk + ch] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
}

// ----------------------------------------------------------------------------------
// Launchers.  Shapes are validated by the C ABI layer before these run.
// ----------------------------------------------------------------------------------
namespace {

struct RowShape {
  int waves;  // waves per row
  int steps;  // 8-element chunks per lane
};

// Smallest register-resident layout that covers the row.
RowShape pick_row_shape(int hidden) {
  const int nchunk = hidden / 8;
  static const RowShape table[] = {{1, 1}, {1, 2}, {1, 4}, {1, 8}, {2, 8}, {4, 8}, {4, 16}};
  for (const RowShape& r : table)
    if (r.waves * kWave * r.steps >= nchunk) return r;
  return {0, 0};
}

template <int ELEM, bool GAMMA, int HAD, int W, int STEPS>
hipError_t launch_mxnorm_t(const MxnormArgs& a) {
  const int64_t rpw = 4 / W;
  const int64_t grid = (a.rows + rpw - 1) / rpw;
  hipLaunchKernelGGL((k_mxnorm<ELEM, GAMMA, HAD, W, STEPS>), dim3((unsigned)grid),
                     dim3(kThreads), 0, (hipStream_t)a.stream,
                     static_cast<const uint4*>(a.x), static_cast<const uint4*>(a.gamma), a.rows,
                     a.hidden, a.p, a.c, a.codes, a.scales, a.rrms);
  return hipGetLastError();
}

template <int ELEM, bool GAMMA, int HAD>
hipError_t launch_mxnorm_shape(const MxnormArgs& a) {
  const RowShape r = pick_row_shape(a.hidden);
  if (r.waves == 1 && r.steps == 1) return launch_mxnorm_t<ELEM, GAMMA, HAD, 1, 1>(a);
  if (r.waves == 1 && r.steps == 2) return launch_mxnorm_t<ELEM, GAMMA, HAD, 1, 2>(a);
  if (r.waves == 1 && r.steps == 4) return launch_mxnorm_t<ELEM, GAMMA, HAD, 1, 4>(a);
  if (r.waves == 1 && r.steps == 8) return launch_mxnorm_t<ELEM, GAMMA, HAD, 1, 8>(a);
  if (r.waves == 2 && r.steps == 8) return launch_mxnorm_t<ELEM, GAMMA, HAD, 2, 8>(a);
  if (r.waves == 4 && r.steps == 8) return launch_mxnorm_t<ELEM, GAMMA, HAD, 4, 8>(a);
  if (r.waves == 4 && r.steps == 16) return launch_mxnorm_t<ELEM, GAMMA, HAD, 4, 16>(a);
  return hipErrorInvalidValue;
}

template <int ELEM, bool GAMMA>
hipError_t launch_mxnorm_had(const MxnormArgs& a) {
  switch (a.had) {
    case 0: return launch_mxnorm_shape<ELEM, GAMMA, 0>(a);
    case 16: return launch_mxnorm_shape<ELEM, GAMMA, 16>(a);
    case 32: return launch_mxnorm_shape<ELEM, GAMMA, 32>(a);
    default: return hipErrorInvalidValue;
  }
}

template <bool GAMMA, int W, int STEPS>
hipError_t launch_rmsnorm_t(const void* x, const void* gamma, int64_t rows, int hidden,
                            float eps, void* y, float* rstd, void* stream) {
  const int64_t rpw = 4 / W;
  const int64_t grid = (rows + rpw - 1) / rpw;
  hipLaunchKernelGGL((k_rmsnorm<GAMMA, W, STEPS>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(x),
                     static_cast<const uint4*>(gamma), rows, hidden, eps,
                     static_cast<uint4*>(y), rstd);
  return hipGetLastError();
}

template <bool GAMMA>
hipError_t launch_rmsnorm_shape(const void* x, const void* gamma, int64_t rows, int hidden,
                                float eps, void* y, float* rstd, void* stream) {
  const RowShape r = pick_row_shape(hidden);
#define MXQ_RMS(Wv, Sv)                                                                   \
  if (r.waves == Wv && r.steps == Sv)                                                     \
    return launch_rmsnorm_t<GAMMA, Wv, Sv>(x, gamma, rows, hidden, eps, y, rstd, stream);
  MXQ_RMS(1, 1) MXQ_RMS(1, 2) MXQ_RMS(1, 4) MXQ_RMS(1, 8) MXQ_RMS(2, 8) MXQ_RMS(4, 8)
  MXQ_RMS(4, 16)
#undef MXQ_RMS
  return hipErrorInvalidValue;
}

}  // namespace

bool row_shape_supported(int hidden) { return pick_row_shape(hidden).waves != 0; }

hipError_t launch_mxnorm(const MxnormArgs& a) {
  if (a.elem == 0)
    return a.gamma ? launch_mxnorm_had<0, true>(a) : launch_mxnorm_had<0, false>(a);
  return a.gamma ? launch_mxnorm_had<1, true>(a) : launch_mxnorm_had<1, false>(a);
}

hipError_t launch_mx_quant(const void* x, int64_t rows, int hidden, int elem, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  const int64_t nchunks = rows * (int64_t)(hidden / 8);
  const int64_t grid = (nchunks + kThreads - 1) / kThreads;
  if (elem == 0)
    hipLaunchKernelGGL(k_mx_quant<0>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, static_cast<const uint4*>(x), nchunks, codes,
                       scales);
  else
    hipLaunchKernelGGL(k_mx_quant<1>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, static_cast<const uint4*>(x), nchunks, codes,
                       scales);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(const void* x, const void* gamma, int64_t rows, int hidden, float eps,
                          void* y, float* rstd, void* stream) {
  return gamma ? launch_rmsnorm_shape<true>(x, gamma, rows, hidden, eps, y, rstd, stream)
               : launch_rmsnorm_shape<false>(x, gamma, rows, hidden, eps, y, rstd, stream);
}

}  // namespace mxq
