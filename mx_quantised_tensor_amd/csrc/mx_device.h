// mx_device.h -- device-side building blocks of the gfx950 MX kernels.
//
// Data layout inside a wavefront: a lane owns 8 consecutive bf16 elements
// (one 16-byte load), so the 32-element MX block is owned by a quad of four
// adjacent lanes.  Block-wide reductions are two quad DPP steps; row-wide
// reductions combine one value per quad.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

constexpr int kElemsPerLane = 8;
constexpr int kWave = 64;

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// ---- bf16 widening (exact: a bf16 pattern is the top half of an fp32) ------
__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }

__device__ __forceinline__ void widen8(const uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ---- cross-lane moves ----------------------------------------------------------
// DPP quad permutations: swap neighbours (1,0,3,2) and swap pairs (2,3,0,1).
constexpr int kDppQuadSwap1 = 0xB1;
constexpr int kDppQuadSwap2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// DPP read with bound_ctrl and a zero `old`, the form the compiler folds
// into the consuming VALU instruction (e.g. v_max_u32_dpp).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp0_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = max(v, dpp0_u32<kDppQuadSwap1>(v));
  v = max(v, dpp0_u32<kDppQuadSwap2>(v));
  return v;
}

// Max / sum over the 16 quads of a wave of quad-uniform values.  Rotations
// by 4 and 8 lanes inside each 16-lane DPP row combine its four quads; the
// four rows are then combined through scalar reads of lanes 0, 16, 32, 48.
// The result is wave-uniform.
__device__ __forceinline__ int wave_max_quads(int v) {
  v = max(v, (int)dpp_u32<kDppRowRor4>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppRowRor8>((uint32_t)v));
  int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)u), hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp_f64_ror4(double v) {
  uint64_t u = __double_as_longlong(v);
  uint32_t lo = dpp_u32<kDppRowRor4>((uint32_t)u), hi = dpp_u32<kDppRowRor4>((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double dpp_f64_ror8(double v) {
  uint64_t u = __double_as_longlong(v);
  uint32_t lo = dpp_u32<kDppRowRor8>((uint32_t)u), hi = dpp_u32<kDppRowRor8>((uint32_t)(u >> 32));
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  uint64_t u = __double_as_longlong(v);
  uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, lane);
  uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
  return __longlong_as_double(((uint64_t)hi << 32) | lo);
}

// Sum of quad-uniform doubles over the 16 quads.  Every operand is an integer
// below 2^53 here, so each addition is exact and the order is immaterial.
__device__ __forceinline__ double wave_sum_quads_f64(double v) {
  v += dpp_f64_ror4(v);
  v += dpp_f64_ror8(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Full-wave fp32 sum (every lane holds a distinct partial); fixed tree.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<kDppQuadSwap1>(v);
  v += dpp_f32<kDppQuadSwap2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  const int iv = __float_as_int(v);
  const float a = __int_as_float(__builtin_amdgcn_readlane(iv, 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(iv, 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(iv, 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(iv, 48));
  return (a + b) + (c + d);
}

// ---- MX block statistics --------------------------------------------------------
// Largest |x| of the 8 bf16 in v as a 15-bit magnitude pattern (the integer
// order of bf16 magnitude patterns is the order of |x|; NaN > Inf > finite).
__device__ __forceinline__ uint32_t absmax8_bf16_bits(const uint4 v) {
  u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
  u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
  u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
  u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
  u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                      __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// Largest |y| of 8 fp32 values, as the bit pattern of a non-negative float
// (IEEE maximum propagates NaN; v_maximum3_f32 with |.| modifiers on gfx950).
__device__ __forceinline__ uint32_t absmax8_f32_bits(const float (&y)[8]) {
  float m = __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(__builtin_fabsf(y[0]), __builtin_fabsf(y[1])),
      __builtin_fabsf(y[2]));
  m = __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(m, __builtin_fabsf(y[3])), __builtin_fabsf(y[4]));
  m = __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(m, __builtin_fabsf(y[5])), __builtin_fabsf(y[6]));
  m = __builtin_elementwise_maximum(m, __builtin_fabsf(y[7]));
  return __float_as_uint(m);
}

// E8M0 byte of a block whose absmax has biased binary exponent field `ef`
// (8 bits; 255 = Inf/NaN; 0 = zero or subnormal): 2^(byte-127) with
// byte - 127 = max(floor(log2 amax) - emax, -127), 0xFF for Inf/NaN.
template <int EMAX>
__device__ __forceinline__ uint32_t e8m0_from_expfield(uint32_t ef) {
  return ef == 255u ? 255u : (uint32_t)max((int)ef - EMAX, 0);
}

// ---- element encoders (gfx950 OCP conversion instructions) -----------------------
// V_CVT_SCALEF32_PK_FP8_F32 / _FP4_F32 divide each input by the scale operand
// and round to nearest even; only the scale's exponent field is read, so the
// E8M0 byte shifted into the fp32 exponent field is the scale itself (field 0
// stands for 2^-127).  Measured on gfx950: the FP4 form saturates at +-6, the
// FP8 form does not (a quotient of 464 or more becomes the NaN code), so the
// E4M3 path clamps y to +-448 * 2^e before converting.
__device__ __forceinline__ float scale_operand(uint32_t e8m0) {
  return __uint_as_float(e8m0 << 23);
}

// 448 * 2^(byte-127) = 1.75 * 2^(byte-119): exponent field byte + 8, fraction .11b.
__device__ __forceinline__ float e4m3_bound(uint32_t e8m0) {
  return __uint_as_float(((e8m0 + 8u) << 23) | 0x600000u);
}

__device__ __forceinline__ uint2 encode8_e4m3(const float (&y)[8], uint32_t e8m0) {
  const float s = scale_operand(e8m0);
  const float b = e4m3_bound(e8m0);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_fmed3f(y[i], -b, b);
  // each word of lo / hi is written by one conversion, so their starting value
  // is irrelevant: seed them with registers that die here (saves two moves)
  i16x2 lo = __builtin_bit_cast(i16x2, v[0]), hi = __builtin_bit_cast(i16x2, v[4]);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[0], v[1], s, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[2], v[3], s, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v[4], v[5], s, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v[6], v[7], s, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// Two E2M1 codes per byte, the even element in the low nibble.
__device__ __forceinline__ uint32_t encode8_e2m1(const float (&y)[8], uint32_t e8m0) {
  const float s = scale_operand(e8m0);
  uint32_t r = __float_as_uint(y[0]);  // every byte is overwritten below
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0], y[1], s, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2], y[3], s, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4], y[5], s, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6], y[7], s, 3);
  return r;
}

// ---- Hadamard butterflies ---------------------------------------------------------
// In-lane stages of the fast Walsh-Hadamard transform over 8 values
// (butterfly distances 1, 2, 4): (a, b) -> (a + b, a - b).
__device__ __forceinline__ void fwht8_inlane(float (&y)[8]) {
#pragma unroll
  for (int h = 1; h < 8; h *= 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if ((j % (2 * h)) < h) {
        float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
}

// A butterfly stage whose two operands sit in partner lanes (CTRL swaps
// them).  The lower lane keeps a + b; the upper lane needs a - b, computed
// as partner + (-own), which IEEE defines to be the same value.
template <int CTRL>
__device__ __forceinline__ void fwht8_crosslane(float (&y)[8], bool upper) {
  const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // bound_ctrl + zero `old`: the move folds into v_add_f32_dpp
    const float partner =
        __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y[j]), CTRL, 0xF, 0xF, true));
    y[j] = partner + __uint_as_float(__float_as_uint(y[j]) ^ flip);
  }
}

}  // namespace mxq
