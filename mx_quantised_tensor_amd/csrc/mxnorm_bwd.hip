// mxnorm_bwd.hip -- gfx950 kernels of the straight-through MXNorm backward.
//
// Source: "MXNorm: Reusing MXFP block scales for efficient tensor
// normalisation" (gist.science summary), "Resumen tecnico" §2, the gradients
// item of "Implementacion": a straight-through estimator reusing RMSNorm's
// gradient, with no memory beyond what RMSNorm keeps.  Reading: the MX cast
// is passed straight through and the forward's rho stands in for rstd, so
// with g = dy * gamma
//     dx_j     = rho * g_j - rho^3 * x_j * (1/D) sum_k x_k g_k
//     dgamma_j = sum over rows of dy_j * x_j * rho.
// dx is evaluated as rho * (g_j - y_j * m), y = rho * x (the normalised row,
// |y| < 2 c K^(1/p)) and m = (1/D) sum_k y_k g_k: no intermediate overflows
// unless dx itself does (rho^3 alone overflows fp32 once rho > 2^42, e.g. for
// an all-zero row, whose rho is c * 2^(127 - emax)), and the products summed
// stay clear of fp32 subnormals for rows of tiny magnitude.
//
// Like the forward, this is an HBM-bound streaming pass (read x and dy, write
// dx: 6 bytes per element); no dense contraction, no MFMA.
//   * one wavefront owns a row at a time (up to hidden 2048 with a gain, 4096
//     without) with the same lane layout as the forward: lane `lane` holds
//     chunk s*64 + lane at step s;
//   * with a gain, waves are persistent over rows (row += total waves) so that
//     each lane accumulates its columns' dgamma in registers across many
//     rows, and each wave keeps the next row's loads in flight while it works
//     on the current one.  With one wave per row, 256 or 512 workgroups of 4
//     waves (more concurrent waves made this pattern slower: 8 waves per CU
//     +18%, 3 waves per SIMD +14%; 128 workgroups are too few; see
//     bwd_groups).  At the end the waves of a workgroup add their
//     accumulators through LDS in a fixed order and the workgroup writes one
//     partial row; a second kernel adds the partial rows column by column in
//     a fixed order.  Both orders depend only on (rows, hidden), so results
//     are run-to-run reproducible;
//   * without a gain every wave takes one row (four per workgroup) up to
//     hidden 2048; above that (up to 4096, but see the wide rows below) a row
//     is split over 2 waves (as in the forward: measured at 16384 x 4096,
//     64.3 against 66.3 us with one wave per row -- a wave's share of the
//     last rows' work is half as long), two rows per workgroup, and the last
//     4096 rows of a long launch over 4 waves each;
//   * rows of more waves (k_mxnorm_bwd_wide): lane `lane` of wave `wir` holds
//     chunk (s*W + wir)*64 + lane at step s, as in the wide forward; the W
//     wave sums of y.g are added through LDS in wave order.  With a gain,
//     rows of 2049 to 4096 elements take 3 to 8 waves of 1 or 2 steps, rows
//     of 4097 to 4608 2 waves of 8 steps, rows up to 8192 8 waves of 2 steps,
//     wider rows 4 waves (up to 16384) or 8 of as many steps (5 to 8) as the
//     width needs, over persistent workgroups, one or two per CU (see
//     gain_layout, bwd_groups); each wave
//     owns distinct columns, so it writes its part of the workgroup's
//     partial row directly.  Without a gain, rows of 3585 to 4096 elements
//     (in launches of 16384 rows or more) take 8 waves of 1 step, rows of
//     4097 to 8192 8 waves of 2 steps, wider rows 4 or 8 waves of 8 steps,
//     one row per workgroup.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "launch.h"
#include "mx_device.h"

namespace mxq {

namespace {

constexpr int kBwdThreads = 256;  // 4 waves per workgroup without a gain
constexpr int kColsumThreads = 256;
constexpr int kColsumCols = 32;    // columns per workgroup of the partial-row sum (128 B of a row)
constexpr int kColsumSlices = 32;  // partial rows b = slice + 32 k per thread
constexpr int kColsumLoads = (int)((kBwdMaxPartials + kColsumSlices - 1) / kColsumSlices);

constexpr int kBwdWaves = 4;  // waves per workgroup of the persistent (gain) kernel

typedef unsigned int u32x4b_t __attribute__((ext_vector_type(4)));
typedef float f32x2b_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2b_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt16(const uint8_t* p) {
  const u32x4b_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4b_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void store_nt16(uint8_t* p, uint32_t a, uint32_t b, uint32_t c,
                                           uint32_t d) {
  const u32x4b_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4b_t*>(p));
}

typedef float f32x4b_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt_f4(float* p, float a, float b, float c, float d) {
  const f32x4b_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4b_t*>(p));
}

__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  const f32x2b_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2b_t));
}

struct BwdArgs {
  const uint8_t* x;
  const uint8_t* dy;
  const uint8_t* gamma;  // nullptr: no gain, no dgamma
  const float* rrms;
  int64_t rows;
  int hidden;
  float inv_d;  // fl(1/hidden)
  uint8_t* dx;
  float* partial;  // [gridDim.x, hidden] when gamma != nullptr
};

template <int STEPS>
__device__ __forceinline__ void load_row(const BwdArgs& a, int64_t row, const uint32_t (&choff)[STEPS],
                                         uint4 (&xv)[STEPS], uint4 (&dv)[STEPS]) {
  const int64_t base = row * (int64_t)a.hidden * 2;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) xv[s] = load_nt16(a.x + base + choff[s]);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) dv[s] = load_nt16(a.dy + base + choff[s]);
}

// dx of one row (and its dgamma contribution added to acc).  W > 1: the row is
// shared by the W waves of the workgroup; s_dot (2 W floats, alternating
// halves by row parity `par`) carries their partial sums of y.g.
// The gain staged in LDS once per workgroup: widened to fp32 (F32: half h,
// elements 4h .. 4h+3, of 8-element chunk c at h * NCH + c, so that the lanes
// of a wave read consecutive 16-byte slots), which takes the widening out of
// both passes (8192 x 8192: 79.6 against 81.3 us), or as bf16 chunks for rows
// of more than 16384 (the fp32 copy would be 128 KiB: 92.7 against 91.5 us).
template <int NCH>
struct GainLds {
  static constexpr bool F32 = NCH <= 2048;
  // 16-byte slots: two per chunk as fp32, one per chunk as bf16
  static constexpr int kSlots = F32 ? 2 * NCH : NCH;
};

template <int NCH>
__device__ __forceinline__ void gain8(const float4* s_gf, uint32_t c, float (&g)[8]) {
  if constexpr (GainLds<NCH>::F32) {
    const float4 a = s_gf[c], b = s_gf[NCH + c];
    g[0] = a.x; g[1] = a.y; g[2] = a.z; g[3] = a.w;
    g[4] = b.x; g[5] = b.y; g[6] = b.z; g[7] = b.w;
  } else {
    widen8(reinterpret_cast<const uint4*>(s_gf)[c], g);
  }
}

// Stage the gain (chunks past the row end repeat the last one and are never
// used).
template <int NCH>
__device__ __forceinline__ void stage_gain(const BwdArgs& a, float4* s_gf, int nthreads) {
  const int nchunk = a.hidden >> 3;
  for (int c = threadIdx.x; c < NCH; c += nthreads) {
    const uint4 raw = *reinterpret_cast<const uint4*>(a.gamma + (uint32_t)min(c, nchunk - 1) * 16u);
    if constexpr (GainLds<NCH>::F32) {
      float f[8];
      widen8(raw, f);
      s_gf[c] = make_float4(f[0], f[1], f[2], f[3]);
      s_gf[NCH + c] = make_float4(f[4], f[5], f[6], f[7]);
    } else {
      reinterpret_cast<uint4*>(s_gf)[c] = raw;
    }
  }
  __syncthreads();
}

template <bool GAMMA, int STEPS, int W = 1>
__device__ __forceinline__ void bwd_row(const BwdArgs& a, int64_t row, int lane,
                                        const uint32_t (&choff)[STEPS], const bool (&act)[STEPS],
                                        const float4* s_gf, uint4 (&xv)[STEPS],
                                        uint4 (&dv)[STEPS], float (&acc)[GAMMA ? STEPS : 1][8],
                                        float* s_dot = nullptr, int wir = 0, int par = 0) {
  constexpr int NCH = STEPS * W * kWave;  // gain chunks staged
  // rho through the constant address space: a scalar load, so waiting for it
  // never waits for vector loads issued after this row's
  const float rho = ((const __attribute__((address_space(4))) float*)a.rrms)[row];

  // sum_k y_k g_k with y_k = fl(rho x_k), fp32: eight FMA chains per lane (one
  // per position in the 8-element chunk, over the lane's chunks in order, so
  // that a wave alone on its SIMD is not held by one 8 x STEPS-long dependent
  // chain), added in a fixed tree, then a fixed tree over the wave
  float dp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) dp[i] = 0.0f;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!act[s]) continue;
    float xf[8], g[8];
    widen8(xv[s], xf);
    widen8(dv[s], g);
    if constexpr (GAMMA) {
      float gf[8];
      gain8<NCH>(s_gf, choff[s] >> 4, gf);
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = g[i] * gf[i];  // exact: 8-bit x 8-bit significands
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) dp[i] = __builtin_fmaf(xf[i] * rho, g[i], dp[i]);
  }
  float dot = ((dp[0] + dp[1]) + (dp[2] + dp[3])) + ((dp[4] + dp[5]) + (dp[6] + dp[7]));
  dot = wave_sum_f32(dot);
  if constexpr (W > 1) {
    // The other half of s_dot is the next row's, and a wave rewrites this
    // half two rows later, after every wave has passed the next row's barrier
    // (and so has read this half).
    if (lane == 0) s_dot[par * W + wir] = dot;
    __syncthreads();
    dot = s_dot[par * W];
#pragma unroll
    for (int w = 1; w < W; ++w) dot += s_dot[par * W + w];
  }
  // Keep only the packed row across the reduction: the barrier stops the
  // compiler from holding the widened products of the first pass (64 more
  // VGPRs); the second pass widens again.
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
    __asm__ volatile("" : "+v"(xv[s].x), "+v"(xv[s].y), "+v"(xv[s].z), "+v"(xv[s].w),
                     "+v"(dv[s].x), "+v"(dv[s].y), "+v"(dv[s].z), "+v"(dv[s].w));
  const float m = dot * a.inv_d;  // mean of y g

  uint8_t* drow = a.dx + row * (int64_t)a.hidden * 2;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!act[s]) continue;
    float xf[8], dyf[8], d[8];
    widen8(xv[s], xf);
    widen8(dv[s], dyf);
    float gf[8];
    if constexpr (GAMMA) gain8<NCH>(s_gf, choff[s] >> 4, gf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float g = GAMMA ? dyf[i] * gf[i] : dyf[i];
      const float y = xf[i] * rho;
      d[i] = rho * __builtin_fmaf(-m, y, g);
      if constexpr (GAMMA) acc[s][i] = __builtin_fmaf(dyf[i], y, acc[s][i]);
    }
    store_nt16(drow + choff[s], bf16x2_rne(d[0], d[1]), bf16x2_rne(d[2], d[3]),
               bf16x2_rne(d[4], d[5]), bf16x2_rne(d[6], d[7]));
  }
}

template <bool GAMMA, int STEPS, bool FULL>
__global__ __launch_bounds__(GAMMA ? kBwdWaves * 64 : kBwdThreads) void k_mxnorm_bwd(
    const BwdArgs a) {
  constexpr int NW = GAMMA ? kBwdWaves : 4;  // waves per workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = a.hidden >> 3;
  uint32_t choff[STEPS];
  bool act[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = s * kWave + lane;
    act[s] = FULL || ch < nchunk;
    choff[s] = (uint32_t)(FULL ? ch : min(ch, nchunk - 1)) * 16u;
  }

  // the gain is widened once per workgroup into LDS (the kernel is persistent)
  __shared__ float4 s_gf[GAMMA ? GainLds<STEPS * kWave>::kSlots : 1];
  if constexpr (GAMMA) stage_gain<STEPS * kWave>(a, s_gf, NW * kWave);

  float acc[GAMMA ? STEPS : 1][8];
#pragma unroll
  for (int s = 0; s < (GAMMA ? STEPS : 1); ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[s][i] = 0.0f;

  const int64_t stride = (int64_t)gridDim.x * NW;
  int64_t row = (int64_t)blockIdx.x * NW + wave;
  if constexpr (GAMMA) {
    // Persistent waves keep the next row in flight while they work on this
    // one, alternating between two register sets (no copies, so nothing
    // waits for the next row before its turn).  The next row's loads are
    // issued before this row's stores, so waiting for them never waits for
    // those stores.  Past the last row the current row is loaded again
    // (harmless, unused).
    uint4 xa[STEPS], da[STEPS], xb[STEPS], db[STEPS];
    if (row < a.rows) load_row<STEPS>(a, row, choff, xa, da);
    while (row < a.rows) {
      const int64_t r1 = row + stride;
      load_row<STEPS>(a, r1 < a.rows ? r1 : row, choff, xb, db);
      bwd_row<GAMMA, STEPS>(a, row, lane, choff, act, s_gf, xa, da, acc);
      row = r1;
      if (row >= a.rows) break;
      const int64_t r2 = row + stride;
      load_row<STEPS>(a, r2 < a.rows ? r2 : row, choff, xa, da);
      bwd_row<GAMMA, STEPS>(a, row, lane, choff, act, s_gf, xb, db, acc);
      row = r2;
    }
  } else {
    if (row < a.rows) {  // one row per wave, as in the forward
      uint4 xv[STEPS], dv[STEPS];
      load_row<STEPS>(a, row, choff, xv, dv);
      bwd_row<GAMMA, STEPS>(a, row, lane, choff, act, s_gf, xv, dv, acc);
    }
  }

  if constexpr (GAMMA) {
    // workgroup partial of dgamma: (((w0 + w1) + w2) + ...), one step at a time
    __shared__ float4 s_red[NW][kWave * 2];
    float* prow = a.partial + (int64_t)blockIdx.x * a.hidden;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      s_red[wave][lane * 2] = make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
      s_red[wave][lane * 2 + 1] = make_float4(acc[s][4], acc[s][5], acc[s][6], acc[s][7]);
      __syncthreads();
      if (wave == 0 && act[s]) {
        float4 lo = s_red[0][lane * 2], hi = s_red[0][lane * 2 + 1];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
          const float4 l2 = s_red[w][lane * 2], h2 = s_red[w][lane * 2 + 1];
          lo.x += l2.x; lo.y += l2.y; lo.z += l2.z; lo.w += l2.w;
          hi.x += h2.x; hi.y += h2.y; hi.z += h2.z; hi.w += h2.w;
        }
        float4* dst = reinterpret_cast<float4*>(prow + (s * kWave + lane) * 8);
        dst[0] = lo;
        dst[1] = hi;
      }
      __syncthreads();
    }
  }
}

// Rows of up to 512 W STEPS elements: a workgroup of W waves owns one row at a
// time (STEPS chunks per lane): 4096 < hidden <= 4096 W with 8 steps, except
// rows of up to 8192 with 8 waves of 2 steps (with a gain those that nearly
// fill 8192), and with a gain rows that nearly fill 4096 with 8 waves of 1
// step; without a gain 2048 < hidden <= 4096 with 2 waves of 4 steps.
template <bool GAMMA, int W, bool FULL, int STEPS = 8>
__global__ __launch_bounds__(W * 64) void k_mxnorm_bwd_wide(const BwdArgs a) {
  const int lane = threadIdx.x & 63;
  const int wir = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = a.hidden >> 3;
  uint32_t choff[STEPS];
  bool act[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = (s * W + wir) * kWave + lane;
    act[s] = FULL || ch < nchunk;
    choff[s] = (uint32_t)(FULL ? ch : min(ch, nchunk - 1)) * 16u;
  }
  __shared__ float s_dot[2 * W];
  __shared__ float4 s_gf[GAMMA ? GainLds<STEPS * W * kWave>::kSlots : 1];
  if constexpr (GAMMA) stage_gain<STEPS * W * kWave>(a, s_gf, W * kWave);
  float acc[GAMMA ? STEPS : 1][8];
#pragma unroll
  for (int s = 0; s < (GAMMA ? STEPS : 1); ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[s][i] = 0.0f;

  const int64_t stride = gridDim.x;
  int64_t row = blockIdx.x;
  if constexpr (GAMMA && W == 8 && STEPS == 8) {
    // 8 waves per workgroup leave 256 registers per wave: one register set
    // (the other waves of the SIMD keep loads in flight)
    int par = 0;
    for (; row < a.rows; row += stride) {
      uint4 xv[STEPS], dv[STEPS];
      load_row<STEPS>(a, row, choff, xv, dv);
      bwd_row<GAMMA, STEPS, W>(a, row, lane, choff, act, s_gf, xv, dv, acc, s_dot, wir, par);
      par ^= 1;
    }
  } else if constexpr (GAMMA) {
    // as in k_mxnorm_bwd: two register sets, the next row's loads in flight
    uint4 xa[STEPS], da[STEPS], xb[STEPS], db[STEPS];
    int par = 0;
    if (row < a.rows) load_row<STEPS>(a, row, choff, xa, da);
    while (row < a.rows) {
      const int64_t r1 = row + stride;
      load_row<STEPS>(a, r1 < a.rows ? r1 : row, choff, xb, db);
      bwd_row<GAMMA, STEPS, W>(a, row, lane, choff, act, s_gf, xa, da, acc, s_dot, wir, par);
      par ^= 1;
      row = r1;
      if (row >= a.rows) break;
      const int64_t r2 = row + stride;
      load_row<STEPS>(a, r2 < a.rows ? r2 : row, choff, xa, da);
      bwd_row<GAMMA, STEPS, W>(a, row, lane, choff, act, s_gf, xb, db, acc, s_dot, wir, par);
      par ^= 1;
      row = r2;
    }
  }
  if constexpr (GAMMA) {
    // this wave's columns of the workgroup's partial row; rows of 8 waves of
    // 1 or 2 steps and rows of 4 waves store them non-temporally (measured on
    // MI355X: 16384 x 4096 66.8 against 67.4 us, 8192 x 8192 68.3 against
    // 68.9, 32768 x 4096 127.5 against 128.5, 4096 x 16384 77.3 against 78.0,
    // 4096 x 10240 49.3 against 49.6; with 3 waves, 8 waves of 5 to 8 steps or
    // one wave per row it was 0.5-2% slower)
    float* prow = a.partial + (int64_t)blockIdx.x * a.hidden;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (!act[s]) continue;
      float* dst = prow + (choff[s] >> 4) * 8;
      if constexpr ((W == 8 && STEPS <= 2) || W == 4) {
        store_nt_f4(dst, acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
        store_nt_f4(dst + 4, acc[s][4], acc[s][5], acc[s][6], acc[s][7]);
      } else {
        reinterpret_cast<float4*>(dst)[0] = make_float4(acc[s][0], acc[s][1], acc[s][2], acc[s][3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(acc[s][4], acc[s][5], acc[s][6], acc[s][7]);
      }
    }
  } else {
    if (row < a.rows) {
      uint4 xv[STEPS], dv[STEPS];
      load_row<STEPS>(a, row, choff, xv, dv);
      bwd_row<GAMMA, STEPS, W>(a, row, lane, choff, act, s_gf, xv, dv, acc, s_dot, wir, 0);
    }
  }
}

// Without a gain at 2048 < hidden <= 4096 (except long launches of rows near
// 4096, which take 8 waves per row): workgroups of 4 waves carrying two
// rows of 2 waves each, and, in launches of kBwdTailMinRows rows or more, the
// last kBwdTailRows rows one per workgroup of 4 waves, so that each wave of
// the launch's last dispatch round has half a row's work (measured against
// one row of 2 waves per 128-thread workgroup: 16384 x 4096 62.96 against
// 64.04 us, 32768 x 4096 125.7 against 128.8, 16384 x 3072 47.2 against
// 48.9).  The waves of an empty row slot (an odd head row count) join the
// row's barrier with no active chunk.
constexpr int64_t kBwdTailRows = 4096;
constexpr int64_t kBwdTailMinRows = 8192;

__global__ __launch_bounds__(kBwdThreads) void k_mxnorm_bwd_pairs(const BwdArgs a,
                                                                  int64_t head_blocks,
                                                                  int64_t tail_rows) {
  __shared__ float s_dot[8];  // head: 2 row slots x (2 parities x 2 waves); tail: 2 x 4
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nchunk = a.hidden >> 3;
  float acc[1][8];  // no dgamma
  const int64_t head_rows = a.rows - tail_rows;
  if ((int64_t)blockIdx.x >= head_blocks) {
    const int64_t row = head_rows + ((int64_t)blockIdx.x - head_blocks);
    uint32_t choff[2];
    bool act[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int ch = (s * 4 + wave) * kWave + lane;
      act[s] = ch < nchunk;
      choff[s] = (uint32_t)min(ch, nchunk - 1) * 16u;
    }
    uint4 xv[2], dv[2];
    load_row<2>(a, row, choff, xv, dv);
    bwd_row<false, 2, 4>(a, row, lane, choff, act, nullptr, xv, dv, acc, s_dot, wave, 0);
    return;
  }
  const int rslot = wave >> 1, wir = wave & 1;
  int64_t row = (int64_t)blockIdx.x * 2 + rslot;
  const bool ok = row < head_rows;
  if (!ok) row = 0;  // a valid row to read rho and x from; nothing is stored
  uint32_t choff[4];
  bool act[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int ch = (s * 2 + wir) * kWave + lane;
    act[s] = ok && ch < nchunk;
    choff[s] = (uint32_t)min(ch, nchunk - 1) * 16u;
  }
  uint4 xv[4], dv[4];
  load_row<4>(a, row, choff, xv, dv);
  bwd_row<false, 4, 2>(a, row, lane, choff, act, nullptr, xv, dv, acc, s_dot + rslot * 4, wir, 0);
}

// dgamma_j = sum over the G <= kBwdMaxPartials partial rows, in a fixed order.
// Thread (slice, q) of a workgroup loads the float4 of columns 4q..4q+3 of
// partial rows slice, slice + 32, ... (all loads issued before the adds; a
// load instruction reads full 128-byte lines of 8 partial rows) and adds them
// in that order; the 32 slice sums of a column are then added in four runs of
// 8 consecutive slices, and the four run sums in order.  (16 columns per
// workgroup read half lines: 2048 x 32768, 256 partial rows: 11.6 us.)
__global__ __launch_bounds__(kColsumThreads) void k_colsum(const float* __restrict__ partial,
                                                           int G, int hidden,
                                                           float* __restrict__ out) {
  __shared__ float s_part[kColsumSlices][kColsumCols];
  __shared__ float s_run[4][kColsumCols];
  const int q = threadIdx.x & 7;
  const int slice = threadIdx.x >> 3;
  const int col0 = blockIdx.x * kColsumCols + q * 4;  // hidden % 32 == 0: in range
  float4 v[kColsumLoads];
#pragma unroll
  for (int k = 0; k < kColsumLoads; ++k) {
    const int b = slice + k * kColsumSlices;
    v[k] = b < G ? *reinterpret_cast<const float4*>(partial + (int64_t)b * hidden + col0)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 acc = v[0];
#pragma unroll
  for (int k = 1; k < kColsumLoads; ++k) {
    acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
  }
  s_part[slice][q * 4 + 0] = acc.x;
  s_part[slice][q * 4 + 1] = acc.y;
  s_part[slice][q * 4 + 2] = acc.z;
  s_part[slice][q * 4 + 3] = acc.w;
  __syncthreads();
  if (threadIdx.x < 4 * kColsumCols) {
    const int c = threadIdx.x % kColsumCols, run = threadIdx.x / kColsumCols;
    constexpr int kRun = kColsumSlices / 4;
    float t = s_part[run * kRun][c];
#pragma unroll
    for (int i = 1; i < kRun; ++i) t += s_part[run * kRun + i][c];
    s_run[run][c] = t;
  }
  __syncthreads();
  if (threadIdx.x < kColsumCols) {
    const int c = threadIdx.x;
    out[blockIdx.x * kColsumCols + c] = ((s_run[0][c] + s_run[1][c]) + s_run[2][c]) + s_run[3][c];
  }
}

template <bool GAMMA, int STEPS>
hipError_t launch_bwd_t(const BwdArgs& a, int groups, void* stream) {
  const dim3 block(GAMMA ? kBwdWaves * 64 : kBwdThreads);
  if (a.hidden == 512 * STEPS)
    hipLaunchKernelGGL((k_mxnorm_bwd<GAMMA, STEPS, true>), dim3(groups), block, 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((k_mxnorm_bwd<GAMMA, STEPS, false>), dim3(groups), block, 0,
                       (hipStream_t)stream, a);
  return hipGetLastError();
}

template <bool GAMMA, int W, int STEPS = 8>
hipError_t launch_bwd_wide_t(const BwdArgs& a, int groups, void* stream) {
  if (a.hidden == 512 * STEPS * W)
    hipLaunchKernelGGL((k_mxnorm_bwd_wide<GAMMA, W, true, STEPS>), dim3(groups), dim3(W * 64), 0,
                       (hipStream_t)stream, a);
  else
    hipLaunchKernelGGL((k_mxnorm_bwd_wide<GAMMA, W, false, STEPS>), dim3(groups), dim3(W * 64),
                       0, (hipStream_t)stream, a);
  return hipGetLastError();
}

// Row layout of the backward with a gain: `waves` waves of `steps` chunks
// per lane own a row (1 wave: k_mxnorm_bwd, its steps set by the width; more:
// k_mxnorm_bwd_wide).  From 2049 to 4096 elements and from 4609 to 8192, few
// steps over many waves: a row's loads and its dot are spread over more
// waves, and the persistent workgroups (one or two per CU, see bwd_groups)
// keep 6 to 10 waves per CU.  Measured on MI355X (same-process A/B, the
// partial-row sum included) against one wave of 4 or 8 steps per row up to
// 4096 and 2 waves of 8 steps at 8192: 16384 x 2336 45.8 against 49.0 us,
// 16384 x 2560 46.3 against 50.6, 16384 x 3072 53.7 against 57.8 (6 waves
// of 1 step: 54.7), 16384 x 3584 60.7 against 65.3, 16384 x 3712 66.0
// against 67.4, 16384 x 4096 67.4 against 71.4, 8192 x 4096 36.6 against
// 41.2, 32768 x 4096 129.1 against 134.7, 8192 x 5120 50.5 against 51.2,
// 8192 x 6144 53.5 against 60.0, 8192 x 8192 69.0 against 76.9.  At 2048
// columns (4 waves of 1 step: +1.5-32%) and from 4097 to 4608 (8 waves of 2
// steps: +2.7%) the older layouts stay; a prefetch 2 or 3 rows ahead, 4
// waves of 2 steps at 8192 columns and 16 waves of 2 steps at 16384 measured
// slower or the same.  Above 8192 elements, 4 waves (up to 16384) or 8 of
// as many steps as the width needs (5 to 8) against 8 steps: 4096 x 10240
// 49.5 against 54.9 us, 4096 x 12288 58.7 against 61.9, 2048 x 20480 55.2
// against 59.7, 2048 x 24576 64.8 against 67.5 (without a gain the same fit
// measured 0.2-1% faster or 2.5% slower, so those rows keep 8 steps).
struct GainLayout {
  int waves, steps;
};
GainLayout gain_layout(int hidden) {
  if (hidden > 8192) {
    const int w = hidden > 16384 ? 8 : 4;
    return {w, (hidden / 8 + w * kWave - 1) / (w * kWave)};  // 5 to 8 steps
  }
  if (hidden > 4608) return {8, 2};
  if (hidden > 4096) return {2, 8};
  if (hidden > 3584) return {8, 1};
  if (hidden > 3072) return {7, 1};
  if (hidden > 2560) return {3, 2};
  if (hidden > 2048) return {5, 1};
  return {1, 0};
}

template <bool GAMMA>
hipError_t launch_bwd_steps(const BwdArgs& a, int groups, void* stream) {
  if constexpr (GAMMA) {
    const GainLayout gl = gain_layout(a.hidden);
    // {1, 0}, {2, 8}, {4, 8} and {8, 8} take the generic launches below
    switch (gl.waves * 16 + gl.steps) {
      case 5 * 16 + 1: return launch_bwd_wide_t<GAMMA, 5, 1>(a, groups, stream);
      case 3 * 16 + 2: return launch_bwd_wide_t<GAMMA, 3, 2>(a, groups, stream);
      case 7 * 16 + 1: return launch_bwd_wide_t<GAMMA, 7, 1>(a, groups, stream);
      case 8 * 16 + 1: return launch_bwd_wide_t<GAMMA, 8, 1>(a, groups, stream);
      case 8 * 16 + 2: return launch_bwd_wide_t<GAMMA, 8, 2>(a, groups, stream);
      case 4 * 16 + 5: return launch_bwd_wide_t<GAMMA, 4, 5>(a, groups, stream);
      case 4 * 16 + 6: return launch_bwd_wide_t<GAMMA, 4, 6>(a, groups, stream);
      case 4 * 16 + 7: return launch_bwd_wide_t<GAMMA, 4, 7>(a, groups, stream);
      case 8 * 16 + 5: return launch_bwd_wide_t<GAMMA, 8, 5>(a, groups, stream);
      case 8 * 16 + 6: return launch_bwd_wide_t<GAMMA, 8, 6>(a, groups, stream);
      case 8 * 16 + 7: return launch_bwd_wide_t<GAMMA, 8, 7>(a, groups, stream);
      default: break;
    }
  } else {
    // one row per 512-thread workgroup of 8 waves of 2 steps, measured on
    // MI355X against 2 waves of 8 steps: 8192 x 8192 61.5 against 64.8 us,
    // 8192 x 7168 54.8 against 58.3, 8192 x 4608 35.6 against 37.2 (4 waves
    // of 4 steps in between); at 16384 and 32768 columns more waves with
    // fewer steps measured the same or slower.  Rows that nearly fill 4096,
    // in launches of 16384 rows or more: 8 waves of 1 step (16384 x 4096
    // 62.1-62.4 against 62.9-63.0 us with k_mxnorm_bwd_pairs, 32768 rows the
    // same, 4 waves of 2 steps 63.4; at 8192 and 4096 rows the pairs are
    // 0.5-1.4% faster, and at 3072 columns 0.1%)
    if (a.hidden > 4096 && a.hidden <= 8192)
      return launch_bwd_wide_t<GAMMA, 8, 2>(a, groups, stream);
    if (a.hidden > 3584 && a.hidden <= 4096 && a.rows >= 16384)
      return launch_bwd_wide_t<GAMMA, 8, 1>(a, groups, stream);
  }
  if (a.hidden > 16384) return launch_bwd_wide_t<GAMMA, 8>(a, groups, stream);
  if (a.hidden > 8192) return launch_bwd_wide_t<GAMMA, 4>(a, groups, stream);
  if (a.hidden > 4096) return launch_bwd_wide_t<GAMMA, 2>(a, groups, stream);
  if constexpr (!GAMMA) {
    if (a.hidden > 2048) {
      const int64_t tail = a.rows >= kBwdTailMinRows ? kBwdTailRows : 0;
      const int64_t head_blocks = (a.rows - tail + 1) / 2;
      hipLaunchKernelGGL(k_mxnorm_bwd_pairs, dim3((unsigned)(head_blocks + tail)),
                         dim3(kBwdThreads), 0, (hipStream_t)stream, a, head_blocks, tail);
      return hipGetLastError();
    }
  }
  const int nchunk = a.hidden / 8;
  if (nchunk <= 64) return launch_bwd_t<GAMMA, 1>(a, groups, stream);
  if (nchunk <= 128) return launch_bwd_t<GAMMA, 2>(a, groups, stream);
  if (nchunk <= 256) return launch_bwd_t<GAMMA, 4>(a, groups, stream);
  return launch_bwd_t<GAMMA, 8>(a, groups, stream);
}

}  // namespace

// The allocation-free backward's workspace: the dgamma partial rows live in
// this array, which every GPU the library runs on holds until the process
// ends.  In host code its name is only a stand-in for the symbol, not a device
// address: kernels get the address hipGetSymbolAddress returns, looked up once
// per device with that device current.  Every partial row a launch reads is
// written by the same launch first, so nothing has to be cleared between calls.
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t bwd_scratch(int device, float** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_addr[device].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[device].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (addr == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<float*>(addr);
      g_scratch_addr[device].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

int64_t bwd_groups(int64_t rows, int hidden) {
  const int w = gain_layout(hidden).waves;
  if (w == 1) {
    // measured on MI355X with 4 waves per workgroup (the partial-row sum
    // included): rows of 512 or 1024 elements (1 or 2 chunks per lane, fewer
    // bytes in flight per wave) stream fastest with 512 workgroups (131072 x
    // 512: 68.5 against 101.5 us with 192; 65536 x 1024: 70.9 against 82.2),
    // rows of 2048 with 256 (16384 x 2048: 37.2 against 38.4); when rows of
    // 3072 and 4096 ran one wave per row, 216 (16384 x 3072: 57.9-58.2
    // against 60.4-60.9; 16384 x 4096: 71.8-72.0 against 72.6-73.2)
    const int nchunk = hidden / 8;
    const int64_t cap = nchunk <= 128 ? 512 : nchunk <= 256 ? 256 : 216;
    const int64_t need = (rows + kBwdWaves - 1) / kBwdWaves;
    return need < cap ? need : cap;
  }
  // measured on MI355X (the partial-row sum included): 512 workgroups (two
  // per CU) for 2, 3 and 5 waves per row, 256 (one per CU) for 4, 7 and 8
  // (16384 x 2560 with 5 waves: 46.3 against 52.2 us with 256; 16384 x 3072
  // with 3 waves: 53.7 against 61.1; 16384 x 3584 with 7 waves: 60.7 against
  // 64.4 with 512; 8 waves of 1 or 2 steps with 512: 16384 x 4096 72.4
  // against 67.6, 8192 x 8192 74.3 against 69.0, 32768 x 4096 143.2 against
  // 129.2)
  const int64_t cap = (w == 2 || w == 3 || w == 5) ? 512 : 256;
  return rows < cap ? rows : cap;
}

hipError_t launch_mxnorm_bwd(const BwdLaunch& l) {
  BwdArgs a;
  a.x = static_cast<const uint8_t*>(l.x);
  a.dy = static_cast<const uint8_t*>(l.dy);
  a.gamma = static_cast<const uint8_t*>(l.gamma);
  a.rrms = l.rrms;
  a.rows = l.rows;
  a.hidden = l.hidden;
  a.inv_d = 1.0f / (float)l.hidden;
  a.dx = static_cast<uint8_t*>(l.dx);
  a.partial = l.workspace;
  // with a gain the workgroups are persistent (one dgamma partial row each);
  // without one a row takes one wave up to hidden 2048 (four rows per
  // workgroup) and a workgroup of 2 or more waves above
  const int groups = (int)(l.gamma ? bwd_groups(l.rows, l.hidden)
                          : l.hidden <= 2048 ? (l.rows + 3) / 4 : l.rows);
  if (groups > 0) {
    const hipError_t e = l.gamma ? launch_bwd_steps<true>(a, groups, l.stream)
                                 : launch_bwd_steps<false>(a, groups, l.stream);
    if (e != hipSuccess) return e;
  }
  if (l.gamma == nullptr) return hipSuccess;
  hipLaunchKernelGGL(k_colsum, dim3((unsigned)(l.hidden / kColsumCols)), dim3(kColsumThreads), 0,
                     (hipStream_t)l.stream, l.workspace, groups, l.hidden, l.dgamma);
  return hipGetLastError();
}

}  // namespace mxq
