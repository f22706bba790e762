// mxnorm_kernels.hip -- gfx950 kernels of the MXNorm library and their launchers.
//
// Sources (by page title and section):
//   [P1] "MXNorm: Reusing MXFP block scales for efficient tensor
//        normalisation" (gist.science summary), "Resumen tecnico" §1-§3.
//   [P2] the same paper (gptget.net summary) with the authors' abstract.
//   [P3] MXFP4 pre-training on AMD MI355X (gist.science summary),
//        "Metodologia", "Hallazgos" 2 (deterministic H16 / H32 rotation).
//
// Every kernel here is a streaming codec bound by HBM bandwidth (the rotation
// kernels with their VALU work close behind): there is no dense contraction on
// this path, so no MFMA.  The design points are
//   * a lane owns 8 consecutive bf16 (one 16-byte load); a quad of lanes owns
//     a 32-element MX block, so block reductions are two quad DPP steps;
//   * one wavefront owns a whole row (hidden <= 2048, and rotated rows up to
//     4096) and keeps it in VGPRs between the row statistic and the cast --
//     one barrier (after the gain copy), at most 64 VGPRs, 8 waves per SIMD to
//     keep HBM requests in flight;
//   * wider rows are owned by 2, 4 or 8 waves, the two row reductions meeting
//     in LDS; at 2048 < hidden <= 4096 without rotation 2 waves per row
//     measured faster than one (16384 x 4096: 33.4 against 34.0 us; E2M1 27.7
//     against 28.9 us): a wave's cast is half as long, and the cast of the
//     rows that arrive last is what the launch waits for at its end (with H16
//     one wave per row stays faster); for the same reason the last 2048 rows
//     of an E4M3 launch of 8192 rows or more are cast by 4 waves each (at
//     2048 columns, rows otherwise one per wave, the last 1536);
//   * x is loaded and the codes stored non-temporally (each byte is touched
//     once); the gain comes from L2, staged once per workgroup in LDS (by
//     LDS-DMA loads as bf16, or widened to fp32 where that measured faster);
//   * workgroups keep the hardware's round-robin spread over the 8 XCDs, so
//     the whole chip sweeps one contiguous region of HBM at a time (giving
//     each XCD its own contiguous range of rows measured ~5% slower).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"
#include "mx_device.h"

namespace mxq {

constexpr int kThreads = 256;     // 4 waves per workgroup
constexpr int kInactive = -256;   // block exponent of a lane past the row end

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

// ---- streaming memory access ----------------------------------------------------
#define MXQ_LDS __attribute__((address_space(3)))
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Raw buffer over `bytes` bytes at p (stride 0): loads at or past `bytes`
// read as zero.
__device__ __forceinline__ rsrc_t row_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 load_stream16(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int ELEM>
__device__ __forceinline__ void store_codes_stream(uint8_t* __restrict__ dst, const float (&y)[8],
                                                   uint32_t e8m0) {
  if constexpr (ELEM == 0) {
    const uint2 c = encode8_e4m3(y, e8m0);
    const u32x2_t v = {c.x, c.y};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(dst));
  } else {
    __builtin_nontemporal_store(encode8_e2m1(y, e8m0), reinterpret_cast<uint32_t*>(dst));
  }
}

// ---- the MXNorm row statistic ([P1] §2 "Formula"; [P2] abstract) -----------------
// Two readings of the block magnitude mt_k (SRC):
//   kSrcScales: mt_k = 2^(e_k + emax), e_k the E8M0 exponent the MX cast of x
//     gives block k.  From the bf16 exponent field f of the block absmax,
//     u = e_k + emax + 127 = max(f, emax) (the E8M0 clamp at -127 included).
//   kSrcAbsmax: mt_k = the block absmax m_k itself = M_k * 2^(u - 134) with
//     u = max(f, 1) and the 8-bit integer M_k = f ? 128 + fraction : fraction.
// u = 255 marks a block holding NaN or Inf.
constexpr int kSrcScales = 0;
constexpr int kSrcAbsmax = 1;

// m: the lane's largest 15-bit magnitude pattern (bf16 bits of |x|), before
// the quad maximum.
template <int SRC, int EMAX>
__device__ __forceinline__ int block_u_from(uint32_t m, int& mp, int p_shift) {
  m = quad_max_u32(m);
  const int f = (int)(m >> 7);
  if constexpr (SRC == kSrcScales) {
    (void)p_shift;
    mp = 1;
    return max(f, EMAX);
  } else {
    const int M = (int)(m & 0x7F) | (f != 0 ? 0x80 : 0);
    mp = p_shift ? M * M : M;
    return max(f, 1);
  }
}

// The lane's 8 values either as packed bf16 (the 15-bit magnitudes come from
// the bit patterns) or already widened to fp32 (the magnitude of the largest
// |x|, an exact bf16 value, is the top half of its fp32 pattern: v_maximum3
// with |.| modifiers, 4 instructions instead of 8 on the packed words; NaN and
// Inf keep exponent field 255).
__device__ __forceinline__ uint32_t lane_mag(const uint4 v) { return absmax8_bf16_bits(v); }
__device__ __forceinline__ uint32_t lane_mag(const float (&x)[8]) {
  return absmax8_f32_bits(x) >> 16;
}

// The terms of the exact power sum, as doubles built from their exponent:
//   kSrcScales: S = sum_k 2^(40 - t_k), t_k = p (E1 - u_k) <= 40;
//   kSrcAbsmax: S = sum_k M_k^p 2^(24 - t_k), t_k <= 24.
// The double whose high word is (1023 + W - t) << 20 (low word 0) is 2^(W - t);
// M_k^p < 2^16, so every term is exact, and S < 2^53 (K <= 1024): summing the
// terms in fp64 is exact in any order.
template <int SRC>
struct PowerSum {
  static constexpr int kW = SRC == kSrcScales ? 40 : 24;
  int hbase;  // ((1023 + W) << 20) - (E1 << pk)
  int umin;   // E1 - W/p
  int pk;     // 20 + (p - 1): (p (E1 - u)) << 20 == (E1 - u) << pk for p in {1, 2}
  __device__ __forceinline__ PowerSum(int E1, int p_shift) {
    pk = 20 + p_shift;
    hbase = ((1023 + kW) << 20) - (E1 << pk);
    umin = E1 - (kW >> p_shift);
  }
  __device__ __forceinline__ double term(int u, int mp) const {
    const double pw = __hiloint2double(u >= umin ? hbase + (u << pk) : 0, 0);
    if constexpr (SRC == kSrcScales) {
      (void)mp;
      return pw;
    } else {
      return pw * (double)mp;
    }
  }
};

// rho = fl(c / r) * 2^shift, r = fl(fl(S)/K) (p = 1) or fl(sqrt(fl(fl(S)/K))),
// shift = 40/p - (E1 - 127) (kSrcScales) or 24/p + 7 - (E1 - 127) (kSrcAbsmax).
// Each step is one correctly rounded fp32 operation.  fl(S/K) is evaluated
// as S * (1/K) in fp64 and rounded once: the product is within 2^-53 of S/K
// (1/K exact or correctly rounded), and a 24-bit S divided by K <= 2^10 is
// never within 2^-52 of a float rounding boundary.  The square root and the
// division are IEEE fp32 operations (the library is built with correctly
// rounded fp32 divide and sqrt): shorter dependent chains than their fp64
// forms, which the rows that arrive last in a launch wait on.  E1 == 255
// (NaN/Inf in the row) gives NaN; S == 0 (an all-zero row, absmax reading)
// gives +Inf.
template <int SRC>
__device__ __forceinline__ float rho_from_stat(int E1, double S, int p_shift, float c,
                                               double inv_k) {
  if (E1 >= 255) return __uint_as_float(0x7FC00000u);
  const float Sf = (float)S;  // exact in fp64 below 2^53; one rounding here
  const float mu = (float)((double)Sf * inv_k);
  const float r = p_shift == 0 ? mu : sqrtf(mu);
  const float q = c / r;
  const int shift = SRC == kSrcScales ? (40 >> p_shift) - (E1 - 127)
                                      : (24 >> p_shift) + 7 - (E1 - 127);
  return (float)ldexp((double)q, shift);
}

// ---- normalise (+gain), rotate, re-derive the block scale from y, cast ----------
// ([P1] §2 "Implementacion": scale the values and produce the quantisation
// scales in the same pass; [P3]: H16 / H32 rotation before the MXFP4 cast.)
template <int ELEM, bool GAMMA, int HAD>
__device__ __forceinline__ uint32_t cast_chunk(const float (&x)[8], const float (&g)[8], float rho,
                                               int lane, uint8_t* __restrict__ dst) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = x[i] * rho;
  if constexpr (GAMMA) {
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
  store_codes_stream<ELEM>(dst, y, sb);
  return sb;
}

// ----------------------------------------------------------------------------------
// MXNorm forward, one wave per row (hidden <= 512 * STEPS <= 4096), four rows
// per workgroup.  Lane `lane` owns chunk s*64 + lane of the row at step s.
// ----------------------------------------------------------------------------------
struct WaveArgs {
  const uint8_t* x;
  const uint8_t* gamma;
  int64_t rows;
  int hidden;
  int p_shift;   // p - 1
  float c;
  double inv_k;  // 1 / K
  uint8_t* codes;
  uint8_t* scales;
  float* rrms;
  int scales_dwords;  // K % 4 == 0 and scales 4-byte aligned
  int64_t head_blocks;  // k_mxnorm_wide, k_mxnorm_wave_tail: workgroups before the tail part
  int64_t tail_rows;    // the same kernels: rows of the tail part (at the end)
};

// Rows of up to 4 chunks per lane are widened to fp32 once, before the row
// statistic, and kept (32 VGPRs at 4 chunks); with 8 chunks per lane the
// statistic reads the packed words and the cast widens them.
template <int STEPS>
struct RowRegs {
  static constexpr bool kWiden = STEPS <= 4;
  float xf[kWiden ? STEPS : 1][8];
  __device__ __forceinline__ void widen(const uint4 (&v)[STEPS]) {
    if constexpr (kWiden) {
#pragma unroll
      for (int s = 0; s < STEPS; ++s) widen8(v[s], xf[s]);
    }
  }
  __device__ __forceinline__ uint32_t mag(const uint4 (&v)[STEPS], int s) const {
    if constexpr (kWiden) return lane_mag(xf[s]);
    else return lane_mag(v[s]);
  }
  __device__ __forceinline__ void values(const uint4 (&v)[STEPS], int s, float (&out)[8]) const {
    if constexpr (kWiden) {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = xf[s][i];
    } else {
      widen8(v[s], out);
    }
  }
};

// The whole forward of one row held in VGPRs (v: the row; s_gain: the gain,
// staged in LDS, chunk s * 64 + lane at index s * 64 + lane).
// How k_mxnorm_wave stages the gain in LDS: rows of 4 or 8 chunks per lane
// widen it to fp32 once per workgroup (half h, elements 4h .. 4h+3, of chunk c
// at h * NCH + c, so that the lanes of a wave read consecutive 16-byte slots),
// which takes 8 widening instructions per chunk out of the cast (8192 x 2048:
// 10.20 against 10.35 us); shorter rows keep the bf16 copy by LDS-DMA, whose
// shorter path to LDS is what the small, latency-bound launches need (256 x
// 768: 2.15 against 2.26 us).
template <int STEPS>
struct WaveGain {
  static constexpr bool F32 = STEPS >= 4;
  static constexpr int kSlots = F32 ? 2 * STEPS * kWave : STEPS * kWave;  // 16-byte slots
};

template <int ELEM, bool GAMMA, int HAD, int STEPS, bool FULL, int SRC>
__device__ __forceinline__ void wave_row(const WaveArgs& a, int64_t row, int lane,
                                         const bool (&act)[STEPS], const uint4 (&v)[STEPS],
                                         const float4* s_gain, uint32_t* __restrict__ s_sc) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  constexpr int CB = Elem<ELEM>::kCodeBytesPerLane;
  const int K = a.hidden >> 5;
  RowRegs<STEPS> rr;
  rr.widen(v);
  int u[STEPS], mp[STEPS];
  int umax = kInactive;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    int us = block_u_from<SRC, EMAX>(rr.mag(v, s), mp[s], a.p_shift);
    if constexpr (!FULL) us = act[s] ? us : kInactive;
    u[s] = us;
    umax = max(umax, us);
  }
  const int E1 = wave_max_quads(umax);

  float rho;
  {
    const PowerSum<SRC> ps(E1, a.p_shift);
    double S = 0.0;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) S += ps.term(u[s], mp[s]);
    S = wave_sum_quads_f64(S);
    rho = rho_from_stat<SRC>(E1, S, a.p_shift, a.c, a.inv_k);
  }
  if (a.rrms != nullptr && lane == 0) a.rrms[row] = rho;

  uint8_t* crow = a.codes + row * (int64_t)(ELEM == 0 ? a.hidden : a.hidden / 2);
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!FULL && !act[s]) continue;  // quad-uniform; the DPP inside stays in the quad
    float x[8], gf[8];
    rr.values(v, s, x);
    if constexpr (GAMMA && WaveGain<STEPS>::F32) {
      const float4 g0 = s_gain[s * kWave + lane], g1 = s_gain[STEPS * kWave + s * kWave + lane];
      gf[0] = g0.x; gf[1] = g0.y; gf[2] = g0.z; gf[3] = g0.w;
      gf[4] = g1.x; gf[5] = g1.y; gf[6] = g1.z; gf[7] = g1.w;
    } else if constexpr (GAMMA) {
      widen8(reinterpret_cast<const uint4*>(s_gain)[s * kWave + lane], gf);
    }
    const uint32_t sb = cast_chunk<ELEM, GAMMA, HAD>(
        x, gf, rho, lane, crow + (uint32_t)(s * kWave + lane) * (uint32_t)CB);
    reinterpret_cast<uint8_t*>(s_sc)[s * 16 + (lane >> 2)] = (uint8_t)sb;
  }
  // the scale bytes written above are read back by other lanes of the wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint8_t* srow = a.scales + row * K;
  if (a.scales_dwords) {  // K / 4 <= STEPS * 4 <= 32 dwords: one store per lane
    if (lane < (K >> 2)) reinterpret_cast<uint32_t*>(srow)[lane] = s_sc[lane];
  } else {
#pragma unroll
    for (int j = 0; j < (STEPS * 16 + kWave - 1) / kWave; ++j) {
      const int i = j * kWave + lane;
      if (i < K) srow[i] = reinterpret_cast<const uint8_t*>(s_sc)[i];
    }
  }
}

template <int STEPS, bool FULL>
__device__ __forceinline__ void lane_chunks(int lane, int nchunk, bool (&act)[STEPS],
                                            uint32_t (&choff)[STEPS]) {
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = s * kWave + lane;
    act[s] = FULL || ch < nchunk;  // uniform over each quad (nchunk % 4 == 0)
    choff[s] = (uint32_t)(FULL ? ch : min(ch, nchunk - 1)) * 16u;  // clamped: stays in the row
  }
}

// The gain is staged once per workgroup in LDS by gfx950's LDS-DMA buffer loads
// (no VGPRs: 53 instead of 78 at hidden 4096, so 8 waves per SIMD instead of
// 6, and a quarter of the gain's L2 reads), issued ahead of the row loads; one
// barrier after they land.  Measured against requesting the whole gain into
// VGPRs per wave, when this kernel still served 16384 x 4096 without rotation:
// 34.0 against 34.6 us; H16 -> E2M1 at 32768 x 4096: 60.9 against 62.6 us.
// Workgroup blk: rows 4 blk .. 4 blk + 3 of those below rlim.
template <int ELEM, bool GAMMA, int HAD, int STEPS, bool FULL, int SRC>
__device__ __forceinline__ void wave_rows(const WaveArgs& a, int64_t blk, int64_t rlim) {
  constexpr int NCH = STEPS * kWave;  // chunk slots of a row
  constexpr bool GF32 = WaveGain<STEPS>::F32;
  __shared__ uint32_t s_sc[4][STEPS * 4];  // the row's scale bytes, per wave
  __shared__ float4 s_gain[GAMMA ? WaveGain<STEPS>::kSlots : 1];  // layout: WaveGain
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blk * 4 + wave;
  const bool row_ok = row < rlim;  // waves past the end still stage the gain and meet the barrier

  uint32_t choff[STEPS];  // byte offset of the lane's chunk (32-bit: SGPR row base)
  bool act[STEPS];
  lane_chunks<STEPS, FULL>(lane, a.hidden >> 3, act, choff);
  constexpr int kGainPerThread = (NCH + kThreads - 1) / kThreads;
  uint4 graw[GAMMA && GF32 ? kGainPerThread : 1];
  if constexpr (GAMMA && GF32) {
    // thread i loads chunks i, i + 256 of the gain (chunks past the row end
    // repeat the last one and are never used)
    const int last = (a.hidden >> 3) - 1;
#pragma unroll
    for (int j = 0; j < kGainPerThread; ++j) {
      const int c = j * kThreads + (int)threadIdx.x;
      graw[j] = reinterpret_cast<const uint4*>(a.gamma)[min(c, last)];
    }
  } else if constexpr (GAMMA) {
    // wave w copies steps w, w + 4 of the gain by LDS-DMA; chunks past the
    // row end read as zero (buffer range) and are never used
    const rsrc_t rg = row_rsrc(a.gamma, (uint32_t)a.hidden * 2u);
#pragma unroll
    for (int j = 0; j < (STEPS + 3) / 4; ++j) {
      const int s = j * 4 + wave;
      if (s < STEPS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rg, (MXQ_LDS void*)((MXQ_LDS uint8_t*)s_gain + s * kWave * 16), 16,
            (int)((uint32_t)(s * kWave + lane) * 16u), 0, 0, 0);
    }
  }
  // The gain loads stay ahead of the row loads (the LDS-DMA wait below counts
  // on that order).
  if constexpr (GAMMA) asm volatile("" ::: "memory");
  const uint8_t* xrow = a.x + (row_ok ? row : 0) * (int64_t)a.hidden * 2;
  uint4 v[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) v[s] = load_stream16(xrow + choff[s]);
  if constexpr (GAMMA && GF32) {
#pragma unroll
    for (int j = 0; j < kGainPerThread; ++j) {
      const int c = j * kThreads + (int)threadIdx.x;
      if (c < NCH) {
        float f[8];
        widen8(graw[j], f);
        s_gain[c] = make_float4(f[0], f[1], f[2], f[3]);
        s_gain[NCH + c] = make_float4(f[4], f[5], f[6], f[7]);
      }
    }
    __syncthreads();
  } else if constexpr (GAMMA) {
    // the copies were issued before the STEPS row loads: at most STEPS loads
    // outstanding means the copies have landed
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(STEPS) : "memory");
    __syncthreads();
  }
  if (!row_ok) return;  // whole wave, after the only barrier
  wave_row<ELEM, GAMMA, HAD, STEPS, FULL, SRC>(a, row, lane, act, v, s_gain, s_sc[wave]);
}

template <int ELEM, bool GAMMA, int HAD, int STEPS, bool FULL, int SRC>
__global__ __launch_bounds__(kThreads) void k_mxnorm_wave(const WaveArgs a) {
  wave_rows<ELEM, GAMMA, HAD, STEPS, FULL, SRC>(a, blockIdx.x, a.rows);
}

// ----------------------------------------------------------------------------------
// MXNorm forward with a rotation ([P3] "Metodologia") on rows of exactly 4096,
// a lane owning whole 16-element groups, so stages h = 1, 2, 4, 8 of the
// transform run in-lane (and for H32 only h = 16 crosses lanes).  The
// butterflies are the same operations in the same order as in k_mxnorm_wave,
// so the results are identical.  Two ways to get the groups into lanes:
//   * EXCH = false: group g = t * 64 + lane at step t, two 16-byte loads 16
//     bytes apart; an MX block is the lane pair (l, l ^ 1);
//   * EXCH = true: contiguous 1 KiB loads of chunks t*128 + lane and
//     t*128 + 64 + lane, then partner lanes (l, l ^ 1) swap halves by DPP on
//     the packed bf16 words: even lane 2m holds group t*64 + m, odd lane
//     2m + 1 group t*64 + 32 + m; an MX block is the lane pair (l, l ^ 2).
// Measured on 32768 x 4096 against one wave per row with 8-element chunks:
// H32 -> E2M1 63.2 against 69.7 us and H32 -> E4M3 73.0 against 76.0 us with
// EXCH = false (EXCH = true: 64.3 us); H16 with gain -> E2M1 60.1 against
// 61.3 us and -> E4M3 66.2 against 68.9 us with EXCH = true (EXCH = false: no
// faster), but H16 without gain 60.8 against 59.7 us: H32 runs here with
// EXCH = false, H16 with a gain with EXCH = true, H16 without one does not.
// ----------------------------------------------------------------------------------
template <int ELEM, bool GAMMA, int HAD, bool EXCH>
__global__ __launch_bounds__(kThreads) void k_mxnorm_group16(const WaveArgs a) {
  constexpr int kHidden = 4096;
  constexpr int T = kHidden / (16 * kWave);  // groups per lane
  constexpr int K = kHidden / 32;
  constexpr int NG = kHidden / 16;           // 16-element groups per row
  constexpr int EMAX = Elem<ELEM>::kEmax;
  static_assert(HAD == 16 || HAD == 32, "rotation size");
  __shared__ uint32_t s_sc[4][K / 4];  // each wave's scale bytes
  // The gain is widened to fp32 once per workgroup and staged in LDS, quarter
  // q of group g (elements 4q .. 4q+3) at q * NG + g, so that the lanes of a
  // wave read consecutive 16-byte slots (no bank conflicts); against bf16 in
  // LDS this takes 16 widening instructions per group out of the cast, which
  // these VALU-bound kernels pay for (workload 5: 58.4 against 59.9 us).
  __shared__ float4 s_gainf[GAMMA ? kHidden / 4 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool row_ok = row < a.rows;  // waves past the end still stage the gain and meet the barrier
  uint4 graw[GAMMA ? kHidden / 8 / kThreads : 1];
  if constexpr (GAMMA) {
    // thread i loads 8-element chunks i and i + 256 (group c / 2, half c % 2)
#pragma unroll
    for (int j = 0; j < kHidden / 8 / kThreads; ++j)
      graw[j] = reinterpret_cast<const uint4*>(a.gamma)[j * kThreads + threadIdx.x];
  }
  if constexpr (GAMMA) asm volatile("" ::: "memory");  // keep the gain loads ahead of the row loads
  // DPP control reaching the lane that holds the other group of the lane's MX
  // block, and the one reaching the quad's other block
  constexpr int kBlk = EXCH ? kDppQuadSwap2 : kDppQuadSwap1;
  constexpr int kQuad = EXCH ? kDppQuadSwap1 : kDppQuadSwap2;
  const int blk_bit = EXCH ? 2 : 1;  // lane bit telling the block's upper group
  const bool even = (lane & 1) == 0;
  const uint8_t* xrow = a.x + (row_ok ? row : 0) * (int64_t)(kHidden * 2);
  uint4 v[2 * T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if constexpr (EXCH) {
      v[2 * t] = load_stream16(xrow + (uint32_t)(t * 2 * kWave + lane) * 16u);
      v[2 * t + 1] = load_stream16(xrow + (uint32_t)(t * 2 * kWave + kWave + lane) * 16u);
    } else {
      const uint32_t off = (uint32_t)(t * kWave + lane) * 32u;
      // cached loads: the pair of 16-byte loads 16 bytes apart touches each
      // line twice (measured 2% faster than non-temporal loads for H32)
      v[2 * t] = *reinterpret_cast<const uint4*>(xrow + off);
      v[2 * t + 1] = *reinterpret_cast<const uint4*>(xrow + off + 16u);
    }
  }
  if constexpr (GAMMA) {
#pragma unroll
    for (int j = 0; j < kHidden / 8 / kThreads; ++j) {
      const int c = j * kThreads + threadIdx.x;
      float f[8];
      widen8(graw[j], f);
      const int q = 2 * (c & 1);
      s_gainf[q * NG + (c >> 1)] = make_float4(f[0], f[1], f[2], f[3]);
      s_gainf[(q + 1) * NG + (c >> 1)] = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
  }
  if (!row_ok) return;  // whole wave, after the only barrier
  if constexpr (EXCH) {
    // even lane: keeps chunk A (group t*64 + m, first half), takes the odd
    // partner's A (second half); odd lane: keeps B (group t*64 + 32 + m,
    // second half), takes the even partner's B (first half)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint4 A = v[2 * t], B = v[2 * t + 1];
      const uint4 snd = even ? B : A;
      uint4 rcv;
      rcv.x = dpp_u32<kDppQuadSwap1>(snd.x);
      rcv.y = dpp_u32<kDppQuadSwap1>(snd.y);
      rcv.z = dpp_u32<kDppQuadSwap1>(snd.z);
      rcv.w = dpp_u32<kDppQuadSwap1>(snd.w);
      v[2 * t] = even ? A : rcv;
      v[2 * t + 1] = even ? rcv : B;
    }
  }

  // block exponents (the E8M0 scales of x): the pair's two 16-element halves
  int u[T];
  int umax = kInactive;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    uint32_t m = max(absmax8_bf16_bits(v[2 * t]), absmax8_bf16_bits(v[2 * t + 1]));
    m = max(m, dpp0_u32<kBlk>(m));
    u[t] = max((int)(m >> 7), EMAX);
    umax = max(umax, u[t]);
  }
  umax = max(umax, (int)dpp0_u32<kQuad>((uint32_t)umax));  // quad-uniform
  const int E1 = wave_max_quads(umax);
  float rho;
  {
    const PowerSum<kSrcScales> ps(E1, a.p_shift);
    double S = 0.0;
#pragma unroll
    for (int t = 0; t < T; ++t) S += ps.term(u[t], 1);
    if (lane & blk_bit) S = 0.0;  // a block is held by a lane pair: count it once
    S += dpp_f64<kQuad>(S);  // the quad's two blocks (exact: integer-valued terms)
    S = wave_sum_quads_f64(S);
    rho = rho_from_stat<kSrcScales>(E1, S, a.p_shift, a.c, a.inv_k);
  }
  if (a.rrms != nullptr && lane == 0) a.rrms[row] = rho;

  uint8_t* crow = a.codes + row * (int64_t)(ELEM == 0 ? kHidden : kHidden / 2);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int g = EXCH ? t * kWave + (lane >> 1) + (even ? 0 : kWave / 2) : t * kWave + lane;
    float lo[8], hi[8];  // elements 0..7 and 8..15 of the group
    widen8(v[2 * t], lo);
    widen8(v[2 * t + 1], hi);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = lo[i] * rho;
      hi[i] = hi[i] * rho;
    }
    if constexpr (GAMMA) {
      float g0[8], g1[8];
      const float4 q0 = s_gainf[g], q1 = s_gainf[NG + g];
      const float4 q2 = s_gainf[2 * NG + g], q3 = s_gainf[3 * NG + g];
      g0[0] = q0.x; g0[1] = q0.y; g0[2] = q0.z; g0[3] = q0.w;
      g0[4] = q1.x; g0[5] = q1.y; g0[6] = q1.z; g0[7] = q1.w;
      g1[0] = q2.x; g1[1] = q2.y; g1[2] = q2.z; g1[3] = q2.w;
      g1[4] = q3.x; g1[5] = q3.y; g1[6] = q3.z; g1[7] = q3.w;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lo[i] = lo[i] * g0[i];
        hi[i] = hi[i] * g1[i];
      }
    }
    fwht8_inlane(lo);  // h = 1, 2, 4 within each half
    fwht8_inlane(hi);
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // h = 8 across the halves
      const float p = lo[j], q = hi[j];
      lo[j] = p + q;
      hi[j] = p - q;
    }
    if constexpr (HAD == 32) {  // h = 16 with the lane holding the block's other group
      fwht8_crosslane<kBlk>(lo, (lane & blk_bit) != 0);
      fwht8_crosslane<kBlk>(hi, (lane & blk_bit) != 0);
    }
    constexpr float norm = HAD == 16 ? 0.25f : 0x1.6a09e6p-3f;  // fl32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo[i] = lo[i] * norm;
      hi[i] = hi[i] * norm;
    }
    uint32_t mb = max(absmax8_f32_bits(lo), absmax8_f32_bits(hi));
    mb = max(mb, dpp0_u32<kBlk>(mb));
    const uint32_t sb = e8m0_from_expfield<EMAX>(mb >> 23);
    if constexpr (ELEM == 0) {
      const uint2 c0 = encode8_e4m3(lo, sb), c1 = encode8_e4m3(hi, sb);
      const u32x4_t o = {c0.x, c0.y, c1.x, c1.y};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(crow + (uint32_t)g * 16u));
    } else {
      const u32x2_t o = {encode8_e2m1(lo, sb), encode8_e2m1(hi, sb)};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(crow + (uint32_t)g * 8u));
    }
    if (!(lane & blk_bit)) reinterpret_cast<uint8_t*>(s_sc[wave])[g >> 1] = (uint8_t)sb;
  }
  // the scale bytes written above are read back by other lanes of the wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint8_t* srow = a.scales + row * K;
  if (a.scales_dwords) {
    if (lane < K / 4) reinterpret_cast<uint32_t*>(srow)[lane] = s_sc[wave][lane];
  } else {
#pragma unroll
    for (int j = 0; j < K / kWave; ++j)
      srow[j * kWave + lane] = reinterpret_cast<const uint8_t*>(s_sc[wave])[j * kWave + lane];
  }
}

// ----------------------------------------------------------------------------------
// MXNorm forward with a rotation ([P3] "Metodologia") then E2M1 on rows of
// exactly 4096, a lane owning whole 32-element groups: group g = t*64 + lane at
// step t (four 16-byte loads 16 bytes apart, cached, so the lines they share
// are fetched once), which is one MX block, so every stage of the H32
// transform (and of H16 on each half) runs in-lane and the block maxima need no
// cross-lane step; its 16 code bytes are one 16-byte store.  Against
// 16-element groups per lane this drops the cross-lane stage of H32 (a sign
// flip and a DPP add per value) and the block pairs' DPP steps -- these
// kernels are VALU-bound (H32 -> E2M1 with a gain: 863 against 977 VALU
// instructions per row; 32768 x 4096: 59.1 against 62.3 us; H16 without a
// gain 59.1 against 60.7 us).  With E4M3 codes (32 bytes per lane, two strided
// stores) it measured slower (H16 -> E4M3: 73.5 against 66.4 us), so E4M3
// keeps k_mxnorm_group16.  The butterflies are the same operations in the
// same order, so the results are identical.  The gain is staged once per
// workgroup as fp32, eighth e of group g (elements 4e .. 4e+3) at e * 128 + g,
// so a wave's gain reads are consecutive 16-byte slots.
// ----------------------------------------------------------------------------------
template <bool GAMMA, int HAD>
__global__ __launch_bounds__(kThreads) void k_mxnorm_lane32(const WaveArgs a) {
  constexpr int kHidden = 4096;
  constexpr int T = kHidden / (32 * kWave);  // 32-groups (MX blocks) per lane
  constexpr int K = kHidden / 32;
  constexpr int EMAX = Elem<1>::kEmax;
  static_assert(HAD == 16 || HAD == 32, "rotation size");
  __shared__ uint32_t s_sc[4][K / 4];  // each wave's scale bytes
  __shared__ float4 s_gainf[GAMMA ? kHidden / 4 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  const bool row_ok = row < a.rows;  // waves past the end still stage the gain and meet the barrier
  uint4 graw[GAMMA ? kHidden / 8 / kThreads : 1];
  if constexpr (GAMMA) {
    // thread i loads 8-element chunks i and i + 256 (group c / 4, eighths
    // 2 (c % 4) and 2 (c % 4) + 1)
#pragma unroll
    for (int j = 0; j < kHidden / 8 / kThreads; ++j)
      graw[j] = reinterpret_cast<const uint4*>(a.gamma)[j * kThreads + threadIdx.x];
    asm volatile("" ::: "memory");  // keep the gain loads ahead of the row loads
  }
  const uint8_t* xrow = a.x + (row_ok ? row : 0) * (int64_t)(kHidden * 2);
  uint4 v[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[t][i] = *reinterpret_cast<const uint4*>(xrow + (uint32_t)((t * kWave + lane) * 64 + i * 16));
  if constexpr (GAMMA) {
#pragma unroll
    for (int j = 0; j < kHidden / 8 / kThreads; ++j) {
      const int c = j * kThreads + threadIdx.x;
      float f[8];
      widen8(graw[j], f);
      const int e = 2 * (c & 3);
      s_gainf[e * (K) + (c >> 2)] = make_float4(f[0], f[1], f[2], f[3]);
      s_gainf[(e + 1) * (K) + (c >> 2)] = make_float4(f[4], f[5], f[6], f[7]);
    }
    __syncthreads();
  }
  if (!row_ok) return;  // whole wave, after the only barrier

  // block exponents (the E8M0 scales of x), one block per lane and step
  int u[T];
  int umax = kInactive;
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const uint32_t m = max(max(absmax8_bf16_bits(v[t][0]), absmax8_bf16_bits(v[t][1])),
                           max(absmax8_bf16_bits(v[t][2]), absmax8_bf16_bits(v[t][3])));
    u[t] = max((int)(m >> 7), EMAX);
    umax = max(umax, u[t]);
  }
  umax = max(umax, (int)dpp0_u32<kDppQuadSwap1>((uint32_t)umax));
  umax = max(umax, (int)dpp0_u32<kDppQuadSwap2>((uint32_t)umax));  // quad-uniform
  const int E1 = wave_max_quads(umax);
  float rho;
  {
    const PowerSum<kSrcScales> ps(E1, a.p_shift);
    double S = 0.0;
#pragma unroll
    for (int t = 0; t < T; ++t) S += ps.term(u[t], 1);
    S += dpp_f64<kDppQuadSwap1>(S);  // exact: integer-valued terms
    S += dpp_f64<kDppQuadSwap2>(S);
    S = wave_sum_quads_f64(S);
    rho = rho_from_stat<kSrcScales>(E1, S, a.p_shift, a.c, a.inv_k);
  }
  if (a.rrms != nullptr && lane == 0) a.rrms[row] = rho;

  uint8_t* crow = a.codes + row * (int64_t)(kHidden / 2);
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int g = t * kWave + lane;
    float y[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[8];
      widen8(v[t][i], f);
#pragma unroll
      for (int k = 0; k < 8; ++k) y[8 * i + k] = f[k] * rho;
    }
    if constexpr (GAMMA) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float4 q = s_gainf[e * K + g];
        y[4 * e] = y[4 * e] * q.x;
        y[4 * e + 1] = y[4 * e + 1] * q.y;
        y[4 * e + 2] = y[4 * e + 2] * q.z;
        y[4 * e + 3] = y[4 * e + 3] * q.w;
      }
    }
    // butterfly distances 1, 2, 4, 8 (each 16-element half), then 16 for H32
#pragma unroll
    for (int h = 1; h < HAD; h *= 2) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if ((j % (2 * h)) < h) {
          const float p = y[j], q = y[j + h];
          y[j] = p + q;
          y[j + h] = p - q;
        }
      }
    }
    constexpr float norm = HAD == 16 ? 0.25f : 0x1.6a09e6p-3f;  // fl32(1/sqrt(32))
#pragma unroll
    for (int i = 0; i < 32; ++i) y[i] = y[i] * norm;
    float m8[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) m8[i][k] = y[8 * i + k];
    const uint32_t mb = max(max(absmax8_f32_bits(m8[0]), absmax8_f32_bits(m8[1])),
                            max(absmax8_f32_bits(m8[2]), absmax8_f32_bits(m8[3])));
    const uint32_t sb = e8m0_from_expfield<EMAX>(mb >> 23);
    const u32x4_t o = {encode8_e2m1(m8[0], sb), encode8_e2m1(m8[1], sb),
                       encode8_e2m1(m8[2], sb), encode8_e2m1(m8[3], sb)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(crow + (uint32_t)g * 16u));
    reinterpret_cast<uint8_t*>(s_sc[wave])[g] = (uint8_t)sb;
  }
  // the scale bytes written above are read back by other lanes of the wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint8_t* srow = a.scales + row * K;
  if (a.scales_dwords) {
    if (lane < K / 4) reinterpret_cast<uint32_t*>(srow)[lane] = s_sc[wave][lane];
  } else {
#pragma unroll
    for (int j = 0; j < K / kWave; ++j)
      srow[j * kWave + lane] = reinterpret_cast<const uint8_t*>(s_sc[wave])[j * kWave + lane];
  }
}

// ----------------------------------------------------------------------------------
// MXNorm forward with a row owned by W waves (4/W rows per workgroup): 2048 <
// hidden <= 4096 without rotation, and 4096 < hidden <= 32768; the two row
// reductions cross waves through LDS.  Lane `lane` of wave `wir` owns chunk
// (wir*STEPS + s)*64 + lane at step s: each wave streams its own contiguous
// part of the row (measured 0.6-1.4% faster at 8192 and 32768 than waves
// interleaving 1 KiB steps, the same at 4096).
//
// The rows of workgroup `blk` of this part are row0 + blk * RPW + rslot, those
// below `rlim` valid.  LDS: s_max, s_sum [NW], s_sc [NW * STEPS * 4] (each
// wave's scale bytes, 16 per step), s_gain [W * STEPS * 64] (the row's gain,
// chunk c at c).
// ----------------------------------------------------------------------------------
template <int ELEM, bool GAMMA, int HAD, int W, int STEPS, int SRC>
__device__ __forceinline__ void wide_rows(const WaveArgs& a, int64_t blk, int64_t row0,
                                          int64_t rlim, int* s_max, double* s_sum,
                                          uint32_t* s_sc, uint4* s_gain) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  constexpr int CB = Elem<ELEM>::kCodeBytesPerLane;
  constexpr int NW = W > 4 ? W : 4;  // waves per workgroup
  constexpr int RPW = NW / W;        // rows per workgroup
  static_assert(W == 2 || W == 4 || W == 8, "waves per row");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rslot = wave / W;
  const int wir = wave % W;
  const int64_t row = row0 + blk * RPW + rslot;
  const bool row_ok = row < rlim;  // waves past the end still join the barriers
  const int nchunk = a.hidden >> 3;
  const int K = a.hidden >> 5;
  uint32_t* const wsc = s_sc + wave * STEPS * 4;

  // The gain is staged in LDS by LDS-DMA loads issued ahead of the row loads
  // (wave w copies chunk groups w, w + NW, ...; chunks past the row end read
  // as zero and are never used); they have landed once the row has, before
  // the statistic's first barrier.
  if constexpr (GAMMA) {
    const rsrc_t rg = row_rsrc(a.gamma, (uint32_t)a.hidden * 2u);
#pragma unroll
    for (int j = 0; j < (W * STEPS + NW - 1) / NW; ++j) {
      const int grp = j * NW + wave;  // W STEPS groups of 64 chunks in all
      if ((W * STEPS) % NW == 0 || grp < W * STEPS)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rg, (MXQ_LDS void*)((MXQ_LDS uint8_t*)s_gain + grp * kWave * 16), 16,
            (int)((uint32_t)(grp * kWave + lane) * 16u), 0, 0, 0);
    }
  }
  const uint8_t* xrow = a.x + (row_ok ? row : 0) * (int64_t)a.hidden * 2;
  uint4 v[STEPS];
  bool act[STEPS];
  uint32_t choff[STEPS];
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = (wir * STEPS + s) * kWave + lane;
    act[s] = row_ok && ch < nchunk;
    choff[s] = (uint32_t)min(ch, nchunk - 1) * 16u;
    v[s] = load_stream16(xrow + choff[s]);
  }

  RowRegs<STEPS> rr;
  rr.widen(v);
  int u[STEPS], mp[STEPS];
  int umax = kInactive;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int us = block_u_from<SRC, EMAX>(rr.mag(v, s), mp[s], a.p_shift);
    u[s] = act[s] ? us : kInactive;
    umax = max(umax, u[s]);
  }
  umax = wave_max_quads(umax);
  if (lane == 0) s_max[wave] = umax;
  if constexpr (GAMMA) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the gain copies
  __syncthreads();
  int E1 = s_max[rslot * W];
#pragma unroll
  for (int w = 1; w < W; ++w) E1 = max(E1, s_max[rslot * W + w]);

  const PowerSum<SRC> ps(E1, a.p_shift);
  double S = 0.0;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) S += ps.term(u[s], mp[s]);
  S = wave_sum_quads_f64(S);
  if (lane == 0) s_sum[wave] = S;
  __syncthreads();
  S = s_sum[rslot * W];
#pragma unroll
  for (int w = 1; w < W; ++w) S += s_sum[rslot * W + w];
  const float rho = rho_from_stat<SRC>(E1, S, a.p_shift, a.c, a.inv_k);
  if (a.rrms != nullptr && row_ok && wir == 0 && lane == 0) a.rrms[row] = rho;

  uint8_t* crow = a.codes + row * (int64_t)(ELEM == 0 ? a.hidden : a.hidden / 2);
  uint8_t* srow = a.scales + row * K;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    if (!act[s]) continue;  // quad-uniform
    const int ch = (wir * STEPS + s) * kWave + lane;
    float x[8], gf[8];
    rr.values(v, s, x);
    if constexpr (GAMMA) widen8(s_gain[ch], gf);
    const uint32_t sb = cast_chunk<ELEM, GAMMA, HAD>(x, gf, rho, lane,
                                                     crow + (uint32_t)ch * (uint32_t)CB);
    reinterpret_cast<uint8_t*>(wsc)[s * 16 + (lane >> 2)] = (uint8_t)sb;
  }
  // Step s of this wave covers blocks (wir STEPS + s) * 16 .. + 15 of the row: 16
  // scale bytes gathered in LDS, written as four dwords (or bytes when the
  // row's scales are not dword-aligned).  Other lanes of the wave read them.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (a.scales_dwords) {
    const int s = lane >> 2, q = lane & 3;  // step, dword within the step
    if (s < STEPS && row_ok) {
      const int b0 = (wir * STEPS + s) * 16;  // first block of the step
      if (b0 + 4 * q < K) reinterpret_cast<uint32_t*>(srow + b0)[q] = wsc[s * 4 + q];
    }
  } else {
#pragma unroll
    for (int j = 0; j < (STEPS * 16 + kWave - 1) / kWave; ++j) {
      const int i = j * kWave + lane;  // byte i of this wave's gathered scales
      const int s = i >> 4;
      const int blk = (wir * STEPS + s) * 16 + (i & 15);
      if (s < STEPS && row_ok && blk < K)
        srow[blk] = reinterpret_cast<const uint8_t*>(wsc)[i];
    }
  }
}


// Rows per launch that k_mxnorm_wide<2 waves, 4 to 8 steps> hands, at the end
// of the grid, to workgroups owning one row with 4 waves of half as many steps
// (E4M3 only).  The launch ends on the row statistic and cast of the rows
// whose data arrive last; in the last dispatch round each wave then casts half
// as much.  Measured at hidden 4096, E4M3 with gain: 8192 rows 17.91 against
// 18.52 us, 16384 rows 32.99 against 33.54 us, 32768 rows 63.73 against 64.37
// us, 65536 rows within noise; E2M1 (a shorter cast per element) was slower.
// 8192 rows of 4608 to 8192 elements: 20.4-20.6 against 21.0 us at 4608,
// 22.3-22.5 against 23.0 at 5120, 26.3-26.4 against 27.0-27.1 at 6144,
// 30.5-30.6 against 31.2-31.3 at 7168, 33.9-34.0 against 34.8 at 8192
// (16384 rows: 0.5-1% faster); 3-step rows (2049 to 3072 elements) gained
// nothing at 3072 and lost 1.4-2.5% at 2336 and 2560, so they keep none.
constexpr int64_t kWideTailRows = 2048;
constexpr int64_t kWideTailMinRows = 8192;

template <int ELEM, bool GAMMA, int HAD, int W, int STEPS, int SRC>
__global__ __launch_bounds__((W > 4 ? W : 4) * kWave) void k_mxnorm_wide(const WaveArgs a) {
  constexpr int NW = W > 4 ? W : 4;
  constexpr bool kTail = ELEM == 0 && W == 2 && STEPS >= 4;
  constexpr int TS = (STEPS + 1) / 2;  // steps per lane of the tail part's 4 waves
  constexpr int kGainSlots = kTail && 4 * TS > W * STEPS ? 4 * TS * kWave : W * STEPS * kWave;
  __shared__ int s_max[NW];
  __shared__ double s_sum[NW];
  __shared__ uint32_t s_sc[NW * STEPS * 4];  // the tail part's NW * TS * 4 fit
  __shared__ uint4 s_gain[GAMMA ? kGainSlots : 1];
  if constexpr (kTail) {
    // the tail part: 4 waves of (STEPS + 1) / 2 steps over the same row width
    if ((int64_t)blockIdx.x >= a.head_blocks) {
      wide_rows<ELEM, GAMMA, HAD, 4, TS, SRC>(a, (int64_t)blockIdx.x - a.head_blocks,
                                            a.rows - a.tail_rows, a.rows, s_max, s_sum, s_sc,
                                            s_gain);
      return;
    }
  }
  wide_rows<ELEM, GAMMA, HAD, W, STEPS, SRC>(a, blockIdx.x, 0, a.rows - a.tail_rows, s_max,
                                            s_sum, s_sc, s_gain);
}

// Rows of 2048 elements to E4M3 without rotation, in launches of
// kWaveTailMinRows rows or more: k_mxnorm_wave's one wave per row (4 chunks
// per lane), except for the last kWaveTailRows rows, each owned by a workgroup
// of 4 waves (1 chunk per lane).  At 8192 rows every wave of the launch is
// resident at once, and the launch ends on the statistic and cast of the rows
// whose data arrive last, the last ones dispatched; there each wave then
// casts a quarter as much.  Measured (same-process A/B, E4M3 with gain):
// 8192 x 2048 9.77 against 10.15 us (without gain 9.74-9.85 against 10.05),
// 16384 x 2048 17.53 against 17.86 us; tails of 768 and 2048 rows gained
// less, 2 waves per tail row nothing, and at 4096 rows the tail was slower.
constexpr int64_t kWaveTailRows = 1536;
constexpr int64_t kWaveTailMinRows = 8192;

template <int ELEM, bool GAMMA, int SRC>
__global__ __launch_bounds__(kThreads) void k_mxnorm_wave_tail(const WaveArgs a) {
  if ((int64_t)blockIdx.x >= a.head_blocks) {
    __shared__ int s_max[4];
    __shared__ double s_sum[4];
    __shared__ uint32_t s_sc[4 * 4];
    __shared__ uint4 s_gain[GAMMA ? 4 * kWave : 1];
    wide_rows<ELEM, GAMMA, 0, 4, 1, SRC>(a, (int64_t)blockIdx.x - a.head_blocks,
                                        a.rows - a.tail_rows, a.rows, s_max, s_sum, s_sc, s_gain);
    return;
  }
  wave_rows<ELEM, GAMMA, 0, 4, true, SRC>(a, blockIdx.x, a.rows - a.tail_rows);
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
  const int64_t ch = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (ch >= nchunks) return;  // nchunks % 4 == 0: quads stay whole
  float y[8];
  widen8(x[ch], y);
  const uint32_t m = quad_max_u32(lane_mag(y));
  const uint32_t sb = e8m0_from_expfield<EMAX>(m >> 7);
  store_codes_stream<ELEM>(codes + ch * Elem<ELEM>::kCodeBytesPerLane, y, sb);
  if ((threadIdx.x & 3) == 0) scales[ch >> 2] = (uint8_t)sb;
}

// The same cast of fl32(w * gamma[column]) ([P1] §2 "Implementacion",
// MXNormLinear: the gain folded into the weights of the next linear layer).
// A product of two bf16 values is exact in fp32.
template <int ELEM>
__global__ __launch_bounds__(kThreads) void k_mx_quant_gain(const uint4* __restrict__ w,
                                                             const uint4* __restrict__ gamma,
                                                             int64_t nchunks, int row_chunks,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  constexpr int EMAX = Elem<ELEM>::kEmax;
  const int64_t ch = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (ch >= nchunks) return;
  float y[8], g[8];
  widen8(w[ch], y);
  widen8(gamma[ch % row_chunks], g);
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = y[i] * g[i];
  const uint32_t mb = quad_max_u32(absmax8_f32_bits(y));
  const uint32_t sb = e8m0_from_expfield<EMAX>(mb >> 23);
  store_codes_stream<ELEM>(codes + ch * Elem<ELEM>::kCodeBytesPerLane, y, sb);
  if ((threadIdx.x & 3) == 0) scales[ch >> 2] = (uint8_t)sb;
}

// ----------------------------------------------------------------------------------
// RMSNorm, pass 1 of the two-pass baseline ([P1] §1): full-width fp32 sum of
// squares, rstd = 1/sqrt(mean + eps), bf16 y written to memory.  Same row
// layout as the MXNorm kernels (W waves per row); y is stored with ordinary
// stores so that pass 2 may find it in the Infinity Cache.
// ----------------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));  // RNE
}

template <bool GAMMA, int W, int STEPS>
__global__ __launch_bounds__(kThreads) void k_rmsnorm(const uint8_t* __restrict__ x,
                                                       const uint8_t* __restrict__ gamma,
                                                       int64_t rows, int hidden, float eps,
                                                       uint4* __restrict__ y,
                                                       float* __restrict__ rstd) {
  constexpr int RPW = 4 / W;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rslot = wave / W;
  const int wir = wave % W;
  const int64_t row = (int64_t)blockIdx.x * RPW + rslot;
  const bool row_ok = row < rows;
  if constexpr (W == 1) {
    if (!row_ok) return;  // whole wave; no barriers when a wave owns its row
  }
  const int nchunk = hidden >> 3;

  const uint8_t* xrow = x + (row_ok ? row : 0) * (int64_t)hidden * 2;
  uint4 v[STEPS], gr[GAMMA ? STEPS : 1];
  bool act[STEPS];
  uint32_t choff[STEPS];
  float ss = 0.0f;
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    const int ch = (s * W + wir) * kWave + lane;
    act[s] = row_ok && ch < nchunk;
    choff[s] = (uint32_t)min(ch, nchunk - 1) * 16u;
    v[s] = load_stream16(xrow + choff[s]);
  }
  if constexpr (GAMMA) {
#pragma unroll
    for (int s = 0; s < STEPS; ++s) gr[s] = *reinterpret_cast<const uint4*>(gamma + choff[s]);
  } else {
    gr[0] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    float f[8];
    widen8(v[s], f);
    if (act[s]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(f[i], f[i], ss);
    }
  }
  ss = wave_sum_f32(ss);
  if constexpr (W > 1) {
    __shared__ float s_sum[4];
    if (lane == 0) s_sum[wave] = ss;
    __syncthreads();
    ss = s_sum[rslot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) ss += s_sum[rslot * W + w];
  }
  const float rs = 1.0f / __builtin_sqrtf(ss / (float)hidden + eps);
  if (rstd != nullptr && row_ok && wir == 0 && lane == 0) rstd[row] = rs;

  uint4* yrow = y + row * (int64_t)nchunk;
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
      widen8(gr[s], g);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * g[i];
    }
    yrow[ch] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
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

WaveArgs wave_args(const MxnormArgs& m) {
  WaveArgs a;
  a.x = static_cast<const uint8_t*>(m.x);
  a.gamma = static_cast<const uint8_t*>(m.gamma);
  a.rows = m.rows;
  a.hidden = m.hidden;
  a.p_shift = m.p - 1;
  a.c = m.c;
  a.inv_k = 1.0 / (double)(m.hidden / 32);
  a.codes = m.codes;
  a.scales = m.scales;
  a.rrms = m.rrms;
  a.scales_dwords = ((m.hidden / 32) % 4 == 0) && (((uintptr_t)m.scales & 3) == 0);
  a.head_blocks = 0;
  a.tail_rows = 0;
  return a;
}

template <int ELEM, bool GAMMA, int HAD, int SRC, int STEPS>
hipError_t launch_wave(const MxnormArgs& m) {
  WaveArgs a = wave_args(m);
  if constexpr (ELEM == 0 && HAD == 0 && STEPS == 4) {
    if (m.hidden == 512 * STEPS && m.rows >= kWaveTailMinRows) {
      a.tail_rows = kWaveTailRows;
      a.head_blocks = (m.rows - a.tail_rows + 3) / 4;
      hipLaunchKernelGGL((k_mxnorm_wave_tail<ELEM, GAMMA, SRC>),
                         dim3((unsigned)(a.head_blocks + a.tail_rows)), dim3(kThreads), 0,
                         (hipStream_t)m.stream, a);
      return hipGetLastError();
    }
  }
  const dim3 grid((unsigned)((m.rows + 3) / 4));
  if (m.hidden == 512 * STEPS)
    hipLaunchKernelGGL((k_mxnorm_wave<ELEM, GAMMA, HAD, STEPS, true, SRC>), grid,
                       dim3(kThreads), 0, (hipStream_t)m.stream, a);
  else
    hipLaunchKernelGGL((k_mxnorm_wave<ELEM, GAMMA, HAD, STEPS, false, SRC>), grid,
                       dim3(kThreads), 0, (hipStream_t)m.stream, a);
  return hipGetLastError();
}

template <int ELEM, bool GAMMA, int HAD, int SRC, int W, int STEPS>
hipError_t launch_wide(const MxnormArgs& m) {
  WaveArgs a = wave_args(m);
  constexpr int NW = W > 4 ? W : 4, RPW = NW / W;
  a.tail_rows = (ELEM == 0 && W == 2 && STEPS >= 4 && m.rows >= kWideTailMinRows) ? kWideTailRows : 0;
  a.head_blocks = (m.rows - a.tail_rows + RPW - 1) / RPW;
  const dim3 grid((unsigned)(a.head_blocks + a.tail_rows));
  hipLaunchKernelGGL((k_mxnorm_wide<ELEM, GAMMA, HAD, W, STEPS, SRC>), grid, dim3(NW * kWave),
                     0, (hipStream_t)m.stream, a);
  return hipGetLastError();
}

template <int ELEM, bool GAMMA, int HAD, bool EXCH>
hipError_t launch_group16(const MxnormArgs& m) {
  const WaveArgs a = wave_args(m);
  const dim3 grid((unsigned)((m.rows + 3) / 4));
  hipLaunchKernelGGL((k_mxnorm_group16<ELEM, GAMMA, HAD, EXCH>), grid, dim3(kThreads), 0,
                     (hipStream_t)m.stream, a);
  return hipGetLastError();
}

template <bool GAMMA, int HAD>
hipError_t launch_lane32(const MxnormArgs& m) {
  const WaveArgs a = wave_args(m);
  const dim3 grid((unsigned)((m.rows + 3) / 4));
  hipLaunchKernelGGL((k_mxnorm_lane32<GAMMA, HAD>), grid, dim3(kThreads), 0,
                     (hipStream_t)m.stream, a);
  return hipGetLastError();
}

template <int ELEM, bool GAMMA, int HAD, int SRC>
hipError_t launch_mxnorm_shape(const MxnormArgs& m) {
  const RowShape r = pick_row_shape(m.hidden);
  if (r.waves == 1 && r.steps == 1) return launch_wave<ELEM, GAMMA, HAD, SRC, 1>(m);
  if (r.waves == 1 && r.steps == 2) return launch_wave<ELEM, GAMMA, HAD, SRC, 2>(m);
  if (r.waves == 1 && r.steps == 4) return launch_wave<ELEM, GAMMA, HAD, SRC, 4>(m);
  if (r.waves == 1 && r.steps == 8) {
    // 2048 < hidden <= 4096: 2 waves per row of 3 or 4 steps (as many as
    // the width needs), except with a rotation (its longer cast per element
    // runs faster one wave per row); on rows of exactly 4096, E2M1 rotations
    // with a whole 32-group per lane, H32 and H16 with a gain to E4M3 with
    // whole 16-groups per lane
    if constexpr (HAD == 0) {
      if (m.hidden <= 3072) return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 3>(m);
      return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 4>(m);
    } else {
      if constexpr (SRC == kSrcScales && ELEM == 1) {
        if (m.hidden == 4096) return launch_lane32<GAMMA, HAD>(m);
      }
      if constexpr (SRC == kSrcScales && (HAD == 32 || GAMMA)) {
        if (m.hidden == 4096) return launch_group16<ELEM, GAMMA, HAD, HAD == 16>(m);
      }
      return launch_wave<ELEM, GAMMA, HAD, SRC, 8>(m);
    }
  }
  if (r.waves == 2 && r.steps == 8) {
    // 4096 < hidden <= 8192: 2 waves of as many steps as the width needs (a
    // lane's chunks past the row end still cost their clamped loads and
    // masks).  Measured against 8 steps (and 4 at 2048 < hidden <= 3072), E4M3
    // with gain: 8192 x 4608 21.0 against 21.9 us, 8192 x 5120 23.0 against
    // 23.8, 8192 x 6144 27.1 against 27.5, 8192 x 7168 31.2 against 31.5,
    // 16384 x 2336 21.8 against 22.5, 16384 x 2560 22.2 against 22.8, 16384 x
    // 3072 25.6 against 25.9 (E2M1 21.6 against 22.1); H16 -> E2M1 at 8192 x
    // 6144 25.1 against 26.1
    switch ((m.hidden / 8 + 2 * kWave - 1) / (2 * kWave)) {
      case 5: return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 5>(m);
      case 6: return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 6>(m);
      case 7: return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 7>(m);
      default: return launch_wide<ELEM, GAMMA, HAD, SRC, 2, 8>(m);
    }
  }
  // wider rows likewise: 8192 < hidden <= 16384 on 4 waves of 5 to 8 steps
  // (4096 x 10240 24.1 against 26.1 us with 8 steps, 4096 x 12288 28.3
  // against 28.9); the table's 4 x 16 entry (rows above 16384) on 8 waves of
  // 5 to 8 steps, one 512-thread workgroup per row (half the registers per
  // wave of 4 x 16, and 3% faster at 32768 elements with gain; 2048 x 20480
  // 24.8 against 29.4 us with 8 steps, 2048 x 24576 29.1 against 31.2)
  if (r.waves == 4 && r.steps == 8) {
    switch ((m.hidden / 8 + 4 * kWave - 1) / (4 * kWave)) {
      case 5: return launch_wide<ELEM, GAMMA, HAD, SRC, 4, 5>(m);
      case 6: return launch_wide<ELEM, GAMMA, HAD, SRC, 4, 6>(m);
      case 7: return launch_wide<ELEM, GAMMA, HAD, SRC, 4, 7>(m);
      default: return launch_wide<ELEM, GAMMA, HAD, SRC, 4, 8>(m);
    }
  }
  if (r.waves == 4 && r.steps == 16) {
    switch ((m.hidden / 8 + 8 * kWave - 1) / (8 * kWave)) {
      case 5: return launch_wide<ELEM, GAMMA, HAD, SRC, 8, 5>(m);
      case 6: return launch_wide<ELEM, GAMMA, HAD, SRC, 8, 6>(m);
      case 7: return launch_wide<ELEM, GAMMA, HAD, SRC, 8, 7>(m);
      default: return launch_wide<ELEM, GAMMA, HAD, SRC, 8, 8>(m);
    }
  }
  return hipErrorInvalidValue;
}

template <int ELEM, bool GAMMA, int HAD>
hipError_t launch_mxnorm_src(const MxnormArgs& m) {
  return m.source == kSrcScales ? launch_mxnorm_shape<ELEM, GAMMA, HAD, kSrcScales>(m)
                                : launch_mxnorm_shape<ELEM, GAMMA, HAD, kSrcAbsmax>(m);
}

template <int ELEM, bool GAMMA>
hipError_t launch_mxnorm_had(const MxnormArgs& m) {
  switch (m.had) {
    case 0: return launch_mxnorm_src<ELEM, GAMMA, 0>(m);
    case 16: return launch_mxnorm_src<ELEM, GAMMA, 16>(m);
    case 32: return launch_mxnorm_src<ELEM, GAMMA, 32>(m);
    default: return hipErrorInvalidValue;
  }
}

template <bool GAMMA, int W, int STEPS>
hipError_t launch_rmsnorm_t(const void* x, const void* gamma, int64_t rows, int hidden,
                            float eps, void* y, float* rstd, void* stream) {
  const int64_t rpw = 4 / W;
  const int64_t grid = (rows + rpw - 1) / rpw;
  hipLaunchKernelGGL((k_rmsnorm<GAMMA, W, STEPS>), dim3((unsigned)grid), dim3(kThreads), 0,
                     (hipStream_t)stream, static_cast<const uint8_t*>(x),
                     static_cast<const uint8_t*>(gamma), rows, hidden, eps,
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
  // 2048 < hidden <= 4096: 2 waves per row, as in the MXNorm forward (the
  // baseline gets the same launch shape: 16384 x 4096, 72.4 against 74.1 us
  // for the two passes)
  if (r.waves == 1 && r.steps == 8)
    return launch_rmsnorm_t<GAMMA, 2, 4>(x, gamma, rows, hidden, eps, y, rstd, stream);
  MXQ_RMS(1, 1) MXQ_RMS(1, 2) MXQ_RMS(1, 4) MXQ_RMS(2, 8) MXQ_RMS(4, 8)
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

hipError_t launch_mx_quant_gain(const void* w, const void* gamma, int64_t rows, int hidden,
                                int elem, uint8_t* codes, uint8_t* scales, void* stream) {
  const int64_t nchunks = rows * (int64_t)(hidden / 8);
  const int64_t grid = (nchunks + kThreads - 1) / kThreads;
  if (elem == 0)
    hipLaunchKernelGGL(k_mx_quant_gain<0>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, static_cast<const uint4*>(w),
                       static_cast<const uint4*>(gamma), nchunks, hidden / 8, codes, scales);
  else
    hipLaunchKernelGGL(k_mx_quant_gain<1>, dim3((unsigned)grid), dim3(kThreads), 0,
                       (hipStream_t)stream, static_cast<const uint4*>(w),
                       static_cast<const uint4*>(gamma), nchunks, hidden / 8, codes, scales);
  return hipGetLastError();
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
