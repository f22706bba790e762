// measure.hip -- libmxq_measure.so: measurement references for the MXNorm
// forward, not steps of the method.  Each kernel moves exactly the bytes of an
// E4M3 mxnorm_fwd call (reads x [rows, hidden] bf16; writes rows x hidden code
// bytes, rows x hidden/32 scale bytes and one fp32 value per row) with one of
// several lane layouts, and does no arithmetic beyond XOR: its run time is
// the practical HBM ceiling of that byte pattern on the chip, against which
// the forward's time is compared.
//
// Output (the same for every layout, so one host check covers them all): F is
// the XOR of every 32-bit word of the row (so, as in the forward, no store can
// leave before the whole row has arrived -- across the row's waves through
// LDS, as the forward's row statistic); the 8 code bytes of the row's 16-byte
// input chunk (w0, w1, w2, w3) are the words (w0 ^ w1 ^ F, w2 ^ w3); every
// scale dword of the row is F; the row's fp32 value has the bits of F.
//
// Layouts (a lane's registers hold 16-byte input chunks):
//   kChunk8   : lane `lane` of wave `wir` holds chunk (wir*NCH + s)*64 + lane,
//               one 8-byte code store per chunk -- the forward's layout;
//   kLane16   : a lane holds 16 consecutive elements, group
//               g = (wir*NCH/2 + t)*64 + lane (loads 16 bytes apart), one
//               16-byte code store per group;
//   kLane16X  : contiguous 1 KiB loads (chunks (wir*NCH/2 + t)*128 + lane and
//               + 64 + lane), then neighbouring lanes swap halves by DPP so a
//               lane holds a whole 16-element group, one 16-byte code store.
// W waves own a row (4/W rows per 256-thread workgroup).
//
// The backward's byte pattern (mxq_measure_bwd_pattern): reads x and dy
// [rows, hidden] bf16 and writes dx [rows, hidden] bf16, the bytes of an
// mxnorm_bwd call without a gain, with the backward's lane layout (lane `lane`
// of wave `wir` holds chunk (wir*NCH + s)*64 + lane of x and of dy) over 2
// waves per row (two rows per 256-thread workgroup) or 8 (one row per
// 512-thread workgroup).  F is the XOR of every 32-bit word of the row's x
// and dy (no dx store leaves before the whole row has arrived, as the
// backward's row dot); each 16-byte dx chunk is the word-wise x ^ dy ^ F.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq_measure.h"

namespace {

constexpr int kWave = 64;
constexpr int kChunk8 = 0, kLane16 = 1, kLane16X = 2;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_nt(const uint8_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// XOR over the 64 lanes (quad swaps, row rotations by 4 and 8, then the four
// 16-lane rows through scalar reads): wave-uniform.
__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
  v ^= dpp<0xB1>(v);
  v ^= dpp<0x4E>(v);
  v ^= dpp<0x124>(v);
  v ^= dpp<0x128>(v);
  return (uint32_t)(__builtin_amdgcn_readlane((int)v, 0) ^ __builtin_amdgcn_readlane((int)v, 16) ^
                    __builtin_amdgcn_readlane((int)v, 32) ^ __builtin_amdgcn_readlane((int)v, 48));
}

template <int W, int NCH, int MODE>
__global__ __launch_bounds__(256) void k_pattern(const uint8_t* __restrict__ x, int64_t rows,
                                                 uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales,
                                                 float* __restrict__ rrms) {
  constexpr int HID = W * kWave * 8 * NCH;  // elements per row
  constexpr int RPW = 4 / W;
  static_assert(MODE == kChunk8 || NCH % 2 == 0, "16-element layouts hold chunk pairs");
  __shared__ uint32_t s_f[4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rslot = wave / W, wir = wave % W;
  const int64_t row = (int64_t)blockIdx.x * RPW + rslot;
  const bool row_ok = row < rows;  // waves past the end still meet the barrier
  const uint8_t* xrow = x + (row_ok ? row : 0) * (int64_t)HID * 2;

  uint4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    uint32_t ch;
    if constexpr (MODE == kChunk8) ch = (uint32_t)((wir * NCH + c) * kWave + lane);
    else if constexpr (MODE == kLane16) ch = (uint32_t)(((wir * NCH / 2 + c / 2) * kWave + lane) * 2 + (c & 1));
    else ch = (uint32_t)((wir * NCH / 2 + c / 2) * 2 * kWave + (c & 1) * kWave + lane);
    v[c] = load_nt(xrow + ch * 16u);
  }
  uint32_t f = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) f ^= v[c].x ^ v[c].y ^ v[c].z ^ v[c].w;
  f = wave_xor(f);
  if constexpr (W > 1) {
    if (lane == 0) s_f[wave] = f;
    __syncthreads();
    f = s_f[rslot * W];
#pragma unroll
    for (int w = 1; w < W; ++w) f ^= s_f[rslot * W + w];
  }
  if (!row_ok) return;

  if constexpr (MODE == kLane16X) {
    const bool even = (lane & 1) == 0;
#pragma unroll
    for (int t = 0; t < NCH / 2; ++t) {
      const uint4 A = v[2 * t], B = v[2 * t + 1];
      const uint4 snd = even ? B : A;
      uint4 rcv;
      rcv.x = dpp<0xB1>(snd.x);
      rcv.y = dpp<0xB1>(snd.y);
      rcv.z = dpp<0xB1>(snd.z);
      rcv.w = dpp<0xB1>(snd.w);
      v[2 * t] = even ? A : rcv;
      v[2 * t + 1] = even ? rcv : B;
    }
  }
  uint8_t* crow = codes + row * (int64_t)HID;
  if constexpr (MODE == kChunk8) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const uint32_t ch = (uint32_t)((wir * NCH + c) * kWave + lane);
      const u32x2_t o = {v[c].x ^ v[c].y ^ f, v[c].z ^ v[c].w};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2_t*>(crow + ch * 8u));
    }
  } else {
#pragma unroll
    for (int t = 0; t < NCH / 2; ++t) {
      uint32_t g;
      if constexpr (MODE == kLane16) g = (uint32_t)((wir * NCH / 2 + t) * kWave + lane);
      else g = (uint32_t)((wir * NCH / 2 + t) * kWave + (lane >> 1) + ((lane & 1) ? kWave / 2 : 0));
      const uint4 a = v[2 * t], b = v[2 * t + 1];
      const u32x4_t o = {a.x ^ a.y ^ f, a.z ^ a.w, b.x ^ b.y ^ f, b.z ^ b.w};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(crow + g * 16u));
    }
  }
  constexpr int kDw = HID / 128 / W;  // scale dwords per wave
  uint32_t* srow = reinterpret_cast<uint32_t*>(scales + row * (int64_t)(HID / 32));
  if (lane < kDw) srow[wir * kDw + lane] = f;
  if (wir == 0 && lane == 0) rrms[row] = __uint_as_float(f);
}

template <int W, int NCH>
__global__ __launch_bounds__(W > 4 ? W * 64 : 256) void k_bwd_pattern(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ dy, int64_t rows,
    uint8_t* __restrict__ dx) {
  constexpr int NW = W > 4 ? W : 4;  // waves per workgroup
  constexpr int RPW = NW / W;
  constexpr int HID = W * kWave * 8 * NCH;
  __shared__ uint32_t s_f[NW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rslot = wave / W, wir = wave % W;
  const int64_t row = (int64_t)blockIdx.x * RPW + rslot;
  const bool row_ok = row < rows;  // waves past the end still meet the barrier
  const int64_t base = (row_ok ? row : 0) * (int64_t)HID * 2;
  uint4 a[NCH], b[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t ch = (uint32_t)((wir * NCH + c) * kWave + lane);
    a[c] = load_nt(x + base + ch * 16u);
    b[c] = load_nt(dy + base + ch * 16u);
  }
  uint32_t f = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    f ^= a[c].x ^ a[c].y ^ a[c].z ^ a[c].w ^ b[c].x ^ b[c].y ^ b[c].z ^ b[c].w;
  f = wave_xor(f);
  if (lane == 0) s_f[wave] = f;
  __syncthreads();
  f = s_f[rslot * W];
#pragma unroll
  for (int w = 1; w < W; ++w) f ^= s_f[rslot * W + w];
  if (!row_ok) return;
  uint8_t* drow = dx + row * (int64_t)HID * 2;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const uint32_t ch = (uint32_t)((wir * NCH + c) * kWave + lane);
    const u32x4_t o = {a[c].x ^ b[c].x ^ f, a[c].y ^ b[c].y ^ f, a[c].z ^ b[c].z ^ f,
                       a[c].w ^ b[c].w ^ f};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t*>(drow + ch * 16u));
  }
}

template <int W>
hipError_t launch_bwd(const void* x, const void* dy, int64_t rows, int hidden, void* dx,
                      hipStream_t st) {
  constexpr int NW = W > 4 ? W : 4, RPW = NW / W;
  const dim3 grid((unsigned)((rows + RPW - 1) / RPW)), block(NW * kWave);
  const uint8_t* xp = static_cast<const uint8_t*>(x);
  const uint8_t* dp = static_cast<const uint8_t*>(dy);
  uint8_t* op = static_cast<uint8_t*>(dx);
  switch (hidden / (W * kWave * 8)) {
    case 1: hipLaunchKernelGGL((k_bwd_pattern<W, 1>), grid, block, 0, st, xp, dp, rows, op); break;
    case 2: hipLaunchKernelGGL((k_bwd_pattern<W, 2>), grid, block, 0, st, xp, dp, rows, op); break;
    case 4: hipLaunchKernelGGL((k_bwd_pattern<W, 4>), grid, block, 0, st, xp, dp, rows, op); break;
    case 8: hipLaunchKernelGGL((k_bwd_pattern<W, 8>), grid, block, 0, st, xp, dp, rows, op); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int W, int NCH, int MODE>
hipError_t launch(const void* x, int64_t rows, uint8_t* codes, uint8_t* scales, float* rrms,
                  hipStream_t st) {
  constexpr int RPW = 4 / W;
  hipLaunchKernelGGL((k_pattern<W, NCH, MODE>), dim3((unsigned)((rows + RPW - 1) / RPW)),
                     dim3(256), 0, st, static_cast<const uint8_t*>(x), rows, codes, scales, rrms);
  return hipGetLastError();
}

// NCH chunks per lane for a row of `hidden` over W waves.
template <int W, int MODE>
hipError_t launch_hidden(const void* x, int64_t rows, int hidden, uint8_t* codes, uint8_t* scales,
                         float* rrms, hipStream_t st) {
  const int nch = hidden / (W * kWave * 8);
  switch (nch) {
    case 1:
      if constexpr (MODE == kChunk8) return launch<W, 1, MODE>(x, rows, codes, scales, rrms, st);
      return hipErrorInvalidValue;
    case 2: return launch<W, 2, MODE>(x, rows, codes, scales, rrms, st);
    case 4: return launch<W, 4, MODE>(x, rows, codes, scales, rrms, st);
    case 8: return launch<W, 8, MODE>(x, rows, codes, scales, rrms, st);
    case 16: return launch<W, 16, MODE>(x, rows, codes, scales, rrms, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" {

int mxq_pattern_supported(int layout, int64_t hidden) {
  if (layout < 0 || layout >= MXQ_PATTERN_COUNT) return 0;
  const int waves = (layout == MXQ_PATTERN_TWO_WAVES_CHUNK8 ||
                     layout == MXQ_PATTERN_TWO_WAVES_LANE16 ||
                     layout == MXQ_PATTERN_TWO_WAVES_LANE16X) ? 2 : 1;
  const int min_chunks = (layout == MXQ_PATTERN_ONE_WAVE_CHUNK8 ||
                          layout == MXQ_PATTERN_TWO_WAVES_CHUNK8) ? 1 : 2;
  if (hidden <= 0 || hidden % (waves * kWave * 8) != 0) return 0;
  const int64_t nch = hidden / (waves * kWave * 8);
  return (nch == 1 || nch == 2 || nch == 4 || nch == 8 || nch == 16) && nch >= min_chunks;
}

int mxq_measure_pattern(int layout, const void* x, int64_t rows, int64_t hidden, uint8_t* codes,
                        uint8_t* scales, float* rrms, void* stream) {
  if (rows < 0 || hidden <= 0) return -1;
  if (!mxq_pattern_supported(layout, hidden)) return -3;
  if (rows > ((int64_t)1 << 24) - 1) return -3;
  if (rows == 0) return 0;
  if (x == nullptr || codes == nullptr || scales == nullptr || rrms == nullptr) return -1;
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 15) || ((uintptr_t)scales & 3) ||
      ((uintptr_t)rrms & 3))
    return -2;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  const int h = (int)hidden;
  hipError_t e = hipErrorInvalidValue;
  switch (layout) {
    case MXQ_PATTERN_ONE_WAVE_CHUNK8: e = launch_hidden<1, kChunk8>(x, rows, h, codes, scales, rrms, st); break;
    case MXQ_PATTERN_TWO_WAVES_CHUNK8: e = launch_hidden<2, kChunk8>(x, rows, h, codes, scales, rrms, st); break;
    case MXQ_PATTERN_ONE_WAVE_LANE16: e = launch_hidden<1, kLane16>(x, rows, h, codes, scales, rrms, st); break;
    case MXQ_PATTERN_ONE_WAVE_LANE16X: e = launch_hidden<1, kLane16X>(x, rows, h, codes, scales, rrms, st); break;
    case MXQ_PATTERN_TWO_WAVES_LANE16: e = launch_hidden<2, kLane16>(x, rows, h, codes, scales, rrms, st); break;
    case MXQ_PATTERN_TWO_WAVES_LANE16X: e = launch_hidden<2, kLane16X>(x, rows, h, codes, scales, rrms, st); break;
    default: break;
  }
  return e == hipSuccess ? 0 : -4;
}

int mxq_bwd_pattern_supported(int waves, int64_t hidden) {
  if (waves != 2 && waves != 8) return 0;
  if (hidden <= 0 || hidden % (waves * kWave * 8) != 0) return 0;
  const int64_t nch = hidden / (waves * kWave * 8);
  return nch == 1 || nch == 2 || nch == 4 || nch == 8;
}

int mxq_measure_bwd_pattern(int waves, const void* x, const void* dy, int64_t rows,
                            int64_t hidden, void* dx, void* stream) {
  if (rows < 0 || hidden <= 0) return -1;
  if (!mxq_bwd_pattern_supported(waves, hidden)) return -3;
  if (rows > ((int64_t)1 << 24) - 1) return -3;
  if (rows == 0) return 0;
  if (x == nullptr || dy == nullptr || dx == nullptr) return -1;
  if (((uintptr_t)x & 15) || ((uintptr_t)dy & 15) || ((uintptr_t)dx & 15)) return -2;
  (void)hipGetLastError();
  hipStream_t st = (hipStream_t)stream;
  const hipError_t e = waves == 2 ? launch_bwd<2>(x, dy, rows, (int)hidden, dx, st)
                                  : launch_bwd<8>(x, dy, rows, (int)hidden, dx, st);
  return e == hipSuccess ? 0 : -4;
}

}  // extern "C"
