// mx_gemm.hip -- MXFP8 x MXFP8 matrix product on gfx950 matrix cores.
//
// Source: "MXNorm: Reusing MXFP block scales for efficient tensor
// normalisation" (gist.science summary), "Resumen tecnico" §2,
// "Implementacion", MXNormLinear item: the gain is folded into the weights of
// the following linear layer, which consumes the MX tensor MXNorm emits.
// This is that layer: C[m, n] = sum_k A[m, k] B[n, k] with A (the MX
// activations) and B (the MX weights) both E4M3 codes with one E8M0 scale per
// 32 consecutive k, K-contiguous rows; C in fp32.
//
// A dense contraction, so it runs on MFMA: V_MFMA_SCALE_F32_32X32X64_F8F6F4
// multiplies a 32x64 by a 64x32 MX tile, applying the E8M0 block scales in
// hardware.  Operand layout of that instruction (established on gfx950 with
// one-wave probes): row i of A is held by lanes i and i + 32; lane i + 32h
// holds k = 16h .. 16h+15 in its bytes 0..15 and k = 32 + 16h .. 32+16h+15
// in bytes 16..31; the scale of k-block 0 comes from lane i, of k-block 1
// from lane i + 32 (byte selected by op_sel).  B likewise by column.  The
// 32x32 fp32 result sits in lane l, register r at row (r % 4) + 8 (r / 4) +
// 4 (l / 32), column l % 32.  The unit sums the 64 products of one
// instruction with a short alignment window: measured error up to 2^-11.9 of
// the largest product (not an IEEE fp32 sum); successive instructions
// accumulate in fp32.
//
// Tiling: a 256-thread workgroup computes a 128 x 128 tile of C, each of its
// 4 waves a 64 x 64 quarter (2 x 2 MFMA tiles).  K advances 128 bytes per
// stage: the workgroup copies the 128 x 128-byte slices of A and B and their
// scales into LDS (16-byte chunks XOR-swizzled by row so that the MFMA
// fragment reads are free of bank conflicts) while holding the next stage's
// data in registers.  Workgroups are remapped so that the tiles one XCD runs
// share rows of A and columns of B in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mxq {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kTileM = 128;
constexpr int kTileN = 128;
constexpr int kStageK = 128;                   // bytes (= elements) of K per stage
constexpr int kRowBytes = kStageK;             // LDS row: one stage of one row
constexpr int kGroupM = 8;                     // tile rows per L2 group
constexpr int kXcds = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const uint8_t* a;       // [M, K] E4M3
  const uint8_t* as;      // [M, K/32] E8M0
  const uint8_t* b;       // [N, K]
  const uint8_t* bs;      // [N, K/32]
  float* c;               // [M, N]
  int64_t M, N;
  int K;
  int tiles_m, tiles_n;
};

// LDS offset of 16-byte chunk `chunk` (0..7) of row `row` in a stage slice.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7)) << 4);
}

__global__ __launch_bounds__(kGemmThreads) void k_mx_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t s_a[kTileM * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_b[kTileN * kRowBytes];
  __shared__ uint32_t s_as[kTileM];  // the 4 block scales of the stage, per row
  __shared__ uint32_t s_bs[kTileN];

  // ---- tile of this workgroup: XCD-contiguous ranges, grouped by kGroupM rows
  // Workgroup bid runs on XCD bid % 8; when the tile count divides evenly,
  // give each XCD a contiguous range of the grouped tile order.
  const int ntiles = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int t = ntiles % kXcds == 0 ? (bid % kXcds) * (ntiles / kXcds) + bid / kXcds : bid;
  const int group = t / (kGroupM * g.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(g.tiles_m - first_m, kGroupM);
  const int tm = first_m + (t % (kGroupM * g.tiles_n)) % gm;
  const int tn = (t % (kGroupM * g.tiles_n)) / gm;
  const int64_t m0 = (int64_t)tm * kTileM;
  const int64_t n0 = (int64_t)tn * kTileN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // this wave's 64 x 64 quarter
  const int KB = g.K >> 5;                  // scale bytes per row

  // ---- global -> register copy of one stage: thread `tid` moves the 16-byte
  // chunk (tid & 7) of rows (tid >> 3) + 32 p, p = 0..3, of both A and B
  const int crow = tid >> 3, cchunk = tid & 7;
  const uint8_t* pa[4];
  const uint8_t* pb[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t ra = min(m0 + crow + 32 * p, g.M - 1);  // ragged tiles: clamp, mask later
    const int64_t rb = min(n0 + crow + 32 * p, g.N - 1);
    pa[p] = g.a + ra * g.K + cchunk * 16;
    pb[p] = g.b + rb * g.K + cchunk * 16;
  }
  // scales: threads 0..127 fetch the A row's 4 stage scales, 128..255 B's
  const bool sc_is_a = tid < kTileM;
  const int srow = tid & (kTileM - 1);
  const uint8_t* ps = sc_is_a ? g.as + min(m0 + srow, g.M - 1) * (int64_t)KB
                              : g.bs + min(n0 + srow, g.N - 1) * (int64_t)KB;

  v4i ra[4], rb[4];
  uint32_t rs;
  auto fetch = [&](int k0) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      ra[p] = *reinterpret_cast<const v4i*>(pa[p] + k0);
      rb[p] = *reinterpret_cast<const v4i*>(pb[p] + k0);
    }
    rs = *reinterpret_cast<const uint32_t*>(ps + (k0 >> 5));
  };
  auto stash = [&]() {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      *reinterpret_cast<v4i*>(s_a + lds_off(crow + 32 * p, cchunk)) = ra[p];
      *reinterpret_cast<v4i*>(s_b + lds_off(crow + 32 * p, cchunk)) = rb[p];
    }
    if (sc_is_a) s_as[srow] = rs; else s_bs[srow] = rs;
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;   // fragment row (A) / column (B) within a 32-tile
  const int fh = lane >> 5;   // which 16-byte halves of each k-block this lane holds
  fetch(0);
  for (int k0 = 0; k0 < g.K; k0 += kStageK) {
    __syncthreads();  // the previous stage's fragment reads are done
    stash();
    __syncthreads();
    if (k0 + kStageK < g.K) fetch(k0 + kStageK);  // in flight during the MFMAs

    uint32_t sa_w[2], sb_w[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sa_w[i] = s_as[wm * 64 + i * 32 + fr];
      sb_w[i] = s_bs[wn * 64 + i * 32 + fr];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ar = wm * 64 + i * 32 + fr;
        const int br = wn * 64 + i * 32 + fr;
        const v4i a0 = *reinterpret_cast<const v4i*>(s_a + lds_off(ar, ks * 4 + fh));
        const v4i a1 = *reinterpret_cast<const v4i*>(s_a + lds_off(ar, ks * 4 + 2 + fh));
        const v4i b0 = *reinterpret_cast<const v4i*>(s_b + lds_off(br, ks * 4 + fh));
        const v4i b1 = *reinterpret_cast<const v4i*>(s_b + lds_off(br, ks * 4 + 2 + fh));
        fa[i] = (v8i){a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        fb[i] = (v8i){b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      }
      // block (2 ks + fh) of the stage: lane i carries k-block 0's scale,
      // lane i + 32 k-block 1's (byte 0 after the shift)
      const int sh = 8 * (2 * ks + fh);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[i], fb[j], acc[i][j], 0, 0, 0, (int)(sa_w[i] >> sh), 0, (int)(sb_w[j] >> sh));
    }
  }

  // ---- epilogue: lane l, register r -> row (r%4) + 8(r/4) + 4(l/32), column l%32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + (r & 3) + 8 * (r >> 2) + 4 * fh;
        if (row < g.M && col < g.N) g.c[row * g.N + col] = acc[i][j][r];
      }
    }
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                          const uint8_t* bs, int64_t M, int64_t N, int K, float* c,
                          void* stream) {
  GemmArgs g;
  g.a = a;
  g.as = as;
  g.b = b;
  g.bs = bs;
  g.c = c;
  g.M = M;
  g.N = N;
  g.K = K;
  g.tiles_m = (int)((M + kTileM - 1) / kTileM);
  g.tiles_n = (int)((N + kTileN - 1) / kTileN);
  const unsigned ntiles = (unsigned)g.tiles_m * (unsigned)g.tiles_n;
  hipLaunchKernelGGL(k_mx_gemm, dim3(ntiles), dim3(kGemmThreads), 0, (hipStream_t)stream, g);
  return hipGetLastError();
}

}  // namespace mxq
