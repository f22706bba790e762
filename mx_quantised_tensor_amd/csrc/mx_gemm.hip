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
// Tiling.  A 256-thread workgroup (one wave per SIMD) owns 256 x 256 tiles of
// C; each wave computes a 128 x 128 quarter as 4 x 4 MFMA tiles whose
// accumulators live in AGPRs.  K advances 64 per stage (one MFMA k-step).
// Each stage's slices of A and B (256 x 64 bytes each) and their scales are
// copied from global memory straight into LDS by the gfx950 LDS-DMA loads,
// into a ring of four buffers, up to four stages ahead of the one the waves
// multiply.  16-byte chunks are
// XOR-swizzled by row (applied on the global side of the copy) so that the
// fragment reads are free of bank conflicts.  Fragment reads are
// inline-assembly LDS loads with explicit waits, and the waits for the copies
// are explicit vmcnt counts: the compiler cannot tell that an in-flight copy
// writes another buffer and would otherwise wait for all of them before every
// read.  Workgroups are persistent over tiles; tiles are taken in groups of 8
// tile rows for L2 locality, each XCD a contiguous range.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mxq {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kTile = 256;                      // C tile edge (rows and columns)
constexpr int kStageK = 64;                     // K per stage (bytes = elements)
constexpr int kRowBytes = kStageK;              // one row of a stage slice in LDS
constexpr int kSlice = kTile * kRowBytes;       // 16 KiB: one operand's stage slice
constexpr int kScaleBytes = kTile * 4;          // the aligned scale dword holding the stage
constexpr int kBuf = 2 * kSlice + 2 * kScaleBytes;  // one stage buffer: A, B, scales
constexpr int kRing = 4;                        // stage buffers (3 in flight)
constexpr int kDmaOps = 10;                     // LDS-DMA instructions per wave per stage
constexpr int kGroupM = 8;                      // tile rows per L2 group
constexpr int kXcds = 8;
constexpr int kMaxGroups = 256;                 // one persistent workgroup per CU

#define MXQ_LDS __attribute__((address_space(3)))

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

struct GemmArgs {
  const uint8_t* a;   // [M, K] E4M3
  const uint8_t* as;  // [M, K/32] E8M0
  const uint8_t* b;   // [N, K]
  const uint8_t* bs;  // [N, K/32]
  float* c;           // [M, N]
  int64_t M, N;
  int K;
  int tiles_m, tiles_n;
};

// In LDS, logical 16-byte chunk c (0..3) of row r of a slice is stored at
// r * kRowBytes + ((c ^ ((r >> 1) & 3)) << 4): eight consecutive rows reading
// the same logical chunk touch eight different 16-byte bank groups.

__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  v4i v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}
__device__ __forceinline__ uint32_t lds_read1(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile t of the grouped order -> (tile row, tile column).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int w = t % per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// The DMA of one stage (k0) of the current tile into LDS at BUF: wave w copies
// rows [64 w, 64 w + 64) of the A and B slices (4 x 1 KiB per operand: lane l
// of copy q lands at row 64 w + 16 q + l/4, physical chunk l%4, and reads the
// logical chunk that belongs there) and the two scale bytes of each of those
// rows (the 4-byte-aligned scale word holding the stage's two blocks; LDS-DMA
// writes 4 bytes per lane): kDmaOps instructions.  A macro: the LDS-DMA
// builtin must sit in the kernel body itself.
#define MXQ_GEMM_DMA(BUF, K0)                                                                 \
  do {                                                                                        \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                           \
      const int row = wave * 64 + q * 16 + (lane >> 2);                                       \
      const int chunk = (lane & 3) ^ ((row >> 1) & 3);                                        \
      const uint32_t dst = (BUF) + (uint32_t)((wave * 64 + q * 16) * kRowBytes);             \
      __builtin_amdgcn_global_load_lds((const void*)(arow[q] + (K0) + chunk * 16),            \
                                       (MXQ_LDS void*)(size_t)dst, 16, 0, 0);                 \
      __builtin_amdgcn_global_load_lds((const void*)(brow[q] + (K0) + chunk * 16),            \
                                       (MXQ_LDS void*)(size_t)(dst + kSlice), 16, 0, 0);      \
    }                                                                                         \
    __builtin_amdgcn_global_load_lds((const void*)(ascl + (((K0) >> 5) & ~3)),                \
                                     (MXQ_LDS void*)(size_t)((BUF) + 2 * kSlice + wave * 256), \
                                     4, 0, 0);                                                \
    __builtin_amdgcn_global_load_lds(                                                         \
        (const void*)(bscl + (((K0) >> 5) & ~3)),                                             \
        (MXQ_LDS void*)(size_t)((BUF) + 2 * kSlice + kScaleBytes + wave * 256), 4, 0, 0);     \
  } while (0)

// This lane's fragments of tile pair i of one stage: A rows wm*128 + 32 i + fr
// and B rows wn*128 + 32 i + fr, logical chunks fh (k-block 0 half) and 2 + fh
// (k-block 1 half), and the scale byte of k-block fh of each of the two rows
// (byte SB0 + fh of the row's scale word, SB0 = 0 or 2 by stage parity).
#define MXQ_GEMM_READ(BUF, I, FA, FB, SA, SB, SB0)                                            \
  do {                                                                                        \
    FA[I][0] = lds_read16((BUF) + a_off[I] + c0);                                             \
    FA[I][1] = lds_read16((BUF) + a_off[I] + c1);                                             \
    FB[I][0] = lds_read16((BUF) + b_off[I] + c0);                                             \
    FB[I][1] = lds_read16((BUF) + b_off[I] + c1);                                             \
    SA[I] = lds_read1((BUF) + 2 * kSlice + (uint32_t)((wm * 128 + (I) * 32 + fr) * 4 + (SB0) + fh)); \
    SB[I] = lds_read1((BUF) + 2 * kSlice + kScaleBytes +                                     \
                      (uint32_t)((wn * 128 + (I) * 32 + fr) * 4 + (SB0) + fh));               \
  } while (0)

// Wait for this lane's fragment reads and make their registers visible as
// written here (the compiler cannot see inside the reads).
#define MXQ_GEMM_READ_WAIT(FA, FB, SA, SB)                                                    \
  asm volatile("s_waitcnt lgkmcnt(0)"                                                         \
               : "+v"(FA[0][0]), "+v"(FA[0][1]), "+v"(FA[1][0]), "+v"(FA[1][1]),             \
                 "+v"(FA[2][0]), "+v"(FA[2][1]), "+v"(FA[3][0]), "+v"(FA[3][1]),             \
                 "+v"(FB[0][0]), "+v"(FB[0][1]), "+v"(FB[1][0]), "+v"(FB[1][1]),             \
                 "+v"(FB[2][0]), "+v"(FB[2][1]), "+v"(FB[3][0]), "+v"(FB[3][1]),             \
                 "+v"(SA[0]), "+v"(SA[1]), "+v"(SA[2]), "+v"(SA[3]), "+v"(SB[0]),            \
                 "+v"(SB[1]), "+v"(SB[2]), "+v"(SB[3]))

// The 4 matrix instructions of A tile I of one stage, then an empty statement
// taking their accumulators as inputs: it keeps them ahead of the volatile
// LDS reads that follow (they touch no memory, so the compiler would
// otherwise move them freely).
#define MXQ_GEMM_MFMA_ROW(I, FA, FB, SA, SB)                                                  \
  do {                                                                                        \
    const v8i va = {FA[I][0].x, FA[I][0].y, FA[I][0].z, FA[I][0].w,                           \
                    FA[I][1].x, FA[I][1].y, FA[I][1].z, FA[I][1].w};                          \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                           \
      const v8i vb = {FB[j][0].x, FB[j][0].y, FB[j][0].z, FB[j][0].w,                         \
                      FB[j][1].x, FB[j][1].y, FB[j][1].z, FB[j][1].w};                        \
      acc[I][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc[I][j], 0, 0, 0, \
                                                                  (int)SA[I], 0, (int)SB[j]); \
    }                                                                                         \
    asm volatile("" ::"a"(acc[I][0]), "a"(acc[I][1]), "a"(acc[I][2]), "a"(acc[I][3]));        \
  } while (0)

__global__ __launch_bounds__(kGemmThreads) void k_mx_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing * kBuf];  // 132 KiB of 160
  const uint32_t base = (uint32_t)(size_t)(MXQ_LDS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // this wave's 128 x 128 quarter
  const int fr = lane & 31;                 // fragment row / column within a 32-tile
  const int fh = lane >> 5;                 // which 16-byte half of each k-block
  const int KB = g.K >> 5;
  const int nstages = g.K / kStageK;
  const int ntiles = g.tiles_m * g.tiles_n;

  // This lane's fragment rows inside a buffer.  Every such row is fr modulo 8,
  // so logical chunk c sits at physical chunk c ^ ((fr >> 1) & 3).
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a_off[i] = (uint32_t)((wm * 128 + i * 32 + fr) * kRowBytes);
    b_off[i] = kSlice + (uint32_t)((wn * 128 + i * 32 + fr) * kRowBytes);
  }
  const uint32_t c0 = (uint32_t)((fh ^ ((fr >> 1) & 3)) << 4);
  const uint32_t c1 = (uint32_t)(((2 + fh) ^ ((fr >> 1) & 3)) << 4);

  // Tiles of this workgroup.  Workgroup bid runs on XCD bid % 8: when the
  // counts allow, XCD x takes the contiguous range [x T/8, (x+1) T/8) of the
  // grouped tile order, its G/8 workgroups interleaved over it.
  const int G = (int)gridDim.x;
  const bool by_xcd = ntiles % kXcds == 0 && G % kXcds == 0;
  const int per_x = ntiles / kXcds, xcd = (int)blockIdx.x % kXcds, jx = (int)blockIdx.x / kXcds;
  for (int it = 0;; ++it) {
    int t;
    if (by_xcd) {
      const int w = jx + it * (G / kXcds);
      if (w >= per_x) break;
      t = xcd * per_x + w;
    } else {
      t = (int)blockIdx.x + it * G;
      if (t >= ntiles) break;
    }
    int tm, tn;
    tile_coords(t, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kTile, n0 = (int64_t)tn * kTile;

    // global sources of this wave's DMA rows (ragged tiles: clamped rows)
    const uint8_t* arow[4];
    const uint8_t* brow[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = wave * 64 + q * 16 + (lane >> 2);
      arow[q] = g.a + min(m0 + r, g.M - 1) * (int64_t)g.K;
      brow[q] = g.b + min(n0 + r, g.N - 1) * (int64_t)g.K;
    }
    const uint8_t* ascl = g.as + min(m0 + wave * 64 + lane, g.M - 1) * (int64_t)KB;
    const uint8_t* bscl = g.bs + min(n0 + wave * 64 + lane, g.N - 1) * (int64_t)KB;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Prologue: stages 0..3 in flight; wait for stage 0 (older vector-memory
    // operations, such as the previous tile's C stores, retire first).
    __builtin_amdgcn_s_barrier();  // every wave is done reading the ring
    MXQ_GEMM_DMA(base, 0);
    if (nstages > 1) MXQ_GEMM_DMA(base + kBuf, kStageK);
    if (nstages > 2) MXQ_GEMM_DMA(base + 2 * kBuf, 2 * kStageK);
    if (nstages > 3) MXQ_GEMM_DMA(base + 3 * kBuf, 3 * kStageK);
    if (nstages > 3) wait_vmcnt<3 * kDmaOps>();
    else if (nstages > 2) wait_vmcnt<2 * kDmaOps>();
    else if (nstages > 1) wait_vmcnt<kDmaOps>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    // Stage s: read this stage's fragments, issue its 16 matrix instructions,
    // wait for stage s + 1 to land in every wave; after that barrier every wave
    // is done reading this stage's buffer, which then takes stage s + 4.
    for (int s = 0; s < nstages; ++s) {
      const uint32_t buf = base + (uint32_t)((s & 3) * kBuf);
      v4i fa[4][2], fb[4][2];
      uint32_t sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) MXQ_GEMM_READ(buf, i, fa, fb, sa, sb, (2 * s) & 3);
      MXQ_GEMM_READ_WAIT(fa, fb, sa, sb);
#pragma unroll
      for (int i = 0; i < 4; ++i) MXQ_GEMM_MFMA_ROW(i, fa, fb, sa, sb);
      if (s + 1 < nstages) {
        // stages s+1 .. s+3 were issued; wait for s+1 (later ones may stay out)
        if (s + 3 < nstages) wait_vmcnt<2 * kDmaOps>();
        else if (s + 2 < nstages) wait_vmcnt<kDmaOps>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();  // also: every wave is done reading buffer s & 3
        if (s + 4 < nstages) MXQ_GEMM_DMA(buf, (s + 4) * kStageK);
      }
    }

    // epilogue: lane l, register r -> row (r%4) + 8(r/4) + 4(l/32), column l%32
    const int64_t row0 = m0 + wm * 128 + 4 * fh, col0 = n0 + wn * 128 + fr;
    if (m0 + kTile <= g.M && n0 + kTile <= g.N) {
      float* cb = g.c + row0 * g.N + col0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* crow = cb + (int64_t)(i * 32 + (r & 3) + 8 * (r >> 2)) * g.N;
#pragma unroll
          for (int j = 0; j < 4; ++j) crow[j * 32] = acc[i][j][r];
        }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t col = col0 + j * 32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = row0 + i * 32 + (r & 3) + 8 * (r >> 2);
            if (row < g.M && col < g.N) g.c[row * g.N + col] = acc[i][j][r];
          }
        }
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
  g.tiles_m = (int)((M + kTile - 1) / kTile);
  g.tiles_n = (int)((N + kTile - 1) / kTile);
  const int ntiles = g.tiles_m * g.tiles_n;
  const int groups = ntiles < kMaxGroups ? ntiles : kMaxGroups;
  hipLaunchKernelGGL(k_mx_gemm, dim3(groups), dim3(kGemmThreads), 0, (hipStream_t)stream, g);
  return hipGetLastError();
}

}  // namespace mxq
