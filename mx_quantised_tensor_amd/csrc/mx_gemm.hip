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
// Tiling.  A 256-thread workgroup (one wave per SIMD: the 256 accumulator
// registers of a 128 x 128 quarter fill a lane's AGPRs) owns 256 x 256 tiles
// of C; each wave computes its quarter as 4 x 4 matrix instructions per 64 k
// (a "sub-stage").  Operands reach LDS by the gfx950 LDS-DMA buffer loads in
// copy stages of 128 k: 128-byte row segments, one L2 line each, which the
// memory path moves about 1.6x faster than 64-byte ones.  Two copy buffers
// (2 x 64 KiB) alternate: stage j + 2 is copied while sub-stages 2j + 2 and
// 2j + 3 multiply.  Block scales travel in 16-byte records per row (16
// blocks = 4 copy stages), in three rotating sets, one small copy per stage.
// The wave's fragments of sub-stage u + 1 are read from LDS into a second
// register set while sub-stage u multiplies; LDS reads and copies are spread
// between the 16 matrix instructions so that the in-order wave never stalls
// its matrix unit behind a burst of memory instructions.  16-byte chunks are
// XOR-swizzled by row (applied on the global side of the copy) and scale
// records are rotated by row so that every LDS read is free of bank
// conflicts.  Waits are explicit counts: the compiler cannot tell that an
// in-flight copy writes the other buffer.  Rows beyond M or N fall outside
// the buffer range and read as zero (their outputs are not stored).
// Workgroups are persistent over tiles; tiles are taken in groups of 8 tile
// rows for L2 locality, each XCD a contiguous range; C is written with
// streaming (non-temporal) stores, as fp32 or as bf16 (round to nearest even;
// adjacent lanes swap one value so that each lane stores two neighbouring
// columns).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace mxq {

namespace {

constexpr int kGemmThreads = 256;
constexpr int kTile = 256;                      // C tile edge (rows and columns)
constexpr int kCopyK = 128;                     // k per copy stage (= bytes per row)
constexpr int kSlice = kTile * kCopyK;          // 32 KiB: one operand of one copy stage
constexpr int kBuf = 2 * kSlice;                // 64 KiB: A and B of one copy stage
constexpr int kScaleRec = 16;                   // one row's scale record: 16 blocks
constexpr int kScaleSet = 2 * kTile * kScaleRec;  // 8 KiB: A and B records of a group
constexpr int kScaleSets = 3;
constexpr int kScaleBase = 2 * kBuf;
constexpr int kLds = kScaleBase + kScaleSets * kScaleSet;  // 152 KiB of 160
constexpr int kCopyOps = 18;                    // copy instructions per wave per stage
constexpr int kGroupM = 8;                      // tile rows per L2 group
constexpr int kXcds = 8;
constexpr int kMaxGroups = 256;                 // one persistent workgroup per CU

#define MXQ_LDS __attribute__((address_space(3)))

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct GemmArgs {
  const uint8_t* a;   // [M, K] E4M3
  const uint8_t* as;  // [M, K/32] E8M0
  const uint8_t* b;   // [N, K]
  const uint8_t* bs;  // [N, K/32]
  void* c;            // [M, N] fp32 or bf16
  int64_t M, N;
  int K;
  int tiles_m, tiles_n;
};

// Raw buffer of `bytes` bytes at p (stride 0, 32-bit data format): offsets at
// or past `bytes` read as zero.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// LDS reads with a constant byte offset in the instruction's offset field (the
// fragments of a wave's four 32-row blocks are 4 KiB apart, their scale
// records 512 bytes apart: one address register serves all four).
template <int OFF>
__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  v4i v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
// Block blk (0..3, a constant once the callers' loops are unrolled).
__device__ __forceinline__ v4i lds_read16_blk(uint32_t addr, int blk) {
  switch (blk) {
    case 0: return lds_read16<0>(addr);
    case 1: return lds_read16<32 * kCopyK>(addr);
    case 2: return lds_read16<64 * kCopyK>(addr);
    default: return lds_read16<96 * kCopyK>(addr);
  }
}
__device__ __forceinline__ uint32_t lds_read4_blk(uint32_t addr, int blk) {
  switch (blk) {
    case 0: return lds_read4<0>(addr);
    case 1: return lds_read4<32 * kScaleRec>(addr);
    case 2: return lds_read4<64 * kScaleRec>(addr);
    default: return lds_read4<96 * kScaleRec>(addr);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// g mod 3 for 0 <= g < 2^14 without a division.
__device__ __forceinline__ int mod3(int g) { return g - 3 * ((g * 0x5556) >> 16); }

// Tile t of the grouped order -> (tile row, tile column).
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int per_group = kGroupM * tiles_n;
  const int first_m = (t / per_group) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int w = t % per_group;
  tm = first_m + w % gm;
  tn = w / gm;
}

// LDS layouts.  Copy stage j lives in buffer j & 1: A rows at [0, kSlice), B
// rows at [kSlice, kBuf), row r at r * 128.  Logical 16-byte chunk c of row r
// is stored at physical chunk c ^ swz(r), swz(r) = (r & 7) ^ ((r >> 3) & 3):
// the 16 rows one fragment read touches land on 16 different bank groups.
// Scale group G (copy stages 4G .. 4G+3) lives in set G mod 3: the record of
// A row r at r * 16, of B row r at 4 KiB + r * 16; it holds scale dwords
// 4G .. 4G+3 of the row (blocks 16G .. 16G+15), dword d at position
// (d + (r >> 3)) & 3.

template <bool BF16>
__global__ __launch_bounds__(kGemmThreads) void k_mx_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  const uint32_t base = (uint32_t)(size_t)(MXQ_LDS uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // this wave's 128 x 128 quarter
  const int fr = lane & 31;                 // fragment row / column within a 32-tile
  const int fh = lane >> 5;                 // which 16-byte half of each k-block
  const int K = g.K;
  const int KB = K >> 5;
  const int nstages = K / kCopyK;
  const int ntiles = g.tiles_m * g.tiles_n;

  // Read side.  Every fragment row of this lane is fr modulo 32, so its
  // swizzle is that of fr and its scale-record rotation is (fr >> 3) & 3.
  const int fz = (fr & 7) ^ ((fr >> 3) & 3);
  const int srot = (fr >> 3) & 3;
  // block i of the wave's fragments at + i * 32 rows (immediate offsets)
  const uint32_t a_off = (uint32_t)((wm * 128 + fr) * kCopyK);
  const uint32_t b_off = kSlice + (uint32_t)((wn * 128 + fr) * kCopyK);
  const uint32_t as_off = (uint32_t)((wm * 128 + fr) * kScaleRec);
  const uint32_t bs_off = kTile * kScaleRec + (uint32_t)((wn * 128 + fr) * kScaleRec);
  // chunk offset of sub-stage half v (of a copy stage), k-block h
  uint32_t coff[2][2];
#pragma unroll
  for (int v = 0; v < 2; ++v)
#pragma unroll
    for (int h = 0; h < 2; ++h) coff[v][h] = (uint32_t)(((4 * v + 2 * h + fh) ^ fz) << 4);

  // Copy side: lane -> (row within an 8-row group, physical chunk).
  const int crow = lane >> 3, cphys = lane & 7;

  // Tiles of this workgroup.  Workgroup bid runs on XCD bid % 8: when the
  // counts allow, XCD x takes the contiguous range [x T/8, (x+1) T/8) of the
  // grouped tile order, its G/8 workgroups interleaved over it.
  const int G = (int)gridDim.x;
  const bool by_xcd = ntiles % kXcds == 0 && G % kXcds == 0;
  const int per_x = ntiles / kXcds, xcd = (int)blockIdx.x % kXcds, jx = (int)blockIdx.x / kXcds;
  // Tile of this workgroup's iteration it, or -1 past its last one.
  auto tile_at = [&](int it) -> int {
    if (by_xcd) {
      const int w = jx + it * (G / kXcds);
      return w < per_x ? xcd * per_x + w : -1;
    }
    const int t = (int)blockIdx.x + it * G;
    return t < ntiles ? t : -1;
  };
  int64_t m0 = 0, n0 = 0;  // origin of the tile whose copies are in flight
  rsrc_t ra, rb, rsa, rsb;
  auto set_tile = [&](int t) {
    int tm, tn;
    tile_coords(t, g.tiles_m, g.tiles_n, tm, tn);
    m0 = (int64_t)tm * kTile;
    n0 = (int64_t)tn * kTile;
    const uint32_t rows_a = (uint32_t)min((int64_t)kTile, g.M - m0);
    const uint32_t rows_b = (uint32_t)min((int64_t)kTile, g.N - n0);
    ra = make_rsrc(g.a + m0 * K, rows_a * (uint32_t)K);
    rb = make_rsrc(g.b + n0 * K, rows_b * (uint32_t)K);
    rsa = make_rsrc(g.as + m0 * KB, rows_a * (uint32_t)KB);
    rsb = make_rsrc(g.bs + n0 * KB, rows_b * (uint32_t)KB);
  };

// Copy instruction D (0..15) of copy stage J: operand A for D < 8, B
// otherwise; 8 rows (64 wave + 8 (D % 8) + lane / 8) x 128 bytes, lane l
// filling physical chunk l % 8 with the logical chunk that belongs there.
#define MXQ_GEMM_DATA_OP(J, D)                                                              \
  do {                                                                                      \
    const int t_ = (D) & 7;                                                                 \
    const int rl_ = wave * 64 + t_ * 8 + crow;                                              \
    const int c_ = cphys ^ crow ^ (t_ & 3);                                                 \
    const uint32_t voff_ = (uint32_t)rl_ * (uint32_t)K + (uint32_t)((J) * kCopyK + c_ * 16); \
    const uint32_t dst_ = base + (uint32_t)(((J) & 1) * kBuf) + ((D) >= 8 ? kSlice : 0) +   \
                          (uint32_t)((wave * 64 + t_ * 8) * kCopyK);                        \
    __builtin_amdgcn_raw_ptr_buffer_load_lds((D) >= 8 ? rb : ra,                            \
                                             (MXQ_LDS void*)(size_t)dst_, 16, (int)voff_, 0, \
                                             0, 0);                                         \
  } while (0)

// Scale copy KOP (0..7) of group GRP: operand A for KOP < 4, B otherwise; 16
// rows (64 wave + 16 (KOP % 4) + lane / 4), lane l filling position l % 4 of
// its row's record.  Dwords past the row's end are clamped to its last one
// (never read).
#define MXQ_GEMM_SCALE_OP(GRP, KOP)                                                         \
  do {                                                                                      \
    const int k_ = (KOP), t_ = k_ & 3;                                                      \
    const int rl_ = wave * 64 + t_ * 16 + (lane >> 2);                                      \
    const int q_ = ((lane & 3) - ((2 * t_ + (lane >> 5)) & 3)) & 3;                         \
    const int gq_ = min(4 * (GRP) + q_, KB / 4 - 1);                                        \
    const uint32_t voff_ = (uint32_t)rl_ * (uint32_t)KB + (uint32_t)(4 * gq_);              \
    const uint32_t dst_ = base + kScaleBase + (uint32_t)(mod3(GRP) * kScaleSet) +           \
                          (k_ >= 4 ? kTile * kScaleRec : 0) +                               \
                          (uint32_t)((wave * 64 + t_ * 16) * kScaleRec);                    \
    __builtin_amdgcn_raw_ptr_buffer_load_lds(k_ >= 4 ? rsb : rsa,                           \
                                             (MXQ_LDS void*)(size_t)dst_, 4, (int)voff_, 0, \
                                             0, 0);                                         \
  } while (0)

// Copy instruction X (0..17) of stage J: its 16 data copies, then scale
// copies 2 (J % 4) and 2 (J % 4) + 1 of group J / 4 + 1 (issued once group
// J / 4 - 2, the set's previous tenant, is no longer read; landed long before
// stage 4 (J / 4 + 1) is read).
#define MXQ_GEMM_OP(J, X)                                                                   \
  do {                                                                                      \
    if ((X) < 16) MXQ_GEMM_DATA_OP(J, X);                                                   \
    else MXQ_GEMM_SCALE_OP(((J) >> 2) + 1, 2 * ((J) & 3) + (X) - 16);                       \
  } while (0)

// Fragment read R (0..23) of sub-stage U into NA/NB (operand chunks) and
// NSA/NSB (the scale dword of the sub-stage's copy stage).
#define MXQ_GEMM_READ(U, R, NA, NB, NSA, NSB)                                               \
  do {                                                                                      \
    const int ur_ = (U);                                                                    \
    if ((R) < 16) {                                                                         \
      const int ii_ = (R) >> 2, h_ = ((R) >> 1) & 1;                                        \
      const uint32_t b_ = base + (uint32_t)(((ur_ >> 1) & 1) * kBuf) + coff[ur_ & 1][h_];   \
      if ((R) & 1) NB[ii_][h_] = lds_read16_blk(b_ + b_off, ii_);                           \
      else NA[ii_][h_] = lds_read16_blk(b_ + a_off, ii_);                                   \
    } else {                                                                                \
      const int jr_ = ur_ >> 1;                                                             \
      const uint32_t s_ = base + kScaleBase + (uint32_t)(mod3(jr_ >> 2) * kScaleSet) +      \
                          (uint32_t)((((jr_ & 3) + srot) & 3) * 4);                         \
      if ((R) < 20) NSA[(R) - 16] = lds_read4_blk(s_ + as_off, (R) - 16);                   \
      else NSB[(R) - 20] = lds_read4_blk(s_ + bs_off, (R) - 20);                            \
    }                                                                                       \
  } while (0)

// Wait for this lane's fragment reads and make their registers visible as
// written here (the compiler cannot see inside the reads); then move each
// lane's scale byte of sub-stage U (byte 2 (U % 2) + fh of the dword) to byte 0.
#define MXQ_GEMM_READ_DONE(U, NA, NB, NSA, NSB)                                             \
  do {                                                                                      \
    asm volatile("s_waitcnt lgkmcnt(0)"                                                     \
                 : "+v"(NA[0][0]), "+v"(NA[0][1]), "+v"(NA[1][0]), "+v"(NA[1][1]),          \
                   "+v"(NA[2][0]), "+v"(NA[2][1]), "+v"(NA[3][0]), "+v"(NA[3][1]),          \
                   "+v"(NB[0][0]), "+v"(NB[0][1]), "+v"(NB[1][0]), "+v"(NB[1][1]),          \
                   "+v"(NB[2][0]), "+v"(NB[2][1]), "+v"(NB[3][0]), "+v"(NB[3][1]),          \
                   "+v"(NSA[0]), "+v"(NSA[1]), "+v"(NSA[2]), "+v"(NSA[3]), "+v"(NSB[0]),    \
                   "+v"(NSB[1]), "+v"(NSB[2]), "+v"(NSB[3]));                               \
    const uint32_t sh_ = 8 * fh + 16 * ((U) & 1);                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                      \
      NSA[i_] >>= sh_;                                                                      \
      NSB[i_] >>= sh_;                                                                      \
    }                                                                                       \
  } while (0)

// Prologue copies of the tile set by set_tile: stage 0, the first copies of
// scale groups 0 and 1, stage 1.  Issued once every wave is done reading the
// LDS of the tile before (or at the start).
#define MXQ_GEMM_PROLOGUE_ISSUE()                                                           \
  do {                                                                                      \
    _Pragma("unroll") for (int x = 0; x < kCopyOps; ++x) MXQ_GEMM_OP(0, x);                 \
    _Pragma("unroll") for (int k = 0; k < 8; ++k) MXQ_GEMM_SCALE_OP(0, k);                  \
    if (nstages > 1) {                                                                      \
      _Pragma("unroll") for (int x = 0; x < kCopyOps; ++x) MXQ_GEMM_OP(1, x);               \
    }                                                                                       \
  } while (0)

  int tile = tile_at(0);
  if (tile < 0) return;
  set_tile(tile);
  MXQ_GEMM_PROLOGUE_ISSUE();
  for (int it = 0;; ++it) {


    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Stage 0 (and scale group 0) landed: the previous tile's stores, issued
    // after these copies, may still be in flight behind them.
    if (nstages > 1) wait_vmcnt<kCopyOps>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();

    v4i xa[4][2], xb[4][2], ya[4][2], yb[4][2];
    uint32_t xsa[4], xsb[4], ysa[4], ysb[4];
#pragma unroll
    for (int r = 0; r < 24; ++r) MXQ_GEMM_READ(0, r, xa, xb, xsa, xsb);
    MXQ_GEMM_READ_DONE(0, xa, xb, xsa, xsb);

// Sub-stage U = 2j + ODD: its 16 matrix instructions from CA/CB/CSA/CSB, with
// the reads of sub-stage U + 1 into NA/NB/NSA/NSB spread over the first 12
// and, in odd sub-stages, the copies of stage j + 2 over all 16 (buffer j % 2
// is free: every wave passed the barrier after reading its last sub-stage).
// Even sub-stages end by waiting for stage j + 1 and a barrier.  The empty
// statement after each instruction keeps it ahead of the memory instructions
// that follow (it touches no memory, so the compiler would move it freely).
#define MXQ_GEMM_SUBSTAGE(U, ODD, CA, CB, CSA, CSB, NA, NB, NSA, NSB)                       \
    do {                                                                                    \
      const int u_ = (U);                                                                   \
      const int j_ = u_ >> 1;                                                               \
      const bool rd_ = (ODD) ? (j_ + 1 < nstages) : true;                                   \
      const bool cp_ = (ODD) && (j_ + 2 < nstages);                                         \
      _Pragma("unroll") for (int m = 0; m < 16; ++m) {                                      \
        if (cp_) {                                                                          \
          MXQ_GEMM_OP(j_ + 2, m);                                                           \
          if (m < 2) MXQ_GEMM_OP(j_ + 2, 16 + m);                                           \
        }                                                                                   \
        if (m < 12 && rd_) {                                                                \
          MXQ_GEMM_READ(u_ + 1, 2 * m, NA, NB, NSA, NSB);                                   \
          MXQ_GEMM_READ(u_ + 1, 2 * m + 1, NA, NB, NSA, NSB);                               \
        }                                                                                   \
        const int i = m >> 2, j = m & 3;                                                    \
        const v8i va = {CA[i][0].x, CA[i][0].y, CA[i][0].z, CA[i][0].w,                     \
                        CA[i][1].x, CA[i][1].y, CA[i][1].z, CA[i][1].w};                    \
        const v8i vb = {CB[j][0].x, CB[j][0].y, CB[j][0].z, CB[j][0].w,                     \
                        CB[j][1].x, CB[j][1].y, CB[j][1].z, CB[j][1].w};                    \
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc[i][j], 0, 0, 0, \
                                                                    (int)CSA[i], 0, (int)CSB[j]); \
        asm volatile("" ::"a"(acc[i][j]));                                                  \
      }                                                                                     \
      if (rd_) MXQ_GEMM_READ_DONE(u_ + 1, NA, NB, NSA, NSB);                                \
      if (!(ODD) && j_ + 1 < nstages) {                                                     \
        wait_vmcnt<0>();                                                                    \
        __builtin_amdgcn_s_barrier();                                                       \
        asm volatile("" ::: "memory");                                                      \
      }                                                                                     \
    } while (0)

    for (int u = 0; u < 2 * nstages; u += 2) {
      MXQ_GEMM_SUBSTAGE(u, 0, xa, xb, xsa, xsb, ya, yb, ysa, ysb);
      MXQ_GEMM_SUBSTAGE(u + 1, 1, ya, yb, ysa, ysb, xa, xb, xsa, xsb);
    }
#undef MXQ_GEMM_SUBSTAGE

    // Every wave is done reading this tile's LDS: the next tile's first copies
    // go out now and land while this tile's results are stored.
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int64_t em0 = m0, en0 = n0;
    tile = tile_at(it + 1);
    if (tile >= 0) {
      set_tile(tile);
      MXQ_GEMM_PROLOGUE_ISSUE();
    }

    // epilogue: lane l, register r -> row (r%4) + 8(r/4) + 4(l/32), column l%32
    const int64_t row0 = em0 + wm * 128 + 4 * fh, col0 = en0 + wn * 128 + fr;
    const bool full = em0 + kTile <= g.M && en0 + kTile <= g.N;
    if (!BF16 && full) {
      float* cb = static_cast<float*>(g.c) + row0 * g.N + col0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* crow_p = cb + (int64_t)(i * 32 + (r & 3) + 8 * (r >> 2)) * g.N;
#pragma unroll
          for (int j = 0; j < 4; ++j) __builtin_nontemporal_store(acc[i][j][r], crow_p + j * 32);
        }
    } else if (BF16 && full && (g.N & 1) == 0 && g.N <= (1 << 22)) {
      // Registers r, r + 1 (r even) hold rows R, R + 1 of this lane's column.
      // The even lane of a pair stores columns (2c, 2c + 1) of row R, the odd
      // lane those of row R + 1.  Each lane rounds its two rows to one bf16
      // pair, swaps the pair with its partner, and one byte permute picks the
      // halves it stores: (own R, partner R) on the even lane, (partner R + 1,
      // own R + 1) on the odd one.  Buffer stores over the tile: the lane's
      // byte offset in one register, the row's in a scalar, the 32-column
      // block's in the instruction (64-bit row pointers ran out of registers).
      const bool odd = (lane & 1) != 0;
      const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // bytes of {partner, own}
      const uint32_t nb = (uint32_t)g.N * 2u;                  // bytes per row of C
      const rsrc_t rc = make_rsrc(static_cast<__bf16*>(g.c) + em0 * g.N + en0, kTile * nb);
      const uint32_t lane_off = (uint32_t)(wm * 128 + 4 * fh + (odd ? 1 : 0)) * nb +
                                (uint32_t)(wn * 128 + (fr & ~1)) * 2u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row_off = (i * 32 + (r & 3) + 8 * (r >> 2)) * (int)nb;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // read the two accumulators out of their AGPRs one at a time
            // (left to itself the allocator keeps all 256 in VGPRs to feed the
            // converts, and the rest of the kernel spills)
            float lo, hi;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(lo) : "a"(acc[i][j][r]));
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(hi) : "a"(acc[i][j][r + 1]));
            const bf16x2 own = {(__bf16)lo, (__bf16)hi};
            const uint32_t ow = __builtin_bit_cast(uint32_t, own);
            const uint32_t pw = (uint32_t)__builtin_amdgcn_mov_dpp(
                (int)ow, 0xB1 /* quad_perm 1,0,3,2 */, 0xF, 0xF, true);
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(pw, ow, sel), rc,
                                                  (int)(lane_off + 64u * j), row_off,
                                                  2 /* nt */);
          }
          __builtin_amdgcn_sched_barrier(0);
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
            if (row < g.M && col < g.N) {
              if (BF16) {
                float v;  // read out of its AGPR on its own, as in the fast path
                asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(acc[i][j][r]));
                static_cast<__bf16*>(g.c)[row * g.N + col] = (__bf16)v;
              } else {
                static_cast<float*>(g.c)[row * g.N + col] = acc[i][j][r];
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (tile < 0) break;
  }
#undef MXQ_GEMM_PROLOGUE_ISSUE
#undef MXQ_GEMM_READ_DONE
#undef MXQ_GEMM_READ
#undef MXQ_GEMM_OP
#undef MXQ_GEMM_SCALE_OP
#undef MXQ_GEMM_DATA_OP
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                          const uint8_t* bs, int64_t M, int64_t N, int K, void* c, bool c_bf16,
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
  if (c_bf16)
    hipLaunchKernelGGL(k_mx_gemm<true>, dim3(groups), dim3(kGemmThreads), 0, (hipStream_t)stream, g);
  else
    hipLaunchKernelGGL(k_mx_gemm<false>, dim3(groups), dim3(kGemmThreads), 0, (hipStream_t)stream,
                       g);
  return hipGetLastError();
}

}  // namespace mxq
