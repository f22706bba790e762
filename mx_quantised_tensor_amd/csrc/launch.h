// launch.h -- internal interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

struct MxnormArgs {
  const void* x;
  const void* gamma;  // nullptr: no gain
  int64_t rows;
  int hidden;
  int p;
  float c;
  int had;     // 0, 16 or 32
  int source;  // 0: E8M0-scale block magnitudes, 1: exact block absmax
  int elem;  // 0 = E4M3, 1 = E2M1
  uint8_t* codes;
  uint8_t* scales;
  float* rrms;  // nullptr: not written
  void* stream;
};

bool row_shape_supported(int hidden);
hipError_t launch_mxnorm(const MxnormArgs& a);
hipError_t launch_mx_quant(const void* x, int64_t rows, int hidden, int elem, uint8_t* codes,
                           uint8_t* scales, void* stream);
hipError_t launch_rmsnorm(const void* x, const void* gamma, int64_t rows, int hidden, float eps,
                          void* y, float* rstd, void* stream);

// MXFP8 x MXFP8 matrix product C[M, N] = A[M, K] B[N, K]^T (K % 128 == 0),
// C fp32, or bf16 (round to nearest even) when c_bf16.
hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                          const uint8_t* bs, int64_t M, int64_t N, int K, void* c, bool c_bf16,
                          void* stream);
// MX cast of fl32(w * gamma) along rows of w (the gain folded into a weight).
hipError_t launch_mx_quant_gain(const void* w, const void* gamma, int64_t rows, int hidden,
                                int elem, uint8_t* codes, uint8_t* scales, void* stream);

// Straight-through MXNorm backward.  hidden <= kBwdMaxHidden.
constexpr int kBwdMaxHidden = 32768;
// Persistent workgroups of the backward with a gain, at most (one dgamma
// partial row each): 512 or 256 of 4 waves for rows of up to 1024 or 2048
// elements (one wave per row); then 512 of 5 waves (up to 2560), 512 of 3
// (3072), 256 of 7 (3584), 256 of 8 (4096), 512 of 2 (4608), 256 of 8
// (8192), 256 of 4 or 8 for wider rows.
constexpr int64_t kBwdMaxPartials = 512;

struct BwdLaunch {
  const void* x;
  const void* dy;
  const void* gamma;  // nullptr: no gain, no dgamma
  const float* rrms;
  int64_t rows;
  int hidden;
  void* dx;
  float* dgamma;     // required iff gamma
  float* workspace;  // bwd_groups(rows, hidden) * hidden floats, required iff gamma
  void* stream;
};

int64_t bwd_groups(int64_t rows, int hidden);
hipError_t launch_mxnorm_bwd(const BwdLaunch& l);

// Scratch of the allocation-free backward: a static device array of this many
// bytes per GPU (the largest workspace any supported shape needs: 256 partial
// rows of 32768 columns).  bwd_scratch returns its device address on `device`,
// which must be the current device; the address is looked up once per device.
constexpr size_t kBwdScratchBytes = (size_t)32 << 20;
hipError_t bwd_scratch(int device, float** out);

}  // namespace mxq
