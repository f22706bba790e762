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
  int had;   // 0, 16 or 32
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

}  // namespace mxq
