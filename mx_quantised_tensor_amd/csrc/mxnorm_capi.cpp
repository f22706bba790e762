// mxnorm_capi.cpp -- the C ABI of libmxnorm.so (declared in include/mxnorm.h):
// argument validation, defaults and kernel dispatch.  Every check runs on the
// host before anything is enqueued; the library never allocates, frees or
// synchronises.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "launch.h"
#include "mxnorm.h"

namespace {

// Default c(p, 32): Gaussian activations, log-uniform row scale, power-of-two
// block magnitudes: c = (E[M^p] (1 - 2^-p) / (p ln 2))^(1/p) with M the max of
// 32 i.i.d. |N(0,1)| (E[M] = 2.3470792, E[M^2] = 5.7095053), rounded to fp32.
constexpr float kDefaultC1 = 0x1.b16c5ep+0f;  // 1.6930598
constexpr float kDefaultC2 = 0x1.c1ed54p+0f;  // 1.7575276
// Exact block absmax: c = E[M^p]^(1/p), rounded to fp32.
constexpr float kDefaultAbsC1 = 0x1.2c6d18p+1f;  // 2.3470793
constexpr float kDefaultAbsC2 = 0x1.31d9bcp+1f;  // 2.3894572

// Limits per call that keep every launch below 2^32 threads (a workgroup of
// 256 threads per row at most; one thread per 8 elements at most).
constexpr int64_t kMaxRows = ((int64_t)1 << 24) - 1;
constexpr int64_t kMaxElems = (int64_t)1 << 34;
// The matrix product advances K in stages of 128.
constexpr int64_t kMatmulK = 128;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

mxq_status check_shape(int64_t rows, int64_t hidden, mxq_elem elem) {
  if (rows < 0 || hidden <= 0 || hidden % MXQ_BLOCK != 0) return MXQ_EINVAL;
  if (elem != MXQ_E4M3 && elem != MXQ_E2M1) return MXQ_EINVAL;
  if (hidden > MXQ_MAX_HIDDEN || !mxq::row_shape_supported((int)hidden))
    return MXQ_EUNSUPPORTED;
  if (rows > kMaxRows || rows > kMaxElems / hidden) return MXQ_EUNSUPPORTED;
  return MXQ_OK;
}

mxq_status check_mx_outputs(const void* x, const uint8_t* codes, const uint8_t* scales) {
  if (x == nullptr || codes == nullptr || scales == nullptr) return MXQ_EINVAL;
  if (!aligned(x, 16) || !aligned(codes, 16)) return MXQ_EALIGN;
  return MXQ_OK;
}

mxq_status status_of(hipError_t e) { return e == hipSuccess ? MXQ_OK : MXQ_EHIP; }

// Every argument check of mx_matmul (shapes, limits, pointers, alignment), so
// that a composed call can run them all before its first launch.  MXQ_OK with
// M == 0 or N == 0 means there is nothing to do.
mxq_status check_matmul(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                        const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, const void* c,
                        mxq_out c_type) {
  if (M < 0 || N < 0 || K <= 0 || K % MXQ_BLOCK != 0) return MXQ_EINVAL;
  if (c_type != MXQ_OUT_F32 && c_type != MXQ_OUT_BF16) return MXQ_EINVAL;
  if (K % kMatmulK != 0 || K > MXQ_MAX_HIDDEN * 4) return MXQ_EUNSUPPORTED;
  if (M > kMaxRows * 4 || N > kMaxRows * 4) return MXQ_EUNSUPPORTED;
  if (((M + 127) / 128) * ((N + 127) / 128) >= ((int64_t)1 << 31)) return MXQ_EUNSUPPORTED;
  if (M == 0 || N == 0) return MXQ_OK;
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return MXQ_EINVAL;
  if (!aligned(a_codes, 16) || !aligned(b_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(b_scales, 4) || !aligned(c, 4))
    return MXQ_EALIGN;
  return MXQ_OK;
}

mxq_status mxnorm_common(const void* x, const void* gamma, int64_t rows, int64_t hidden, int p,
                         float c, mxq_source source, int had, mxq_elem elem, uint8_t* codes,
                         uint8_t* scales, float* rrms, mxq_stream_t stream) {
  mxq_status st = check_shape(rows, hidden, elem);
  if (st != MXQ_OK) return st;
  if (p != 1 && p != 2) return MXQ_EINVAL;
  if (source != MXQ_SRC_SCALES && source != MXQ_SRC_ABSMAX) return MXQ_EINVAL;
  if (!(c >= 0.0f) || !isfinite(c)) return MXQ_EINVAL;
  if (had != 0 && had != 16 && had != 32) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  st = check_mx_outputs(x, codes, scales);
  if (st != MXQ_OK) return st;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_EALIGN;
  if (rrms != nullptr && !aligned(rrms, 4)) return MXQ_EALIGN;
  mxq::MxnormArgs a;
  a.x = x;
  a.gamma = gamma;
  a.rows = rows;
  a.hidden = (int)hidden;
  a.p = p;
  a.c = c == 0.0f ? mxnorm_default_c_for(p, source) : c;
  a.had = had;
  a.source = (int)source;
  a.elem = (int)elem;
  a.codes = codes;
  a.scales = scales;
  a.rrms = rrms;
  a.stream = stream;
  (void)hipGetLastError();  // clear an unrelated earlier error
  return status_of(mxq::launch_mxnorm(a));
}

}  // namespace

extern "C" {

mxq_status mx_quant(const void* x, int64_t rows, int64_t hidden, mxq_elem elem, uint8_t* codes,
                    uint8_t* scales, mxq_stream_t stream) {
  mxq_status st = check_shape(rows, hidden, elem);
  if (st != MXQ_OK) return st;
  if (rows == 0) return MXQ_OK;
  st = check_mx_outputs(x, codes, scales);
  if (st != MXQ_OK) return st;
  (void)hipGetLastError();
  return status_of(mxq::launch_mx_quant(x, rows, (int)hidden, (int)elem, codes, scales, stream));
}

mxq_status mxnorm_fwd(const void* x, const void* gamma, int64_t rows, int64_t hidden, int p,
                      float c, mxq_elem elem, uint8_t* codes, uint8_t* scales, float* rrms,
                      mxq_stream_t stream) {
  return mxnorm_common(x, gamma, rows, hidden, p, c, MXQ_SRC_SCALES, 0, elem, codes, scales,
                       rrms, stream);
}

mxq_status mxnorm_hadamard_fwd(const void* x, const void* gamma, int64_t rows, int64_t hidden,
                               int p, float c, int had, mxq_elem elem, uint8_t* codes,
                               uint8_t* scales, float* rrms, mxq_stream_t stream) {
  if (had != 16 && had != 32) return MXQ_EINVAL;
  return mxnorm_common(x, gamma, rows, hidden, p, c, MXQ_SRC_SCALES, had, elem, codes, scales,
                       rrms, stream);
}

mxq_status mxnorm_fwd_ex(const void* x, const void* gamma, int64_t rows, int64_t hidden, int p,
                         float c, mxq_source source, int had, mxq_elem elem, uint8_t* codes,
                         uint8_t* scales, float* rrms, mxq_stream_t stream) {
  return mxnorm_common(x, gamma, rows, hidden, p, c, source, had, elem, codes, scales, rrms,
                       stream);
}

mxq_status rmsnorm_mxquant_fwd(const void* x, const void* gamma, int64_t rows, int64_t hidden,
                               float eps, mxq_elem elem, void* y_workspace, uint8_t* codes,
                               uint8_t* scales, float* rstd, mxq_stream_t stream) {
  mxq_status st = check_shape(rows, hidden, elem);
  if (st != MXQ_OK) return st;
  if (!(eps >= 0.0f) || !isfinite(eps)) return MXQ_EINVAL;
  if (rows == 0) return MXQ_OK;
  st = check_mx_outputs(x, codes, scales);
  if (st != MXQ_OK) return st;
  if (y_workspace == nullptr) return MXQ_EINVAL;
  if (!aligned(y_workspace, 16)) return MXQ_EALIGN;
  if (gamma != nullptr && !aligned(gamma, 16)) return MXQ_EALIGN;
  if (rstd != nullptr && !aligned(rstd, 4)) return MXQ_EALIGN;
  (void)hipGetLastError();
  hipError_t e = mxq::launch_rmsnorm(x, gamma, rows, (int)hidden, eps, y_workspace, rstd, stream);
  if (e != hipSuccess) return MXQ_EHIP;
  return status_of(
      mxq::launch_mx_quant(y_workspace, rows, (int)hidden, (int)elem, codes, scales, stream));
}

mxq_status mx_quant_gain(const void* w, const void* gamma, int64_t rows, int64_t hidden,
                         mxq_elem elem, uint8_t* codes, uint8_t* scales, mxq_stream_t stream) {
  mxq_status st = check_shape(rows, hidden, elem);
  if (st != MXQ_OK) return st;
  if (rows == 0) return MXQ_OK;
  st = check_mx_outputs(w, codes, scales);
  if (st != MXQ_OK) return st;
  if (gamma == nullptr) return MXQ_EINVAL;
  if (!aligned(gamma, 16)) return MXQ_EALIGN;
  (void)hipGetLastError();
  return status_of(
      mxq::launch_mx_quant_gain(w, gamma, rows, (int)hidden, (int)elem, codes, scales, stream));
}

mxq_status mx_matmul(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                     const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* c,
                     mxq_out c_type, mxq_stream_t stream) {
  const mxq_status st = check_matmul(a_codes, a_scales, b_codes, b_scales, M, N, K, c, c_type);
  if (st != MXQ_OK || M == 0 || N == 0) return st;
  (void)hipGetLastError();
  return status_of(mxq::launch_mx_gemm(a_codes, a_scales, b_codes, b_scales, M, N, (int)K, c,
                                       c_type == MXQ_OUT_BF16, stream));
}

mxq_status mxnorm_linear_fwd(const void* x, int64_t rows, int64_t hidden, int p, float c,
                             const uint8_t* w_codes, const uint8_t* w_scales,
                             int64_t out_features, uint8_t* x_codes, uint8_t* x_scales,
                             float* rrms, void* out, mxq_out out_type, mxq_stream_t stream) {
  mxq_status st = check_shape(rows, hidden, MXQ_E4M3);
  if (st != MXQ_OK) return st;
  if (p != 1 && p != 2) return MXQ_EINVAL;
  if (!(c >= 0.0f) || !isfinite(c)) return MXQ_EINVAL;
  if (out_features < 0) return MXQ_EINVAL;
  if (out_type != MXQ_OUT_F32 && out_type != MXQ_OUT_BF16) return MXQ_EINVAL;
  if (hidden % kMatmulK != 0) return MXQ_EUNSUPPORTED;
  // the product's checks first: nothing is launched unless both calls are valid
  st = check_matmul(x_codes, x_scales, w_codes, w_scales, rows, out_features, hidden, out,
                    out_type);
  if (st != MXQ_OK) return st;
  if (rows == 0 || out_features == 0) return MXQ_OK;
  if (x == nullptr) return MXQ_EINVAL;
  if (!aligned(x, 16)) return MXQ_EALIGN;
  if (rrms != nullptr && !aligned(rrms, 4)) return MXQ_EALIGN;
  st = mxnorm_common(x, nullptr, rows, hidden, p, c, MXQ_SRC_SCALES, 0, MXQ_E4M3, x_codes,
                     x_scales, rrms, stream);
  if (st != MXQ_OK) return st;
  return mx_matmul(x_codes, x_scales, w_codes, w_scales, rows, out_features, hidden, out,
                   out_type, stream);
}

size_t mxnorm_bwd_workspace_bytes(int64_t rows, int64_t hidden) {
  if (rows < 0 || hidden <= 0 || hidden % MXQ_BLOCK != 0 || hidden > mxq::kBwdMaxHidden ||
      rows > kMaxRows)
    return 0;
  return (size_t)mxq::bwd_groups(rows, (int)hidden) * (size_t)hidden * sizeof(float);
}

}  // extern "C"

namespace {

// mxnorm_bwd's argument checks; the workspace is checked only if `check_ws`.
mxq_status check_bwd(const void* x, const void* dy, const void* gamma, const float* rrms,
                     int64_t rows, int64_t hidden, const void* dx, const float* dgamma,
                     bool check_ws, const float* workspace) {
  if (rows < 0 || hidden <= 0 || hidden % MXQ_BLOCK != 0) return MXQ_EINVAL;
  if (hidden > mxq::kBwdMaxHidden || rows > kMaxRows || rows > kMaxElems / hidden)
    return MXQ_EUNSUPPORTED;
  if (gamma != nullptr) {
    if (dgamma == nullptr || (check_ws && rows > 0 && workspace == nullptr)) return MXQ_EINVAL;
    if (!aligned(gamma, 16) || !aligned(dgamma, 4) || (check_ws && !aligned(workspace, 16)))
      return MXQ_EALIGN;
  }
  if (rows > 0) {
    if (x == nullptr || dy == nullptr || rrms == nullptr || dx == nullptr) return MXQ_EINVAL;
    if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || !aligned(rrms, 4))
      return MXQ_EALIGN;
  }
  return MXQ_OK;
}

}  // namespace

extern "C" {

mxq_status mxnorm_bwd(const void* x, const void* dy, const void* gamma, const float* rrms,
                      int64_t rows, int64_t hidden, void* dx, float* dgamma, float* workspace,
                      mxq_stream_t stream) {
  const mxq_status st = check_bwd(x, dy, gamma, rrms, rows, hidden, dx, dgamma, true, workspace);
  if (st != MXQ_OK) return st;
  if (rows == 0 && gamma == nullptr) return MXQ_OK;  // nothing to do
  mxq::BwdLaunch l;
  l.x = x;
  l.dy = dy;
  l.gamma = gamma;
  l.rrms = rrms;
  l.rows = rows;
  l.hidden = (int)hidden;
  l.dx = dx;
  l.dgamma = dgamma;
  l.workspace = workspace;
  l.stream = stream;
  (void)hipGetLastError();
  return status_of(mxq::launch_mxnorm_bwd(l));
}

mxq_status mxnorm_bwd_noalloc(const void* x, const void* dy, const void* gamma, const float* rrms,
                              int64_t rows, int64_t hidden, void* dx, float* dgamma,
                              mxq_stream_t stream) {
  mxq_status st = check_bwd(x, dy, gamma, rrms, rows, hidden, dx, dgamma, false, nullptr);
  if (st != MXQ_OK) return st;
  float* ws = nullptr;
  if (gamma != nullptr && rows > 0) {
    if (mxnorm_bwd_workspace_bytes(rows, hidden) > mxq::kBwdScratchBytes) return MXQ_EUNSUPPORTED;
    // the scratch of the device the work runs on, which must be the current one
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return MXQ_EHIP;
    if (stream != nullptr) {
      hipDevice_t sdev = -1;
      if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return MXQ_EHIP;
      if ((int)sdev != dev) return MXQ_EINVAL;
    }
    if (mxq::bwd_scratch(dev, &ws) != hipSuccess) return MXQ_EHIP;
  }
  return mxnorm_bwd(x, dy, gamma, rrms, rows, hidden, dx, dgamma, ws, stream);
}

size_t mxnorm_bwd_noalloc_scratch_bytes(void) { return mxq::kBwdScratchBytes; }

float mxnorm_default_c(int p) {
  if (p == 1) return kDefaultC1;
  if (p == 2) return kDefaultC2;
  return 0.0f;
}

float mxnorm_default_c_for(int p, mxq_source source) {
  if (source == MXQ_SRC_SCALES) return mxnorm_default_c(p);
  if (source != MXQ_SRC_ABSMAX) return 0.0f;
  if (p == 1) return kDefaultAbsC1;
  if (p == 2) return kDefaultAbsC2;
  return 0.0f;
}

const char* mxq_status_str(mxq_status s) {
  switch (s) {
    case MXQ_OK: return "MXQ_OK";
    case MXQ_EINVAL: return "MXQ_EINVAL: invalid argument";
    case MXQ_EALIGN: return "MXQ_EALIGN: pointer misaligned";
    case MXQ_EUNSUPPORTED: return "MXQ_EUNSUPPORTED: shape outside the library's limits";
    case MXQ_EHIP: return "MXQ_EHIP: HIP launch failed";
  }
  return "MXQ_UNKNOWN";
}

const char* mxq_version(void) { return "mxnorm-gfx950 0.1.0"; }

}  // extern "C"
