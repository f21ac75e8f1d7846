// The C ABI of libmhc: host-side argument checks, then dispatch to the HIP
// kernels on the caller's stream.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/mhc.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxT = (int64_t{1} << 31) - 1;
constexpr int kMaxD = 1 << 20;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

size_t state_bytes(int32_t dtype) { return dtype == MHC_BF16 ? 2 : 4; }

// Common checks of mhc_params; on success fills the element counts.
mhc_status check_params(const mhc_params* p) {
  if (!p) return MHC_ERR_NULL;
  if (p->T < 0 || p->T > kMaxT) return MHC_ERR_SHAPE;
  if (p->n < 1 || p->n > 16) return MHC_ERR_SHAPE;
  if (p->d < 1 || p->d > kMaxD) return MHC_ERR_SHAPE;
  if (p->t_max < 0 || p->t_max > 1000) return MHC_ERR_SHAPE;
  if (!std::isfinite(p->eps) || p->eps < 0.0f) return MHC_ERR_SHAPE;
  if (!std::isfinite(p->alpha_pre) || !std::isfinite(p->alpha_res) || !std::isfinite(p->alpha_post))
    return MHC_ERR_SHAPE;
  if (p->dtype != MHC_FP32 && p->dtype != MHC_BF16) return MHC_ERR_DTYPE;
  if (p->maps != MHC_MAPS_MHC && p->maps != MHC_MAPS_HC) return MHC_ERR_SHAPE;
  if (p->n != 1 && p->n != 2 && p->n != 4 && p->n != 8) return MHC_ERR_UNSUPPORTED;
  if (p->d % 8 != 0) return MHC_ERR_UNSUPPORTED;
  // Element counts must fit comfortably in 64-bit byte offsets.
  const double elems = static_cast<double>(p->T) * p->n * p->d;
  if (elems * 4.0 > 9.0e18) return MHC_ERR_SHAPE;
  return MHC_OK;
}

mhc::DeviceInfo device_info() {
  // Per-device attribute cache; the only state the library keeps.
  static std::mutex mu;
  static int cus[64] = {0};
  mhc::DeviceInfo info;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  info.device = dev;
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && dev < 64) {
    if (cus[dev] == 0) {
      int v = 0;
      if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
      cus[dev] = v;
    }
    info.num_cus = cus[dev];
  }
  return info;
}

mhc_status from_hip(hipError_t e) { return e == hipSuccess ? MHC_OK : MHC_ERR_HIP; }

}  // namespace

namespace mhc {

// mhc_pre's argument checks.  With check_workspace false the workspace is
// the library's own (mhc_pre_noalloc) and is not checked here.
mhc_status check_pre_call(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* h,
                          const float* H, const void* workspace, size_t workspace_bytes, bool check_workspace) {
  mhc_status st = check_params(p);
  if (st != MHC_OK) return st;
  if (p->T == 0) return MHC_OK;
  if (!X || !phi || !bias || !h || !H) return MHC_ERR_NULL;
  const size_t need = pre_workspace_bytes(p->T, p->n, p->d);
  if (check_workspace) {
    if (need > 0 && !workspace) return MHC_ERR_WORKSPACE;
    if (workspace_bytes < need) return MHC_ERR_WORKSPACE;
  }
  if (!aligned16(X) || !aligned16(h) || !aligned16(H) || !aligned16(phi) || !aligned16(bias)) return MHC_ERR_ALIGN;
  if (check_workspace && need > 0 && !aligned16(workspace)) return MHC_ERR_ALIGN;
  const int m = p->n * p->n + 2 * p->n;
  const size_t sb = state_bytes(p->dtype);
  const Range rX = range_of(X, static_cast<size_t>(p->T) * p->n * p->d * sb);
  const Range rphi = range_of(phi, static_cast<size_t>(p->n) * p->d * m * 4);
  const Range rb = range_of(bias, static_cast<size_t>(m) * 4);
  const Range rh = range_of(h, static_cast<size_t>(p->T) * p->d * sb);
  const Range rH = range_of(H, static_cast<size_t>(p->T) * m * 4);
  if (overlap(rh, rX) || overlap(rh, rphi) || overlap(rh, rb) || overlap(rh, rH)) return MHC_ERR_ALIAS;
  if (overlap(rH, rX) || overlap(rH, rphi) || overlap(rH, rb)) return MHC_ERR_ALIAS;
  if (check_workspace && need > 0) {
    const Range rw = range_of(workspace, need);
    if (overlap(rw, rX) || overlap(rw, rphi) || overlap(rw, rb) || overlap(rw, rh) || overlap(rw, rH))
      return MHC_ERR_ALIAS;
  }
  return MHC_OK;
}

}  // namespace mhc

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

const char* mhc_status_string(int s) {
  switch (s) {
    case MHC_OK: return "ok";
    case MHC_ERR_NULL: return "a required pointer is NULL";
    case MHC_ERR_SHAPE: return "a size or hyperparameter is out of range";
    case MHC_ERR_DTYPE: return "unknown state dtype (expected MHC_FP32 or MHC_BF16)";
    case MHC_ERR_ALIGN: return "a tensor base pointer is not 16-byte aligned";
    case MHC_ERR_UNSUPPORTED: return "shape not supported (n must be 1, 2, 4 or 8, the backward n <= 4; d a multiple of 8)";
    case MHC_ERR_ALIAS: return "an output overlaps an input";
    case MHC_ERR_WORKSPACE: return "workspace missing or too small";
    case MHC_ERR_HIP: return "a HIP call or kernel launch failed";
    case MHC_ERR_SCRATCH: return "the call needs more scratch than mhc_pre_noalloc's static buffer holds";
  }
  return "unknown status";
}

size_t mhc_pre_workspace_size(const mhc_params* p) {
  if (check_params(p) != MHC_OK) return 0;
  return mhc::pre_workspace_bytes(p->T, p->n, p->d);
}

mhc_status mhc_pre(const mhc_params* p, const void* X, const float* phi, const float* bias, void* h, float* H,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return mhc_pre_ex(p, X, phi, bias, h, H, workspace, workspace_bytes, MHC_PRE_AUTO, nullptr, stream);
}

mhc_status mhc_pre_ex(const mhc_params* p, const void* X, const float* phi, const float* bias, void* h, float* H,
                      void* workspace, size_t workspace_bytes, int32_t algo, int32_t* algo_used, void* stream) {
  if (algo_used) *algo_used = MHC_PRE_TWO_PASS;
  if (algo != MHC_PRE_AUTO && algo != MHC_PRE_TWO_PASS && algo != MHC_PRE_ONE_PASS &&
      algo != MHC_PRE_ONE_PASS_FALLBACK_TEST)
    return MHC_ERR_SHAPE;
  const mhc_status st = mhc::check_pre_call(p, X, phi, bias, h, H, workspace, workspace_bytes, true);
  if (st != MHC_OK || p->T == 0) return st;
  const mhc::DeviceInfo dev = device_info();
  int used = MHC_PRE_TWO_PASS;
  const hipError_t e = mhc::launch_pre(*p, X, phi, bias, h, H, workspace, workspace_bytes, algo, &used, dev,
                                       static_cast<hipStream_t>(stream));
  if (algo_used) *algo_used = used;
  if (e == hipErrorNotSupported && algo != MHC_PRE_AUTO && algo != MHC_PRE_TWO_PASS) return MHC_ERR_UNSUPPORTED;
  return from_hip(e);
}

mhc_status mhc_post(const mhc_params* p, const void* X, const void* Y, const float* H, void* X_out, void* stream) {
  mhc_status st = check_params(p);
  if (st != MHC_OK) return st;
  if (p->T == 0) return MHC_OK;
  if (!X || !Y || !H || !X_out) return MHC_ERR_NULL;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(H) || !aligned16(X_out)) return MHC_ERR_ALIGN;
  const int m = p->n * p->n + 2 * p->n;
  const size_t sb = state_bytes(p->dtype);
  const size_t xb = static_cast<size_t>(p->T) * p->n * p->d * sb;
  const Range rX = range_of(X, xb), rY = range_of(Y, static_cast<size_t>(p->T) * p->d * sb);
  const Range rH = range_of(H, static_cast<size_t>(p->T) * m * 4), rO = range_of(X_out, xb);
  if (X_out != X && overlap(rO, rX)) return MHC_ERR_ALIAS;
  if (overlap(rO, rY) || overlap(rO, rH)) return MHC_ERR_ALIAS;
  return from_hip(mhc::launch_post(*p, X, Y, H, X_out, static_cast<hipStream_t>(stream)));
}

mhc_status mhc_post_pre(const mhc_params* p, const void* X, const void* Y, const float* H, void* X_out,
                        const float* phi, const float* bias, void* h, float* H_next, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return mhc_post_pre_ex(p, X, Y, H, X_out, phi, bias, h, H_next, workspace, workspace_bytes, MHC_PRE_AUTO, nullptr,
                         stream);
}

mhc_status mhc_post_pre_ex(const mhc_params* p, const void* X, const void* Y, const float* H, void* X_out,
                           const float* phi, const float* bias, void* h, float* H_next, void* workspace,
                           size_t workspace_bytes, int32_t algo, int32_t* algo_used, void* stream) {
  if (algo_used) *algo_used = MHC_PRE_TWO_PASS;
  if (algo != MHC_PRE_AUTO && algo != MHC_PRE_TWO_PASS && algo != MHC_PRE_ONE_PASS &&
      algo != MHC_PRE_ONE_PASS_FALLBACK_TEST)
    return MHC_ERR_SHAPE;
  mhc_status st = check_params(p);
  if (st != MHC_OK) return st;
  if (p->T == 0) return MHC_OK;
  if (!X || !Y || !H || !X_out || !phi || !bias || !h || !H_next) return MHC_ERR_NULL;
  const size_t need = mhc::pre_workspace_bytes(p->T, p->n, p->d);
  if (!workspace || workspace_bytes < need) return MHC_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(H) || !aligned16(X_out) || !aligned16(phi) || !aligned16(bias) ||
      !aligned16(h) || !aligned16(H_next) || !aligned16(workspace))
    return MHC_ERR_ALIGN;
  const int m = p->n * p->n + 2 * p->n;
  const size_t sb = state_bytes(p->dtype);
  const size_t xb = static_cast<size_t>(p->T) * p->n * p->d * sb;
  const size_t hb = static_cast<size_t>(p->T) * p->d * sb;
  const size_t mb = static_cast<size_t>(p->T) * m * 4;
  const Range rX = range_of(X, xb), rO = range_of(X_out, xb);
  if (X_out != X && overlap(rO, rX)) return MHC_ERR_ALIAS;
  const Range ins[4] = {range_of(Y, hb), range_of(H, mb), range_of(phi, static_cast<size_t>(p->n) * p->d * m * 4),
                        range_of(bias, static_cast<size_t>(m) * 4)};
  const Range outs[4] = {rO, range_of(h, hb), range_of(H_next, mb), range_of(workspace, need)};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 4; ++b)
      if (overlap(outs[a], ins[b])) return MHC_ERR_ALIAS;
    if (a > 0 && overlap(outs[a], rX)) return MHC_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return MHC_ERR_ALIAS;
  }
  const bool one_pass = algo == MHC_PRE_ONE_PASS || algo == MHC_PRE_ONE_PASS_FALLBACK_TEST;
  if (one_pass && X_out == X) return MHC_ERR_ALIAS;     // the single pass needs X_{l+1} apart from X_l
  const mhc::DeviceInfo dev = device_info();
  int used = MHC_PRE_TWO_PASS;
  const hipError_t e = mhc::launch_post_pre(*p, X, Y, H, X_out, phi, bias, h, H_next, workspace, workspace_bytes,
                                            algo, &used, dev, static_cast<hipStream_t>(stream));
  if (algo_used) *algo_used = used;
  if (e == hipErrorNotSupported && one_pass) return MHC_ERR_UNSUPPORTED;
  return from_hip(e);
}

size_t mhc_post_bwd_workspace_size(const mhc_params* p) {
  if (check_params(p) != MHC_OK) return 0;
  return mhc::post_bwd_workspace_bytes(p->T, p->n, p->d);
}

mhc_status mhc_post_bwd_ex(const mhc_params* p, const void* X, const void* Y, const float* H, const void* G,
                           void* dX, void* dY, float* dH, void* workspace, size_t workspace_bytes, void* stream) {
  mhc_status st = check_params(p);
  if (st != MHC_OK) return st;
  if (p->T == 0) return MHC_OK;
  if (p->n > 4) return MHC_ERR_UNSUPPORTED;
  if (!X || !Y || !H || !G || !dY || !dH) return MHC_ERR_NULL;      // dX may be NULL: see the header
  const size_t need = mhc::post_bwd_workspace_bytes(p->T, p->n, p->d);
  if (workspace && workspace_bytes < need) return MHC_ERR_WORKSPACE;
  if (need == 0) workspace = nullptr;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(H) || !aligned16(G) || !aligned16(dX) || !aligned16(dY) ||
      !aligned16(dH) || !aligned16(workspace))
    return MHC_ERR_ALIGN;
  const int m = p->n * p->n + 2 * p->n;
  const size_t sb = state_bytes(p->dtype);
  const size_t xb = static_cast<size_t>(p->T) * p->n * p->d * sb;
  const size_t yb = static_cast<size_t>(p->T) * p->d * sb;
  const Range ins[4] = {range_of(X, xb), range_of(Y, yb), range_of(H, static_cast<size_t>(p->T) * m * 4),
                        range_of(G, xb)};
  const Range outs[4] = {range_of(dX, dX ? xb : 0), range_of(dY, yb), range_of(dH, static_cast<size_t>(p->T) * m * 4),
                         range_of(workspace, workspace ? need : 0)};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 4; ++b)
      if (overlap(outs[a], ins[b])) return MHC_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return MHC_ERR_ALIAS;
  }
  return from_hip(mhc::launch_post_bwd(*p, X, Y, H, G, dX, dY, dH, workspace, static_cast<hipStream_t>(stream)));
}

mhc_status mhc_post_bwd(const mhc_params* p, const void* X, const void* Y, const float* H, const void* G, void* dX,
                        void* dY, float* dH, void* stream) {
  return mhc_post_bwd_ex(p, X, Y, H, G, dX, dY, dH, nullptr, 0, stream);
}

size_t mhc_pre_bwd_workspace_size(const mhc_params* p) {
  if (check_params(p) != MHC_OK || p->n > 4) return 0;
  return mhc::pre_bwd_workspace_bytes(p->T, p->n, p->d, p->dtype);
}

mhc_status mhc_pre_bwd(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* D,
                       const float* dH, void* dX, float* dphi, float* dbias, float* dalpha, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return mhc_pre_bwd_ex(p, X, phi, bias, D, dH, nullptr, dX, dphi, dbias, dalpha, workspace, workspace_bytes, stream);
}

mhc_status mhc_pre_bwd_ex(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* D,
                          const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                          void* workspace, size_t workspace_bytes, void* stream) {
  mhc_status st = check_params(p);
  if (st != MHC_OK) return st;
  if (p->n > 4 || p->t_max > mhc::pre_bwd_max_tmax() || p->maps != MHC_MAPS_MHC) return MHC_ERR_UNSUPPORTED;
  if (!dphi || !dbias || !dalpha) return MHC_ERR_NULL;
  if (p->T > 0 && (!X || !phi || !bias || !D || !dH || !dX)) return MHC_ERR_NULL;
  const size_t need = mhc::pre_bwd_workspace_bytes(p->T, p->n, p->d, p->dtype);
  if (!workspace || workspace_bytes < need) return MHC_ERR_WORKSPACE;
  if (!aligned16(X) || !aligned16(phi) || !aligned16(bias) || !aligned16(D) || !aligned16(dH) || !aligned16(dX) ||
      !aligned16(dphi) || !aligned16(dbias) || !aligned16(dalpha) || !aligned16(workspace) || !aligned16(G))
    return MHC_ERR_ALIGN;
  const bool empty = p->T == 0;
  const int m = p->n * p->n + 2 * p->n;
  const size_t sb = state_bytes(p->dtype);
  const size_t xb = static_cast<size_t>(p->T) * p->n * p->d * sb;
  const Range ins[6] = {range_of(X, xb), range_of(phi, empty ? 0 : static_cast<size_t>(p->n) * p->d * m * 4),
                        range_of(bias, empty ? 0 : static_cast<size_t>(m) * 4),
                        range_of(D, static_cast<size_t>(p->T) * p->d * sb),
                        range_of(dH, static_cast<size_t>(p->T) * m * 4), range_of(G, G ? xb : 0)};
  const Range outs[5] = {range_of(dX, xb), range_of(dphi, static_cast<size_t>(p->n) * p->d * m * 4),
                         range_of(dbias, static_cast<size_t>(m) * 4), range_of(dalpha, 3 * 4),
                         range_of(workspace, need)};
  for (int a = 0; a < 5; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(outs[a], ins[b])) return MHC_ERR_ALIAS;
    for (int b = a + 1; b < 5; ++b)
      if (overlap(outs[a], outs[b])) return MHC_ERR_ALIAS;
  }
  const mhc::DeviceInfo dev = device_info();
  return from_hip(mhc::launch_pre_bwd(*p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, workspace, dev,
                                      static_cast<hipStream_t>(stream)));
}

size_t mhc_workspace_size(const mhc_params* p, int32_t op) {
  switch (op) {
    case MHC_OP_PRE:
    case MHC_OP_POST_PRE: return mhc_pre_workspace_size(p);
    case MHC_OP_POST_BWD: return mhc_post_bwd_workspace_size(p);
    case MHC_OP_PRE_BWD: return mhc_pre_bwd_workspace_size(p);
    case MHC_OP_POST:
    case MHC_OP_AMAX:
    default: return 0;
  }
}

mhc_status mhc_amax(int64_t T, int32_t n, int32_t L, const float* H_stack, float* amax, float* gain_fwd,
                    float* gain_bwd, float* composite, void* stream) {
  if (T < 0 || T > kMaxT || n < 1 || n > 16 || L < 0) return MHC_ERR_SHAPE;
  if (n != 1 && n != 2 && n != 4 && n != 8) return MHC_ERR_UNSUPPORTED;
  if (T == 0) return MHC_OK;
  if (L > 0 && !H_stack) return MHC_ERR_NULL;
  if (!amax && !gain_fwd && !gain_bwd && !composite) return MHC_ERR_NULL;
  const int m = n * n + 2 * n;
  const Range rH = range_of(H_stack, static_cast<size_t>(L) * T * m * 4);
  const Range outs[4] = {range_of(amax, amax ? T * 4 : 0), range_of(gain_fwd, gain_fwd ? T * 4 : 0),
                         range_of(gain_bwd, gain_bwd ? T * 4 : 0),
                         range_of(composite, composite ? static_cast<size_t>(T) * n * n * 4 : 0)};
  for (int a = 0; a < 4; ++a) {
    if (L > 0 && overlap(outs[a], rH)) return MHC_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return MHC_ERR_ALIAS;
  }
  return from_hip(mhc::launch_amax(T, n, L, H_stack, amax, gain_fwd, gain_bwd, composite,
                                   static_cast<hipStream_t>(stream)));
}

mhc_status mhc_gelu_half(int64_t count, int32_t dtype, const void* h, void* Y, void* stream) {
  if (count < 0) return MHC_ERR_SHAPE;
  if (dtype != MHC_FP32 && dtype != MHC_BF16) return MHC_ERR_DTYPE;
  if (count == 0) return MHC_OK;
  if (!h || !Y) return MHC_ERR_NULL;
  if (!aligned16(h) || !aligned16(Y)) return MHC_ERR_ALIGN;
  const size_t b = static_cast<size_t>(count) * state_bytes(dtype);
  if (Y != h && overlap(range_of(Y, b), range_of(h, b))) return MHC_ERR_ALIAS;
  return from_hip(mhc::launch_gelu_half(count, dtype, h, Y, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
