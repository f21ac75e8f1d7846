// Internal launch interface between the C ABI (capi.cpp) and the kernels.
// Arguments reaching these functions have been validated by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/mhc.h"

namespace mhc {

struct DeviceInfo {
  int device = 0;
  int num_cus = 256;       // compute units
};

// mhc_post: stream mixing + broadcast-add.
hipError_t launch_post(const mhc_params& p, const void* X, const void* Y, const float* H, void* Xo,
                       hipStream_t stream);

// mhc_pre: workspace bytes and the launch.  algo: MHC_PRE_AUTO, MHC_PRE_TWO_PASS
// or MHC_PRE_ONE_PASS; *used receives the form that ran.
size_t pre_workspace_bytes(int64_t T, int n, int d);
hipError_t launch_pre(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                      float* H, void* workspace, size_t ws_bytes, int algo, int* used, const DeviceInfo& dev,
                      hipStream_t stream);

// mhc_post of layer l fused with mhc_pre of layer l+1 (pre.hip); workspace as mhc_pre's.
hipError_t launch_post_pre(const mhc_params& p, const void* X, const void* Y, const float* Hprev, void* Xout,
                           const float* phi, const float* bias, void* h, float* H, void* workspace, const DeviceInfo& dev,
                           hipStream_t stream);

// mhc_pre for n = 8 (pre8.hip): split-K over 64-position slices, then one
// token per wave.
size_t pre8_workspace_bytes(int64_t T, int d);
hipError_t launch_pre8(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                       void* workspace, const DeviceInfo& dev, hipStream_t stream);

// The single-pass form (pre_fused.hip): hipErrorNotSupported when it does not apply.
// The first kOnePassHeaderBytes of its workspace hold the error word; its
// fallback (launch_pre_gated) keeps the two-pass records after them.
constexpr size_t kOnePassHeaderBytes = 256;
size_t pre_fused_workspace_bytes(int64_t T, int n, int d);
bool pre_fused_preferred(const mhc_params& p, const DeviceInfo& dev);   // what MHC_PRE_AUTO picks
hipError_t launch_pre_fused(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, size_t ws_bytes, const DeviceInfo& dev, hipStream_t stream);

// The two-pass form on a bf16 state (n <= 4), each kernel gated: it runs
// only if *gate == gate_value when it starts, else returns at once.  The
// records go to workspace (pre_partial_bytes of it).
hipError_t launch_pre_gated(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, const DeviceInfo& dev, const unsigned long long* gate,
                            unsigned long long gate_value, hipStream_t stream);

// Split-K partials of mhc_pre's projection plus, per stream i, <D, X_i> over
// the slice (pre.hip).  part: [S][T][pre_part_width(n, true)] floats with
// S = pre_num_slices(d); per token: m partial dot products x . phi, n partial
// <D, X_i>, and the partial sum of squares as an fp64 at float offset
// pre_part_ss_offset(n, true).
int pre_num_slices(int d);
int pre_part_width(int n, bool with_d);
int pre_part_ss_offset(int n, bool with_d);
size_t pre_partial_bytes(int64_t T, int n, int d, bool with_d);   // records + trash slots
hipError_t launch_pre_partial_with_d(const mhc_params& p, const void* X, const void* D, const float* phi, float* part,
                                     const DeviceInfo& dev, hipStream_t stream);

// Backward (bwd.hip).
// workspace: NULL for the scratch-free form, else post_bwd_workspace_bytes()
// bytes (that size is 0 where only the scratch-free form applies).
size_t post_bwd_workspace_bytes(int64_t T, int n, int d);
hipError_t launch_post_bwd(const mhc_params& p, const void* X, const void* Y, const float* H, const void* G, void* dX,
                           void* dY, float* dH, void* workspace, hipStream_t stream);
size_t pre_bwd_workspace_bytes(int64_t T, int n, int d, int dtype);
int pre_bwd_max_tmax();
hipError_t launch_pre_bwd(const mhc_params& p, const void* X, const float* phi, const float* bias, const void* D,
                          const float* dH, void* dX, float* dphi, float* dbias, float* dalpha, void* workspace,
                          const DeviceInfo& dev, hipStream_t stream);

// mhc_amax: composite-map Amax.
hipError_t launch_amax(int64_t T, int n, int L, const float* Hs, float* amax, float* gfwd, float* gbwd,
                       float* comp, hipStream_t stream);

// The stack workload's synthetic sublayer, Y = 0.5 GELU(h).
hipError_t launch_gelu_half(int64_t count, int dtype, const void* h, void* Y, hipStream_t stream);

}  // namespace mhc
