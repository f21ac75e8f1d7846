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

// mhc_pre's argument checks (capi.cpp); check_workspace false skips the
// workspace's (mhc_pre_noalloc supplies its own).
mhc_status check_pre_call(const mhc_params* p, const void* X, const float* phi, const float* bias, const void* h,
                          const float* H, const void* workspace, size_t workspace_bytes, bool check_workspace);

// mhc_post: stream mixing + broadcast-add.
hipError_t launch_post(const mhc_params& p, const void* X, const void* Y, const float* H, void* Xo,
                       hipStream_t stream);

// mhc_pre: workspace bytes and the launch.  algo: MHC_PRE_AUTO, MHC_PRE_TWO_PASS
// or MHC_PRE_ONE_PASS; *used receives the form that ran.
size_t pre_workspace_bytes(int64_t T, int n, int d);
hipError_t launch_pre(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                      float* H, void* workspace, size_t ws_bytes, int algo, int* used, const DeviceInfo& dev,
                      hipStream_t stream);

// mhc_post of layer l fused with mhc_pre of layer l+1 (pre.hip); workspace
// as mhc_pre's.  algo as launch_pre's: the single pass takes the post in
// front of it when Xout does not overlap X; *used receives the form that ran.
hipError_t launch_post_pre(const mhc_params& p, const void* X, const void* Y, const float* Hprev, void* Xout,
                           const float* phi, const float* bias, void* h, float* H, void* workspace, size_t ws_bytes,
                           int algo, int* used, const DeviceInfo& dev, hipStream_t stream);

// mhc_pre for n = 8 (pre8.hip): split-K over 64-position slices, then one
// token per wave.
size_t pre8_workspace_bytes(int64_t T, int d);
hipError_t launch_pre8(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                       void* workspace, const DeviceInfo& dev, hipStream_t stream);

// mhc_pre's workspace is a header, which only the single pass uses, then a
// body for the records of whichever form runs.  Header words (u64): [0] the
// tag of the last single-pass call whose waits ran out, [1] the sequence
// number of the next call, [2] the tag of the current call.
constexpr size_t kPreHeaderBytes = 256;

// The single-pass form (pre_fused.hip): hipErrorNotSupported when it does not
// apply.  It reads and writes the whole workspace, header included.
// force_fallback (a testing aid) makes every workgroup start as if a wait had
// run out, so the fallback kernel recomputes the call.
size_t pre_fused_body_bytes(int n, int d);
// What MHC_PRE_AUTO picks: the single pass when each team gets at least as
// many 16-token tiles as the table gives for its team size S = 8 .. 16
// (mhc_pre, then mhc_post_pre with the post in front).  The entries are the
// crossovers measured on MI355X at n = 4, T = 1024 .. 16384, ties going to
// the two-pass form.  Teams that leave CUs of an XCD idle (S = 11 and 12
// leave 10 and 8 of 32) need more tiles before the single pass wins.
constexpr int kAutoTilesPre[9] = {6, 10, 10, 24, 18, 14, 12, 12, 6};
constexpr int kAutoTilesPostPre[9] = {10, 16, 10, 48, 28, 16, 12, 12, 16};
bool pre_fused_preferred(const mhc_params& p, const DeviceInfo& dev, bool post);
hipError_t launch_pre_fused(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, size_t ws_bytes, bool force_fallback, const DeviceInfo& dev,
                            hipStream_t stream);
// The single pass with layer l's mhc_post in front: X is X_l, Xo (not
// overlapping X) receives X_{l+1}, and h, H are layer l+1's.
hipError_t launch_post_pre_fused(const mhc_params& p, const void* X, const void* Y, const float* Hp, void* Xo,
                                 const float* phi, const float* bias, void* h, float* H, void* workspace,
                                 size_t ws_bytes, bool force_fallback, const DeviceInfo& dev, hipStream_t stream);

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
// G NULL: dX += (pre's terms); G given: dX = sum_j H_res[j][i] G_j + (pre's terms),
// the residual part mhc_post_bwd then skipped (its dX NULL).
hipError_t launch_pre_bwd(const mhc_params& p, const void* X, const float* phi, const float* bias, const void* D,
                          const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                          void* workspace, const DeviceInfo& dev, hipStream_t stream);

// mhc_amax: composite-map Amax.
hipError_t launch_amax(int64_t T, int n, int L, const float* Hs, float* amax, float* gfwd, float* gbwd,
                       float* comp, hipStream_t stream);

// The stack workload's synthetic sublayer, Y = 0.5 GELU(h).
hipError_t launch_gelu_half(int64_t count, int dtype, const void* h, void* Y, hipStream_t stream);

}  // namespace mhc
