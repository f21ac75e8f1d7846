// mhc_pre_noalloc: mhc_pre for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its scratch is a file-scope device array of fixed size, one
// copy per GPU, held from module load until the process ends; the call
// allocates nothing and takes no workspace argument.
//
// In host code the array's name is only a host-side stand-in: its device
// address is looked up once per device with hipGetSymbolAddress (that
// device current) and cached; kernels only ever receive that address.
//
// Every call on a GPU shares that GPU's array, which keeps the last call's
// contents.  mhc_pre needs nothing cleared: the single pass's header (error
// word, sequence number) works from any contents and carries over from one
// call to the next, and the other forms overwrite every record they read.
// Calls that overlap in time on one GPU (other streams, other host threads)
// race on the array: serialise them.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mhc.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = size_t{32} << 20;   // MHC_PRE_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MHC_PRE_NOALLOC_SCRATCH_BYTES, "the header states the limit");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of this device's copy of the array (looked up once).
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

mhc_status mhc_pre_noalloc(const mhc_params* p, const void* X, const float* phi, const float* bias, void* h,
                           float* H, void* stream) {
  // mhc_pre's checks first (the workspace being the library's own), then
  // the scratch limit, then the device address: nothing is enqueued unless
  // all of them pass.
  const mhc_status st = mhc::check_pre_call(p, X, phi, bias, h, H, nullptr, 0, false);
  if (st != MHC_OK || p->T == 0) return st;
  if (mhc_pre_workspace_size(p) > kScratchBytes) return MHC_ERR_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return MHC_ERR_HIP;
  return mhc_pre_ex(p, X, phi, bias, h, H, ws, kScratchBytes, MHC_PRE_AUTO, nullptr, stream);
}

}  // extern "C"
