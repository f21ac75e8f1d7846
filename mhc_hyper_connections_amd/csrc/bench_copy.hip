// A plain streaming copy, the bandwidth reference the benchmark reports
// beside the mHC kernels and the known-size kernel that scales rocprofv3's
// HBM byte counters.  Not part of libmhc: it is built into libmhc_bench.so.
//
// Each 256-thread workgroup moves one contiguous 4 KiB block: one 16-byte
// non-temporal load per thread, then one non-temporal store.  Consecutive
// workgroups take consecutive blocks, so the workgroups dispatched together
// stream neighbouring memory.  On MI355X this shape copied the 512 MiB
// state at 6.4-6.5 TB/s, against 6.0-6.1 TB/s for 16 KiB per workgroup
// (four chunks per thread) and 6.2 TB/s for 8 KiB.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kPer = 1;                                   // 16-byte chunks per thread
constexpr size_t kBlockBytes = static_cast<size_t>(kThreads) * kPer * 16;

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst, size_t nchunks) {
  const size_t base = static_cast<size_t>(blockIdx.x) * (kThreads * kPer) + threadIdx.x;
  u32x4 v[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const size_t i = base + static_cast<size_t>(k) * kThreads;
    v[k] = i < nchunks ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const size_t i = base + static_cast<size_t>(k) * kThreads;
    if (i < nchunks) __builtin_nontemporal_store(v[k], dst + i);
  }
}

}  // namespace

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned device
// pointers, not overlapping) on `stream` (a hipStream_t, NULL = default).
// Returns 0, or 1 for invalid arguments, 2 when the launch failed.
int mhc_bench_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return 0;
  if (!src || !dst || (bytes & 15u) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(dst) & 15u) != 0)
    return 1;
  const size_t nchunks = bytes / 16;
  const size_t blocks = (bytes + kBlockBytes - 1) / kBlockBytes;
  if (blocks > 0x7fffffffu) return 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                     nchunks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
