// mhc_amax on gfx950: per-token composite residual map P = H_L ... H_1 and its
// Amax Gain Magnitude -- largest absolute row sum (forward gain) and column
// sum (backward gain) -- (Dubrov, "DeepSeek mHC: Manifold-Constrained
// Hyper-Connections", section "Het probleem van de samengestelde map";
// "mHC" notes on DeepSeek-V4, the composite mapping of section HC's problems).
// One lane per token keeps the n x n product in registers and multiplies each
// layer's map in from the left.  A diagnostic: tens of bytes per token-layer.
//
// Also here: the synthetic sublayer of the layer-stack workload,
// Y = 0.5 GELU(h) = 0.5 h Phi(h), elementwise in fp32.
#include "device.hpp"
#include "launch.hpp"

namespace mhc {
namespace {

template <int N>
__global__ __launch_bounds__(256) void amax_kernel(int64_t T, int L, const float* __restrict__ Hs,
                                                   float* __restrict__ amax, float* __restrict__ gfwd,
                                                   float* __restrict__ gbwd, float* __restrict__ comp) {
  constexpr int M = N * N + 2 * N;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= T) return;
  float P[N][N];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) P[i][j] = (i == j) ? 1.0f : 0.0f;
  for (int l = 0; l < L; ++l) {
    const float* A = Hs + (static_cast<int64_t>(l) * T + t) * M + N;
    float a[N][N];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) a[i][j] = A[i * N + j];
    float B[N][N];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        float acc = a[i][0] * P[0][j];
#pragma unroll
        for (int k = 1; k < N; ++k) acc = fmaf(a[i][k], P[k][j], acc);
        B[i][j] = acc;
      }
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) P[i][j] = B[i][j];
  }
  float f = 0.0f, b = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float rs = 0.0f, cs = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      rs += fabsf(P[i][j]);
      cs += fabsf(P[j][i]);
    }
    f = fmaxf(f, rs);
    b = fmaxf(b, cs);
  }
  if (gfwd) gfwd[t] = f;
  if (gbwd) gbwd[t] = b;
  if (amax) amax[t] = fmaxf(f, b);
  if (comp) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) comp[t * N * N + i * N + j] = P[i][j];
  }
}

// 0.5 GELU(v) = 0.25 v (1 + erf(v / sqrt 2)) = 0.25 v erfc(u), u = -v / sqrt 2.
// erfc by the Chebyshev-fitted formula of Press, Teukolsky, Vetterling and
// Flannery, Numerical Recipes in C (2nd ed.), section 6.2: for z >= 0,
// erfc(z) = t exp(-z^2 + P(t)) with t = 1 / (1 + z / 2) and P a degree-9
// polynomial, fractional error below 1.2e-7 for every z; erfc(-z) = 2 -
// erfc(z).  Against 1 + erff(x): no cancellation for negative v (near v = -5
// that sum was off by up to about 4% of its value, in bf16 results too), and
// no branch (erff takes one of two ranges per value, and a wave whose values
// fall in both ran both: about 60 instructions a value against about 20;
// T = 4096, d = 2560 bf16 took 12.2 us, now 10.1 us).  Evaluated in fp32 the
// result stays within 2e-5 relative, and 3e-7 absolute, of the exact value
// for |v| <= 12.
__device__ __forceinline__ float gelu_half_f(float v) {
  const float u = -v * 0.70710678118654752f;
  const float z = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float e = t * __expf(fmaf(-z, z, p));
  const float c = (u >= 0.0f) ? e : 2.0f - e;
  return 0.25f * v * c;
}

template <typename ST>
__global__ __launch_bounds__(256) void gelu_half_kernel(int64_t count, const typename ST::elem* h,
                                                        typename ST::elem* y) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t base = c * 8;
  if (base + 8 <= count) {
    Raw8<ST> r = load_raw8<ST>(h + base);
    float v[8];
    unpack8(r, v);
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = gelu_half_f(v[k]);
    store8<ST>(y + base, v);
  } else if (base < count) {
    for (int64_t i = base; i < count; ++i) {
      float v;
      if constexpr (sizeof(typename ST::elem) == 2) v = bf16_lo(h[i]);
      else v = h[i];
      v = gelu_half_f(v);
      if constexpr (sizeof(typename ST::elem) == 2) y[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
      else y[i] = v;
    }
  }
}

}  // namespace

hipError_t launch_amax(int64_t T, int n, int L, const float* Hs, float* amax, float* gfwd, float* gbwd, float* comp,
                       hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((T + 255) / 256);
  switch (n) {
    case 1: hipLaunchKernelGGL(amax_kernel<1>, dim3(blocks), dim3(256), 0, stream, T, L, Hs, amax, gfwd, gbwd, comp); break;
    case 2: hipLaunchKernelGGL(amax_kernel<2>, dim3(blocks), dim3(256), 0, stream, T, L, Hs, amax, gfwd, gbwd, comp); break;
    case 4: hipLaunchKernelGGL(amax_kernel<4>, dim3(blocks), dim3(256), 0, stream, T, L, Hs, amax, gfwd, gbwd, comp); break;
    case 8: hipLaunchKernelGGL(amax_kernel<8>, dim3(blocks), dim3(256), 0, stream, T, L, Hs, amax, gfwd, gbwd, comp); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gelu_half(int64_t count, int dtype, const void* h, void* y, hipStream_t stream) {
  if (count == 0) return hipSuccess;
  const int64_t chunks = (count + 7) / 8;
  const unsigned blocks = static_cast<unsigned>((chunks + 255) / 256);
  if (dtype == MHC_BF16)
    hipLaunchKernelGGL(gelu_half_kernel<BF16>, dim3(blocks), dim3(256), 0, stream, count,
                       static_cast<const uint16_t*>(h), static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(gelu_half_kernel<F32>, dim3(blocks), dim3(256), 0, stream, count, static_cast<const float*>(h),
                       static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace mhc
