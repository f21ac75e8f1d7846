// mhc_post on gfx950: X'[t, i, :] = sum_j H_res[t, i, j] X[t, j, :] + H_post[t, i] Y[t, :]
// (Dubrov, "DeepSeek mHC: Manifold-Constrained Hyper-Connections", section
// "Kernmechanismen", Eq. 3; "mHC" notes on DeepSeek-V4, eq. dsv4-mhc-hc-update
// and the fused Post-Res kernel of table tbl-dsv4-mhc-kernels, which reads
// (n+1) C values per token instead of (3n+1) C).
//
// Pure streaming, bound by HBM: each thread owns chunks of 8 consecutive
// values of d and, for each, reads the chunk of all n streams of X plus the
// chunk of Y (16-byte non-temporal loads), combines them in fp32 registers and
// writes the n output chunks (16-byte non-temporal stores).  A chunk of X is
// read before it is written by the same thread, so X' may be X itself.
// When d/8 is a multiple of 64 (d a multiple of 512) the tiled kernel runs: a
// workgroup covers 4 tokens x 512 values of d, one token per wave, and
// consecutive workgroups walk along d before moving to the next 4 tokens.  The
// token index is then wave-uniform and the n*n + n map values come in through
// scalar loads.  On MI355X this order streams faster than giving a
// workgroup whole tokens (a layout probe moving the same bytes: 180 us
// against 211 us at T = 16384, n = 4, d = 4096).
#include "device.hpp"
#include "launch.hpp"

namespace mhc {
namespace {

constexpr int POST_THREADS = 256;

template <typename ST, int N, int IPT>
__global__ __launch_bounds__(POST_THREADS) void post_kernel(int64_t nchunks, int d8,
                                                            const typename ST::elem* __restrict__ X,
                                                            const typename ST::elem* __restrict__ Y,
                                                            const float* __restrict__ H,
                                                            typename ST::elem* Xo) {
  constexpr int M = N * N + 2 * N;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t group0 = (static_cast<int64_t>(blockIdx.x) * (POST_THREADS / 64) + wave) * IPT;
  const int64_t d = static_cast<int64_t>(d8) * 8;

  Raw8<ST> xr[IPT][N];
  Raw8<ST> yr[IPT];
  int64_t tok[IPT];
  int64_t off[IPT];
  bool ok[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    int64_t c = (group0 + k) * 64 + lane;
    ok[k] = c < nchunks;
    int64_t t = c / d8;
    tok[k] = t;
    off[k] = (c - t * d8) * 8;
    if (ok[k]) {
#pragma unroll
      for (int i = 0; i < N; ++i) xr[k][i] = load_raw8<ST, true>(X + (t * N + i) * d + off[k]);
      yr[k] = load_raw8<ST, true>(Y + t * d + off[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    if (!ok[k]) continue;
    const float* Ht = H + tok[k] * M;
    float res[N][N], post[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int j = 0; j < N; ++j) res[i][j] = Ht[N + i * N + j];
      post[i] = Ht[N + N * N + i];
    }
    float x[N][8], y[8];
#pragma unroll
    for (int i = 0; i < N; ++i) unpack8(xr[k][i], x[i]);
    unpack8(yr[k], y);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float acc = res[i][0] * x[0][e];
#pragma unroll
        for (int j = 1; j < N; ++j) acc = fmaf(res[i][j], x[j][e], acc);
        o[e] = fmaf(post[i], y[e], acc);
      }
      store8<ST, true>(Xo + (tok[k] * N + i) * d + off[k], o);
    }
  }
}

template <typename ST, int N>
__global__ __launch_bounds__(POST_THREADS) void post_tile_kernel(int64_t T, int d8, int nslice,
                                                                 const typename ST::elem* __restrict__ X,
                                                                 const typename ST::elem* __restrict__ Y,
                                                                 const float* __restrict__ H,
                                                                 typename ST::elem* Xo) {
  constexpr int M = N * N + 2 * N;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int b = static_cast<int>(blockIdx.x);
  const int tile = b / nslice;
  const int slice = b - tile * nslice;
  const int64_t t = static_cast<int64_t>(tile) * (POST_THREADS / 64) + wave;     // wave-uniform
  if (t >= T) return;
  const int64_t d = static_cast<int64_t>(d8) * 8;
  const int64_t off = (static_cast<int64_t>(slice) * 64 + lane) * 8;
  Raw8<ST> xr[N], yr;
#pragma unroll
  for (int i = 0; i < N; ++i) xr[i] = load_raw8<ST, true>(X + (t * N + i) * d + off);
  yr = load_raw8<ST, true>(Y + t * d + off);
  const float* Ht = H + t * M;
  float res[N][N], post[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < N; ++j) res[i][j] = Ht[N + i * N + j];
    post[i] = Ht[N + N * N + i];
  }
  float x[N][8], y[8];
#pragma unroll
  for (int i = 0; i < N; ++i) unpack8(xr[i], x[i]);
  unpack8(yr, y);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = res[i][0] * x[0][e];
#pragma unroll
      for (int j = 1; j < N; ++j) acc = fmaf(res[i][j], x[j][e], acc);
      o[e] = fmaf(post[i], y[e], acc);
    }
    store8<ST, true>(Xo + (t * N + i) * d + off, o);
  }
}

template <typename ST, int N>
hipError_t launch_post_t(const mhc_params& p, const void* X, const void* Y, const float* H, void* Xo,
                         hipStream_t stream) {
  typedef typename ST::elem E;
  constexpr int IPT = N >= 8 ? 1 : 2;   // chunks per thread in flight
  const int d8 = p.d / 8;
  const int64_t nchunks = p.T * d8;
  const int64_t per_block = static_cast<int64_t>(POST_THREADS) * IPT;
  const int64_t blocks = (nchunks + per_block - 1) / per_block;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (d8 % 64 == 0) {
    const int nslice = d8 / 64;
    const int64_t tiles = (p.T + POST_THREADS / 64 - 1) / (POST_THREADS / 64);
    if (tiles * nslice > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((post_tile_kernel<ST, N>), dim3(static_cast<unsigned>(tiles * nslice)), dim3(POST_THREADS), 0,
                       stream, p.T, d8, nslice, static_cast<const E*>(X), static_cast<const E*>(Y), H,
                       static_cast<E*>(Xo));
  } else {
    hipLaunchKernelGGL((post_kernel<ST, N, IPT>), dim3(static_cast<unsigned>(blocks)), dim3(POST_THREADS), 0,
                       stream, nchunks, d8, static_cast<const E*>(X), static_cast<const E*>(Y), H,
                       static_cast<E*>(Xo));
  }
  return hipGetLastError();
}

template <typename ST>
hipError_t launch_post_n(const mhc_params& p, const void* X, const void* Y, const float* H, void* Xo,
                         hipStream_t stream) {
  switch (p.n) {
    case 1: return launch_post_t<ST, 1>(p, X, Y, H, Xo, stream);
    case 2: return launch_post_t<ST, 2>(p, X, Y, H, Xo, stream);
    case 4: return launch_post_t<ST, 4>(p, X, Y, H, Xo, stream);
    case 8: return launch_post_t<ST, 8>(p, X, Y, H, Xo, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_post(const mhc_params& p, const void* X, const void* Y, const float* H, void* Xo,
                       hipStream_t stream) {
  if (p.dtype == MHC_BF16) return launch_post_n<BF16>(p, X, Y, H, Xo, stream);
  return launch_post_n<F32>(p, X, Y, H, Xo, stream);
}

}  // namespace mhc
