// Backward of the mHC layer on gfx950: mhc_post_bwd and mhc_pre_bwd.
//
// The pages state only that the layer is trained with a custom backward that
// recomputes the maps instead of storing them ("mHC" notes on DeepSeek-V4,
// table tbl-dsv4-mhc-mixed-precision and the kernel notes; Dubrov, "DeepSeek
// mHC: Manifold-Constrained Hyper-Connections", on the training cost).  The
// formulas below are the chain rule of the forward (post.hip, pre.hip):
//
//   post:  X'_i = sum_j H_res[i][j] X_j + H_post[i] Y
//          dX_j = sum_i H_res[i][j] G_i      dY = sum_i H_post[i] G_i
//          dH_res[i][j] = <G_i, X_j>         dH_post[i] = <G_i, Y>
//   pre:   h = sum_i H_pre[i] X_i
//          dX_i += H_pre[i] D               dH_pre[i] = <D, X_i>
//          maps: sigmoid / 2 sigmoid gates, Sinkhorn reversed over its 2 t_max
//          normalisations (for B = A / s over one line: dA = (dB - <dB, B>) / s),
//          exp -> dl = dlogits;  dz = alpha_blk dl
//          dphi += x_hat dz^T, dbias += dl, dalpha_blk += <dl_blk, z_blk>
//          dx += phi dz / r - (z . dz) x / (K r^2)       (RMSNorm, K = n d)
//
// mhc_pre_bwd runs four launches:
//   A. the forward's split-K partial kernel, extended with <D, X_i>
//      (pre.hip): per slice and token, x . phi, <D, X_i> and sum x^2;
//   B. per token (16 lanes): sums the partials in a fixed order, recomputes
//      r, the logits, gates and Sinkhorn (iterates kept in LDS) and runs the
//      maps' backward; writes g = dz / r, H_pre and (z . dz) / (K r^2) for C,
//      and the token's dlogits and alpha terms for D;
//   C. streams X, D and dX once more: dX += H_pre D + phi g - coef x, and
//      accumulates this chunk of tokens' share of dphi = sum_t x_t g_t^T; in
//      the whole-dX form (G given, mhc_post_bwd having skipped dX) it reads G
//      instead of dX and writes dX = sum_j H_res[j][i] G_j + the same terms;
//   D. fixed-order reductions of the dphi chunks and of dbias, dalpha over T.
#include <type_traits>

#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

// Per-token record written by B for C, 48 floats: g (m) | H_pre (n) | coef |
// zeros up to 32 (one MFMA K-block of g for n <= 4), then H_res by columns,
// H_res[row][col] at 32 + 4 col + row (zeros past n), for C's whole-dX form.
__host__ __device__ constexpr int tok_width(int) { return 48; }
constexpr int kResCol = 32;               // record offset of H_res's columns
// Per-token values written by B for D, column-major [pg_width][Tpad]:
// dlogits (m columns), then the alpha terms pre, res, post.
__host__ __device__ constexpr int pg_width(int n) { return num_maps(n) + 3; }

constexpr int kBwdMaxTmax = 128;          // Sinkhorn iterates kept in LDS: 2 t_max floats per lane
constexpr int APPLY_THREADS = 256;
constexpr int APPLY_CH = 64;              // token records staged per batch in kernel C

// ---- mhc_post_bwd -------------------------------------------------------------
// One wave per token: lanes walk the token's chunks of 8 values, write dX and
// dY, and accumulate the n*n + n dot products, reduced across the wave at the
// end.  H is read with wave-uniform (scalar) loads.
template <typename ST, int N, bool WRITE_DX>
__global__ __launch_bounds__(256) void post_bwd_kernel(int64_t T, int d, const typename ST::elem* __restrict__ X,
                                                       const typename ST::elem* __restrict__ Y,
                                                       const float* __restrict__ H,
                                                       const typename ST::elem* __restrict__ G,
                                                       typename ST::elem* __restrict__ dX,
                                                       typename ST::elem* __restrict__ dY, float* __restrict__ dH) {
  constexpr int M = num_maps(N);
  constexpr int NN = N * N;
  constexpr int NA = NN + N;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                       // wave-uniform
  const float* Ht = H + t * M;
  float res[N][N], post[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < N; ++j) res[i][j] = Ht[N + i * N + j];
    post[i] = Ht[N + NN + i];
  }
  float acc[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = 0.0f;
  const int d8 = d / 8;
  const int64_t xrow = t * N * static_cast<int64_t>(d);
  const int64_t yrow = t * static_cast<int64_t>(d);
  for (int c = lane; c < d8; c += 64) {
    const int64_t off = static_cast<int64_t>(c) * 8;
    Raw8<ST> xr[N], gr[N], yr;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      xr[i] = load_raw8<ST, true>(X + xrow + static_cast<int64_t>(i) * d + off);
      gr[i] = load_raw8<ST, true>(G + xrow + static_cast<int64_t>(i) * d + off);
    }
    yr = load_raw8<ST, true>(Y + yrow + off);
    float x[N][8], g[N][8], y[8];
#pragma unroll
    for (int i = 0; i < N; ++i) {
      unpack8(xr[i], x[i]);
      unpack8(gr[i], g[i]);
    }
    unpack8(yr, y);
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int j = 0; j < N; ++j) {
        float a = acc[i * N + j];
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf(g[i][e], x[j][e], a);
        acc[i * N + j] = a;
      }
      float a = acc[NN + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(g[i][e], y[e], a);
      acc[NN + i] = a;
    }
    if constexpr (WRITE_DX) {
#pragma unroll
      for (int j = 0; j < N; ++j) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float s = res[0][j] * g[0][e];
#pragma unroll
          for (int i = 1; i < N; ++i) s = fmaf(res[i][j], g[i][e], s);
          o[e] = s;
        }
        store8<ST, true>(dX + xrow + static_cast<int64_t>(j) * d + off, o);
      }
    }
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float s = post[0] * g[0][e];
#pragma unroll
      for (int i = 1; i < N; ++i) s = fmaf(post[i], g[i][e], s);
      o[e] = s;
    }
    store8<ST, true>(dY + yrow + off, o);
  }
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    float v = acc[a];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    acc[a] = v;
  }
  if (lane < NA) {
    float v = acc[0];
#pragma unroll
    for (int a = 1; a < NA; ++a) v = (lane == a) ? acc[a] : v;
    dH[t * M + N + lane] = v;               // res (row-major) then post: columns N .. M-1
  }
}

// The NA sums of v[0..NA) over a wave's 64 lanes by a transposed butterfly:
// in each exchange (lane distance 32, 16, ..., 1) a lane keeps half of the
// values it still carries (the upper half if its lane bit is set), adds its
// partner's copy of that half, and hands over the other half; 22 exchanges
// for NA = 20 instead of 6 NA.  Every value still takes the plain butterfly's
// additions in its order, so the sums are bitwise those of reducing each
// value on its own.  Returns the lane's sum and sets a to its index, or -1
// for lanes left with padding.
template <int NA>
__device__ __forceinline__ float wave_sums_transposed(const float (&v)[NA], int lane, int& a) {
  constexpr int C0 = NA, C1 = (C0 + 1) / 2, C2 = (C1 + 1) / 2, C3 = (C2 + 1) / 2, C4 = (C3 + 1) / 2,
                C5 = (C4 + 1) / 2, C6 = (C5 + 1) / 2;
  static_assert(C6 == 1, "at most 64 values");
  float w0[C0];
#pragma unroll
  for (int k = 0; k < C0; ++k) w0[k] = v[k];
  float w1[C1], w2[C2], w3[C3], w4[C4], w5[C5], w6[C6];
  auto stage = [&](auto& src, auto& dst, int c, int h, int mask) {
    const bool up = (lane & mask) != 0;
#pragma unroll
    for (int k = 0; k < h; ++k) {
      const float lo = src[k];
      const float hi = (h + k < c) ? src[h + k] : 0.0f;
      dst[k] = (up ? hi : lo) + __shfl_xor(up ? lo : hi, mask);
    }
  };
  stage(w0, w1, C0, C1, 32);
  stage(w1, w2, C1, C2, 16);
  stage(w2, w3, C2, C3, 8);
  stage(w3, w4, C3, C4, 4);
  stage(w4, w5, C4, C5, 2);
  stage(w5, w6, C5, C6, 1);
  // The lane's slot back through the stages: an upper half adds its offset.
  int i = 0;
  bool ok = true;
  const int cs[7] = {C0, C1, C2, C3, C4, C5, C6};
#pragma unroll
  for (int j = 5; j >= 0; --j) {                 // stage j exchanged over lane bit 5 - j
    if (lane & (1 << (5 - j))) i += cs[j + 1];
    ok = ok && i < cs[j];
  }
  a = ok ? i : -1;
  return w6[0];
}

// The tiled form (d a multiple of 512, with a workspace): a workgroup covers
// 4 tokens x 512 values of d, one token per wave, and consecutive workgroups
// walk along d, the order in which MI355X streams fastest (as for mhc_post).
// A token's n*n + n dot products are then split over its d / 512 slices: each
// wave reduces its slice's across its lanes and writes them to the workspace,
// part[t][slice][a], and a second kernel adds the slices in order into dH.
template <typename ST, int N, bool WRITE_DX>
__global__ __launch_bounds__(256) void post_bwd_tile_kernel(int64_t T, int d8, int nslice,
                                                            const typename ST::elem* __restrict__ X,
                                                            const typename ST::elem* __restrict__ Y,
                                                            const float* __restrict__ H,
                                                            const typename ST::elem* __restrict__ G,
                                                            typename ST::elem* __restrict__ dX,
                                                            typename ST::elem* __restrict__ dY,
                                                            float* __restrict__ part) {
  constexpr int M = num_maps(N);
  constexpr int NN = N * N;
  constexpr int NA = NN + N;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int b = static_cast<int>(blockIdx.x);
  const int tile = b / nslice;
  const int slice = b - tile * nslice;
  const int64_t t = static_cast<int64_t>(tile) * 4 + wave;          // wave-uniform
  if (t >= T) return;
  const int64_t d = static_cast<int64_t>(d8) * 8;
  const int64_t off = (static_cast<int64_t>(slice) * 64 + lane) * 8;
  const int64_t xrow = t * N * d;
  Raw8<ST> xr[N], gr[N], yr;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    xr[i] = load_raw8<ST, true>(X + xrow + static_cast<int64_t>(i) * d + off);
    gr[i] = load_raw8<ST, true>(G + xrow + static_cast<int64_t>(i) * d + off);
  }
  yr = load_raw8<ST, true>(Y + t * d + off);
  const float* Ht = H + t * M;
  float res[N][N], post[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < N; ++j) res[i][j] = Ht[N + i * N + j];
    post[i] = Ht[N + NN + i];
  }
  float x[N][8], g[N][8], y[8];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    unpack8(xr[i], x[i]);
    unpack8(gr[i], g[i]);
  }
  unpack8(yr, y);
  float acc[NA];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      float a = g[i][0] * x[j][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) a = fmaf(g[i][e], x[j][e], a);
      acc[i * N + j] = a;
    }
    float a = g[i][0] * y[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) a = fmaf(g[i][e], y[e], a);
    acc[NN + i] = a;
  }
  if constexpr (WRITE_DX) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float sum = res[0][j] * g[0][e];
#pragma unroll
        for (int i = 1; i < N; ++i) sum = fmaf(res[i][j], g[i][e], sum);
        o[e] = sum;
      }
      store8<ST, true>(dX + xrow + static_cast<int64_t>(j) * d + off, o);
    }
  }
  {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sum = post[0] * g[0][e];
#pragma unroll
      for (int i = 1; i < N; ++i) sum = fmaf(post[i], g[i][e], sum);
      o[e] = sum;
    }
    store8<ST, true>(dY + t * d + off, o);
  }
  int a;
  const float v = wave_sums_transposed<NA>(acc, lane, a);
  if (a >= 0) part[(t * nslice + slice) * NA + a] = v;
}

// dH[t][n + a] = sum over slices, in slice order, of part[t][slice][a].
template <int N>
__global__ __launch_bounds__(256) void post_bwd_reduce_kernel(int64_t T, int nslice, const float* __restrict__ part,
                                                              float* __restrict__ dH) {
  constexpr int M = num_maps(N);
  constexpr int NA = N * N + N;
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q >= T * NA) return;
  const int64_t t = q / NA;
  const int a = static_cast<int>(q - t * NA);
  const float* src = part + t * nslice * NA + a;
  // Slices in order; eight loads out before their sums (a loop with one load
  // per trip waits for each in turn).  Indices past the last slice are
  // clamped to a valid one and their values dropped.
  float v = src[0];
  for (int sl = 1; sl < nslice; sl += 8) {
    const int nb = (nslice - sl < 8) ? nslice - sl : 8;
    float w[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) w[u] = src[static_cast<int64_t>(sl + (u < nb ? u : 0)) * NA];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < nb) v += w[u];
  }
  dH[t * M + N + a] = v;
}

}  // namespace

size_t post_bwd_workspace_bytes(int64_t T, int n, int d) {
  if (T <= 0 || d % 512 != 0 || n > 4) return 0;
  return static_cast<size_t>(T) * static_cast<size_t>(d / 512) * static_cast<size_t>(n * n + n) * sizeof(float);
}

namespace {

template <typename ST, int N>
hipError_t launch_post_bwd_t(const mhc_params& p, const void* X, const void* Y, const float* H, const void* G,
                             void* dX, void* dY, float* dH, void* workspace, hipStream_t stream) {
  typedef typename ST::elem E;
  constexpr int NA = N * N + N;
  if (workspace != nullptr && post_bwd_workspace_bytes(p.T, N, p.d) > 0) {
    const int nslice = p.d / 512;
    const int64_t blocks = (p.T + 3) / 4 * nslice;
    const int64_t rblocks = (p.T * NA + 255) / 256;
    if (blocks > 0x7FFFFFFF || rblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    float* part = static_cast<float*>(workspace);
    if (dX != nullptr)
      hipLaunchKernelGGL((post_bwd_tile_kernel<ST, N, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                         p.T, p.d / 8, nslice, static_cast<const E*>(X), static_cast<const E*>(Y), H,
                         static_cast<const E*>(G), static_cast<E*>(dX), static_cast<E*>(dY), part);
    else
      hipLaunchKernelGGL((post_bwd_tile_kernel<ST, N, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                         p.T, p.d / 8, nslice, static_cast<const E*>(X), static_cast<const E*>(Y), H,
                         static_cast<const E*>(G), static_cast<E*>(dX), static_cast<E*>(dY), part);
    hipLaunchKernelGGL((post_bwd_reduce_kernel<N>), dim3(static_cast<unsigned>(rblocks)), dim3(256), 0, stream, p.T,
                       nslice, part, dH);
    return hipGetLastError();
  }
  const int64_t blocks = (p.T + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (dX != nullptr)
    hipLaunchKernelGGL((post_bwd_kernel<ST, N, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p.T,
                       p.d, static_cast<const E*>(X), static_cast<const E*>(Y), H, static_cast<const E*>(G),
                       static_cast<E*>(dX), static_cast<E*>(dY), dH);
  else
    hipLaunchKernelGGL((post_bwd_kernel<ST, N, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, p.T,
                       p.d, static_cast<const E*>(X), static_cast<const E*>(Y), H, static_cast<const E*>(G),
                       static_cast<E*>(dX), static_cast<E*>(dY), dH);
  return hipGetLastError();
}

// ---- mhc_pre_bwd, launch B: the maps' backward, 16 lanes per token ------------
// Also writes g transposed in blocks of 32 tokens, gT[t / 32][j][t % 32]
// (j < 32, zero for j >= m and for the padding tokens T <= t < Tpad), the
// operand layout of the dphi contraction over tokens in launch C.
// REG: t_max <= kRegTmax, the iterates stay in registers (no LDS, so more
// waves per CU hide the latency of the serial Sinkhorn chain); otherwise
// they go to LDS.
constexpr int kRegTmax = 20;

// Sum over the 16 lanes of a token, the same bits on every lane: quads
// (partners e^1, e^2), then the quad pairs (rotation by 8 within the row),
// then the other pair (rotation by 4: either direction reaches it).  DPP, not
// lane permutes through the LDS unit, which sat on the serial chain.
__device__ __forceinline__ float sum16(float v) {
  v = v + lane_xor1(v);
  v = v + lane_xor2(v);
  v = v + lane_rot8(v);
  return v + lane_rot4(v);
}

// Four tokens per wave; with REG four waves per workgroup (a quarter of the
// workgroups to dispatch: 2.5 us less at T = 16384), otherwise one, whose
// iterates then fill the LDS.
constexpr int token_waves(bool reg) { return reg ? 4 : 1; }

template <int N, bool REG>
__global__ __launch_bounds__(64 * token_waves(REG)) void pre_bwd_token_kernel(int64_t T, int64_t Tpad, int d, int S, int PW, int SSO,
                                                           const float* __restrict__ part,
                                                           const float* __restrict__ bias, float a_pre,
                                                           float a_res, float a_post, float eps, int t_max,
                                                           const float* __restrict__ dH, float* __restrict__ tok,
                                                           float* __restrict__ gT, float* __restrict__ pg) {
  extern __shared__ float iters[];          // [2 t_max][64]: Sinkhorn matrix before each normalisation
  constexpr int M = num_maps(N);
  constexpr int NN = N * N;
  constexpr int TW = tok_width(N);
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4;
  const int e = lane & 15;
  const int64_t t = (static_cast<int64_t>(blockIdx.x) * token_waves(REG) + (threadIdx.x >> 6)) * 4 + q;
  const bool tv = t < T;
  const int colr = N + e;
  const int colg = (e < N) ? e : (N + NN + (e - N));
  const bool is_res = e < NN;
  const bool is_gate = e < 2 * N;

  // The slices' partials, summed in slice order; loaded SB slices at a time
  // (all loads of a batch out before any sum), not one latency per slice.
  constexpr int SB = 8;
  double ss = 0.0, zr = 0.0, zg = 0.0, dp = 0.0;
  if (tv) {
    for (int s0 = 0; s0 < S; s0 += SB) {
      double vss[SB];
      float vr[SB], vg[SB], vd[SB];
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int s = s0 + u;
        vss[u] = 0.0;
        vr[u] = vg[u] = vd[u] = 0.0f;
        if (s < S) {
          const float* P = part + (static_cast<int64_t>(s) * T + t) * PW;
          vss[u] = *reinterpret_cast<const double*>(P + SSO);
          if (is_res) vr[u] = P[colr];
          if (is_gate) vg[u] = P[colg];
          if (e < N) vd[u] = P[M + e];
        }
      }
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        if (s0 + u < S) {
          ss += vss[u];
          if (is_res) zr += vr[u];
          if (is_gate) zg += vg[u];
          if (e < N) dp += vd[u];
        }
      }
    }
  }
  const double inv_r = inv_rms(ss, N * d, eps);

  // Forward maps, as in the forward kernel.
  const float a_gate = (e < N) ? a_pre : a_post;
  float sg = 0.0f;
  if (is_gate) sg = sigmoidf_(logit_of(zg, inv_r, a_gate, bias[colg]));
  float lr = -INFINITY;
  if (is_res) lr = logit_of(zr, inv_r, a_res, bias[colr]);
  // The forward's Sinkhorn (the same max, sums and order: H_res comes out
  // bitwise as the forward wrote it), with the iterates kept.
  float mx = lr;
  if constexpr (NN >= 4) {
    mx = fmaxf(mx, lane_xor1(mx));
    mx = fmaxf(mx, lane_xor2(mx));
  }
  if constexpr (NN >= 16) {
    mx = fmaxf(mx, lane_rot8(mx));
    mx = fmaxf(mx, lane_rot4(mx));
  }
  if (t_max == 0) mx = 0.0f;
  const float m0 = is_res ? expf(lr - mx) : 0.0f;
  float mv = m0;
  float itr[REG ? 2 * kRegTmax : 1];
  auto put = [&](int k, float v) {
    if constexpr (REG) itr[k] = v;
    else iters[k * 64 + lane] = v;
  };
  auto get = [&](int k) -> float {
    if constexpr (REG) return itr[k];
    else return iters[k * 64 + lane];
  };
  auto sk_pass = [&](int it) {
    put(2 * it, mv);
    mv = mv / col_sum<N>(mv);
    put(2 * it + 1, mv);
    mv = mv / row_sum<N>(mv);
  };
  if constexpr (REG) {
#pragma unroll
    for (int it = 0; it < kRegTmax; ++it)
      if (it < t_max) sk_pass(it);
  } else {
    for (int it = 0; it < t_max; ++it) sk_pass(it);
  }

  // Gradients arriving at the maps: res and post from mhc_post_bwd, pre from <D, X_i>.
  float dm = (is_res && tv) ? dH[t * M + colr] : 0.0f;
  float dgate = 0.0f;
  if (e < N) dgate = static_cast<float>(dp);
  else if (is_gate && tv) dgate = dH[t * M + colg];

  // Sinkhorn in reverse.  Step 2 it normalised columns, step 2 it + 1 rows.
  auto sk_back = [&](int st) {
    const float A = get(st);
    const bool col = (st & 1) == 0;     // wave-uniform
    const float sum = col ? col_sum<N>(A) : row_sum<N>(A);
    const float B = A / sum;
    const float dot = col ? col_sum<N>(dm * B) : row_sum<N>(dm * B);
    dm = (dm - dot) / sum;
  };
  if constexpr (REG) {
#pragma unroll
    for (int st = 2 * kRegTmax - 1; st >= 0; --st)
      if (st < 2 * t_max) sk_back(st);
  } else {
    for (int st = 2 * t_max - 1; st >= 0; --st) sk_back(st);
  }
  // exp: the per-token max shift cancels (it scales M0 and dM0 inversely).
  const float dl_res = is_res ? dm * m0 : 0.0f;
  const float dsg = (e < N) ? sg * (1.0f - sg) : 2.0f * sg * (1.0f - sg);
  const float dl_gate = is_gate ? dgate * dsg : 0.0f;

  const float z_res = static_cast<float>(zr * inv_r);
  const float z_gate = static_cast<float>(zg * inv_r);
  const float dz_res = a_res * dl_res;
  const float dz_gate = a_gate * dl_gate;
  float zdz = (is_res ? z_res * dz_res : 0.0f) + (is_gate ? z_gate * dz_gate : 0.0f);
  float tpre = (e < N) ? dl_gate * z_gate : 0.0f;
  float tres = is_res ? dl_res * z_res : 0.0f;
  float tpost = (is_gate && e >= N) ? dl_gate * z_gate : 0.0f;
  zdz = sum16(zdz);
  tpre = sum16(tpre);
  tres = sum16(tres);
  tpost = sum16(tpost);
  if (t >= Tpad) return;
  float* gblk = gT + (t >> 5) * 32 * 32 + (t & 31);
  if (!tv) {                                   // padding token: zero operand column and sums
    gblk[e * 32] = 0.0f;
    gblk[(e + 16) * 32] = 0.0f;
    if (e < pg_width(N)) pg[e * Tpad + t] = 0.0f;
    if (e + 16 < pg_width(N)) pg[(e + 16) * Tpad + t] = 0.0f;
    return;
  }
  const float ir = static_cast<float>(inv_r);
  float* rec = tok + t * TW;
  float* pcol = pg + t;                       // column-major: column c at pg + c * Tpad
  if (is_res) {
    const float gv = dz_res * ir;
    rec[colr] = gv;
    gblk[colr * 32] = gv;
    pcol[colr * Tpad] = dl_res;
  }
  if (is_gate) {
    const float gv = dz_gate * ir;
    rec[colg] = gv;
    gblk[colg * 32] = gv;
    pcol[colg * Tpad] = dl_gate;
  }
  if (M + e < 32) gblk[(M + e) * 32] = 0.0f;
  if (M + 16 + e < 32) gblk[(M + 16 + e) * 32] = 0.0f;
  if (e < N) rec[M + e] = sg;                 // H_pre
  if (e == 0) {
    rec[M + N] = static_cast<float>(static_cast<double>(zdz) * inv_r * inv_r / static_cast<double>(N * d));
    pcol[(M + 0) * Tpad] = tpre;
    pcol[(M + 1) * Tpad] = tres;
    pcol[(M + 2) * Tpad] = tpost;
  }
  if (M + N + 1 + e < kResCol) rec[M + N + 1 + e] = 0.0f;
  if (M + N + 17 + e < kResCol) rec[M + N + 17 + e] = 0.0f;
  // H_res as recomputed above, by columns: lane e writes word e, entry
  // (row e % 4, column e / 4), which lane row * n + column of the token holds.
  {
    const int col = e >> 2, row = e & 3;
    const bool in = row < N && col < N;
    const float hv = __shfl(mv, (lane & ~15) + (in ? row * N + col : 0));
    rec[kResCol + e] = in ? hv : 0.0f;
  }
}

// ---- launch C: dX update and chunked dphi, one position per thread ------------
// Block (x, y): positions k = x * 256 + thread of vec(X) (k = i d + c), tokens
// of chunk y.  Each thread keeps its row of phi and its 24 dphi sums.  With G
// (the whole-dX form) the thread forms mhc_post_bwd's residual part
// sum_j H_res[j][i] G_j itself instead of reading it from dX.
template <typename ST, int N>
__global__ __launch_bounds__(APPLY_THREADS) void pre_bwd_apply_kernel(int64_t T, int d, int64_t tchunk,
                                                                      const typename ST::elem* __restrict__ X,
                                                                      const typename ST::elem* __restrict__ D,
                                                                      const float* __restrict__ phi,
                                                                      const float* __restrict__ tok,
                                                                      const typename ST::elem* __restrict__ G,
                                                                      typename ST::elem* __restrict__ dX,
                                                                      float* __restrict__ dphi_part) {
  constexpr int M = num_maps(N);
  constexpr int TW = tok_width(N);
  __shared__ float rec[APPLY_CH][TW];
  const int K = N * d;
  const int k = blockIdx.x * APPLY_THREADS + threadIdx.x;
  const bool kv = k < K;
  const int kk = kv ? k : 0;
  const int i = kk / d;
  const int c = kk - i * d;
  float ph[M], acc[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    ph[j] = phi[static_cast<int64_t>(kk) * M + j];
    acc[j] = 0.0f;
  }
  const int64_t t_begin = static_cast<int64_t>(blockIdx.y) * tchunk;
  const int64_t t_end = (t_begin + tchunk < T) ? t_begin + tchunk : T;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += APPLY_CH) {
    const int nt = static_cast<int>((t_end - t0 < APPLY_CH) ? t_end - t0 : APPLY_CH);
    __syncthreads();
    for (int q = threadIdx.x; q < nt * TW; q += APPLY_THREADS) rec[q / TW][q % TW] = tok[t0 * TW + q];
    __syncthreads();
    if (!kv) continue;
    for (int tt = 0; tt < nt; ++tt) {
      const int64_t t = t0 + tt;
      const float x = static_cast<float>(load_elem<ST>(X, t * K + k));
      const float dd = static_cast<float>(load_elem<ST>(D, t * d + c));
      float v;
      if (G != nullptr) {
        v = rec[tt][kResCol + 4 * i] * static_cast<float>(load_elem<ST>(G, t * K + c));
#pragma unroll
        for (int q = 1; q < N; ++q)
          v = fmaf(rec[tt][kResCol + 4 * i + q], static_cast<float>(load_elem<ST>(G, t * K + q * d + c)), v);
      } else {
        v = static_cast<float>(load_elem<ST>(dX, t * K + k));
      }
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < M; ++j) {
        const float g = rec[tt][j];
        s = fmaf(ph[j], g, s);
        acc[j] = fmaf(x, g, acc[j]);
      }
      v += fmaf(rec[tt][M + i], dd, s - rec[tt][M + N] * x);
      store_elem<ST>(dX, t * K + k, v);
    }
  }
  if (!kv) return;
  float* out = dphi_part + (static_cast<int64_t>(blockIdx.y) * K + k) * M;
#pragma unroll
  for (int j = 0; j < M; ++j) out[j] = acc[j];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(int64_t count, float* __restrict__ out) {
  const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (q < count) out[q] = 0.0f;
}

// ---- launch C on MFMA (bf16 state) -----------------------------------------------
// Workgroup (slice s, token chunk y): the 256 positions s*256 .. +255 of every
// stream (32 per wave, 8 per lane as in the forward's partial kernel) for the
// chunk's tokens, 16 per tile.
//  * dX update: the lane's 8 positions of one token need (phi g)[k] =
//    sum_j phi[k][j] g[t][j].  One 16x16x32 MFMA block computes 16 phi rows x
//    16 tokens with j as the contraction; the phi rows are loaded in the
//    order that puts output rows 4 (lane/16) + v of block b at positions
//    8 (lane/16) + 4 b + v, i.e. exactly the lane's load-layout positions, so
//    the result is added to x, D and dX in registers.  phi and g enter as two
//    bf16 halves each (hi + lo; the lo x lo product is dropped): ~2^-16
//    relative, so the term stays accurate where it cancels against the others.
//  * dphi += x^T g: a contraction over tokens, so x goes through a wave-local
//    LDS tile of 16 tokens (written in load layout, read as 4 tokens of one
//    position per lane for a 16x16x16 MFMA); g comes from the transposed copy
//    gT.  x is exact in bf16, g = hi + lo, fp32 accumulation.
//  The phi operands live in LDS (the registers hold two tiles in flight and
//  the dphi accumulators); lanes whose 8 columns are all past m hold zeros
//  and are not stored.
constexpr int AM_WAVES = 8;
constexpr int AM_THREADS = AM_WAVES * 64;
constexpr int AM_SLICE = AM_WAVES * 32;
// The tile's X and D go through LDS: loaded with each instruction covering 2
// token rows x 512 bytes (wave w: tokens 2w, 2w+1, lane = 16-byte chunk of
// the slice; on MI355X that streams faster than 16 rows x 64 bytes), read
// back in the MFMA layouts.  16 bytes of padding per token put the 16
// tokens of a read on distinct banks.

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_bf16(const float (&f)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(f[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(f[e] - static_cast<float>(h));
  }
}

__device__ __forceinline__ void split_bf16x4(const f32x4& f, s16x4& hi, s16x4& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const __bf16 h = static_cast<__bf16>(f[e]);
    hi[e] = __builtin_bit_cast(short, h);
    lo[e] = __builtin_bit_cast(short, static_cast<__bf16>(f[e] - static_cast<float>(h)));
  }
}

template <int N>
struct ApplyTile {
  Raw8<BF16> x[N], dv;
  f32x4 ga, gb;          // g[t][8 (lane/16) .. +7]
  float hp[N];           // H_pre[t][i]
  float coef;            // (z . dz) / (K r^2)
  f32x4 gt[(num_maps(N) + 15) / 16];   // gT operand of the tile's dphi block
};

// WHOLE: dX is written, not added to: mhc_post_bwd's residual part
// sum_j H_res[j][i] G_j is formed here from G (read where dX would be) and the
// token records' H_res columns.
template <int N, bool WHOLE>
__global__ __launch_bounds__(AM_THREADS) void pre_bwd_apply_mfma_kernel(int64_t T, int d, int64_t tchunk,
                                                                        const uint16_t* __restrict__ X,
                                                                        const uint16_t* __restrict__ D,
                                                                        const float* __restrict__ phi,
                                                                        const float* __restrict__ tok,
                                                                        const float* __restrict__ gT,
                                                                        const uint16_t* __restrict__ G,
                                                                        uint16_t* __restrict__ dX,
                                                                        float* __restrict__ dphi_part) {
  constexpr int M = num_maps(N);
  constexpr int TW = tok_width(N);
  constexpr int NJB = (M + 15) / 16;
  constexpr int NGQ = (M + 7) / 8;                 // lane groups with any column j < m
  constexpr int STS = (N + 1) * 512 + 16;          // LDS bytes per token: n streams, D, padding
  __shared__ __attribute__((aligned(16))) unsigned char stage_l[16 * STS];
  __shared__ bf16x8 phl[AM_WAVES][N][2][NGQ * 16][2];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int c0w = blockIdx.x * AM_SLICE + 32 * w;
  const int j0 = c0w + 8 * g;
  const bool jv = j0 < d;
  const int jl = jv ? j0 : 0;
  // Load layout: token row trow of the tile, 8 positions at jl0.
  const int trow = 2 * w + (lane >> 5);
  const int jl0 = blockIdx.x * AM_SLICE + 8 * (lane & 31);
  const bool jvl = jl0 < d;
  const int jll = jvl ? jl0 : 0;
  const bool gq = g < NGQ;
  const int lq = gq ? lane : 0;

  if (gq) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int pos = c0w + 8 * (r16 >> 2) + 4 * b + (r16 & 3);
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int col = 8 * g + e;
          f[e] = (pos < d && col < M) ? phi[static_cast<int64_t>(i * d + pos) * M + col] : 0.0f;
        }
        bf16x8 hi, lo;
        split_bf16(f, hi, lo);
        phl[w][i][b][lane][0] = hi;
        phl[w][i][b][lane][1] = lo;
      }
    }
  }
  f32x4 acc[2 * N][NJB];
#pragma unroll
  for (int a = 0; a < 2 * N; ++a) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) acc[a][jb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  __syncthreads();

  const int64_t t_begin = static_cast<int64_t>(blockIdx.y) * tchunk;
  const int64_t t_end = (t_begin + tchunk < T) ? t_begin + tchunk : T;
  const int64_t ntile = (t_end - t_begin + 15) / 16;

  auto load = [&](int64_t q, ApplyTile<N>& b) {
    const int64_t tl = t_begin + q * 16 + trow;
    const int64_t ttl = tl < t_end ? tl : 0;
#pragma unroll
    for (int i = 0; i < N; ++i) b.x[i] = load_raw8<BF16>(X + (ttl * N + i) * d + jll);
    b.dv = load_raw8<BF16>(D + ttl * d + jll);
    const int64_t t = t_begin + q * 16 + r16;
    const int64_t tt = t < t_end ? t : 0;
    const float* rec = tok + tt * TW;
    b.ga = *reinterpret_cast<const f32x4*>(rec + 8 * g);
    b.gb = *reinterpret_cast<const f32x4*>(rec + 8 * g + 4);
#pragma unroll
    for (int i = 0; i < N; ++i) b.hp[i] = rec[M + i];
    b.coef = rec[M + N];
    // With the tile, not later: load completions are counted in order, so a
    // load issued after the next prefetch would make its wait drain that too.
    int64_t t0 = t_begin + q * 16;
    if (t0 >= t_end) t0 = t_begin;                       // padding tile of an odd count: x is zero
    const float* gblk = gT + (t0 >> 5) * 32 * 32 + (t0 & 31) + 4 * g;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) b.gt[jb] = *reinterpret_cast<const f32x4*>(gblk + (16 * jb + r16) * 32);
  };

  // dX of a tile (read, added to, written back), or G in the whole-dX form:
  // two buffers, each loaded with its tile, two tiles ahead of its use.
  // The whole-dX form loads, with G, column lane/16 of the token's H_res.
  const uint16_t* const rsrc = WHOLE ? G : dX;
  f32x4 hc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto load_dx = [&](int64_t q, Raw8<BF16> (&dxo)[N]) {
    const int64_t t = t_begin + q * 16 + r16;
    const int64_t tt = t < t_end ? t : 0;
#pragma unroll
    for (int i = 0; i < N; ++i) dxo[i] = load_raw8<BF16>(rsrc + (tt * N + i) * d + jl);
    if constexpr (WHOLE) hc = *reinterpret_cast<const f32x4*>(tok + tt * TW + kResCol + 4 * g);
  };

  auto step = [&](int64_t q, ApplyTile<N>& b, const Raw8<BF16> (&dxo)[N]) {
    const int64_t t = t_begin + q * 16 + r16;
    const bool ok = t < t_end && jv;
    {
      // Through LDS: zeros for tokens past the chunk and positions past d
      // (the dphi contraction below reads them), then the A layout back.
      const bool okl = t_begin + q * 16 + trow < t_end && jvl;
      unsigned char* row = stage_l + trow * STS + (lane & 31) * 16;
#pragma unroll
      for (int i = 0; i < N; ++i)
        *reinterpret_cast<u32x4*>(row + i * 512) = okl ? b.x[i].v : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(row + N * 512) = okl ? b.dv.v : u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
      const unsigned char* rd = stage_l + r16 * STS + (32 * w + 8 * g) * 2;
#pragma unroll
      for (int i = 0; i < N; ++i) b.x[i].v = *reinterpret_cast<const u32x4*>(rd + i * 512);
      b.dv.v = *reinterpret_cast<const u32x4*>(rd + N * 512);
    }
    float gf[8] = {b.ga[0], b.ga[1], b.ga[2], b.ga[3], b.gb[0], b.gb[1], b.gb[2], b.gb[3]};
    bf16x8 ghi, glo;
    split_bf16(gf, ghi, glo);
    float dv[8];
    unpack8(b.dv, dv);
    const bf16x8 zero8 = {};
#pragma unroll
    for (int i = 0; i < N; ++i) {
      f32x4 o[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const bf16x8 ahi = gq ? phl[w][i][bb][lq][0] : zero8;
        const bf16x8 alo = gq ? phl[w][i][bb][lq][1] : zero8;
        f32x4 c = {0.0f, 0.0f, 0.0f, 0.0f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, ghi, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, glo, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, ghi, c, 0, 0, 0);
        o[bb] = c;
      }
      float x[8], xo[8], r[8];
      unpack8(b.x[i], x);
      if constexpr (WHOLE) {
        // Column i of H_res from lane 16 i + r16 (same token), then
        // sum_q H_res[q][i] G_q in q order.
        float hcol[N];
#pragma unroll
        for (int q = 0; q < N; ++q)
          hcol[q] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (16 * i + r16), __float_as_int(hc[q])));
        float gq[8];
        unpack8(dxo[0], gq);
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[e] = hcol[0] * gq[e];
#pragma unroll
        for (int q = 1; q < N; ++q) {
          unpack8(dxo[q], gq);
#pragma unroll
          for (int e = 0; e < 8; ++e) xo[e] = fmaf(hcol[q], gq[e], xo[e]);
        }
      } else {
        unpack8(dxo[i], xo);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r[e] = xo[e] + fmaf(b.hp[i], dv[e], o[0][e] - b.coef * x[e]);
        r[4 + e] = xo[4 + e] + fmaf(b.hp[i], dv[4 + e], o[1][e] - b.coef * x[4 + e]);
      }
      if (ok) store8<BF16>(dX + (t * N + i) * d + j0, r);     // the one branch around memory: a store
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // No barrier before the contraction: the staged tile was written before
  // the step's barrier and only read since.  The barrier after it lets the
  // next step overwrite the stage.
  auto dphi_tile = [&](const ApplyTile<N>& b) {
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      s16x4 bhi, blo;
      split_bf16x4(b.gt[jb], bhi, blo);
#pragma unroll
      for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          s16x4 a;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            a[u] = *reinterpret_cast<const short*>(stage_l + (4 * g + u) * STS + i * 512 + (32 * w + 16 * bb + r16) * 2);
          f32x4 c = acc[2 * i + bb][jb];
          c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, blo, c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bhi, c, 0, 0, 0);
          acc[2 * i + bb][jb] = c;
        }
      }
    }
    __syncthreads();
  };

  // Tiles in pairs, every prefetch unconditional (tiles past the chunk read
  // token 0 and store nothing): no load behind a branch, so the compiler's
  // waits drain only the buffer about to be used.
  ApplyTile<N> ta, tb;
  if constexpr (WHOLE) {
    // One G buffer, loaded a tile ahead at the end of each step: two would
    // not fit beside the residual's sums.
    Raw8<BF16> da[N];
    load(0, ta);
    load_dx(0, da);
    load(1, tb);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t q = 0; q < ntile; q += 2) {
      step(q, ta, da);
      load_dx(q + 1, da);
      __builtin_amdgcn_sched_barrier(0);
      dphi_tile(ta);
      load(q + 2, ta);
      __builtin_amdgcn_sched_barrier(0);
      step(q + 1, tb, da);
      load_dx(q + 2, da);
      __builtin_amdgcn_sched_barrier(0);
      dphi_tile(tb);
      load(q + 3, tb);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    Raw8<BF16> da[N], db[N];
    load(0, ta);
    load_dx(0, da);
    load(1, tb);
    load_dx(1, db);
    __builtin_amdgcn_sched_barrier(0);
    for (int64_t q = 0; q < ntile; q += 2) {
      step(q, ta, da);
      dphi_tile(ta);
      load(q + 2, ta);
      load_dx(q + 2, da);
      __builtin_amdgcn_sched_barrier(0);
      step(q + 1, tb, db);
      dphi_tile(tb);
      load(q + 3, tb);
      load_dx(q + 3, db);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  float* out = dphi_part + static_cast<int64_t>(blockIdx.y) * N * static_cast<int64_t>(d) * M;
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int col = 16 * jb + r16;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int pos = c0w + 16 * bb + 4 * g + v;
          if (pos < d && col < M) out[static_cast<int64_t>(i * d + pos) * M + col] = acc[2 * i + bb][jb][v];
        }
      }
    }
  }
}

// ---- launch D: fixed-order reductions ------------------------------------------
// One launch for both: blocks 0 .. nbc-1 sum dphi's chunk partials, the
// next m + 3 blocks the columns of pg.
//  * dphi[k][j] = sum over chunks in order.
//  * Column sums of pg [W][Tpad] over tokens: one block per column, thread k
//    adds tokens k, k + 256, ... (coalesced), then a fixed tree.  Columns
//    0 .. m-1 go to dbias, m .. m+2 to dalpha.
__global__ __launch_bounds__(256) void reduce_grads_kernel(int64_t count, int nch, int64_t nbc,
                                                           const float* __restrict__ part, float* __restrict__ out,
                                                           int64_t Tpad, int m, const float* __restrict__ pg,
                                                           float* __restrict__ dbias, float* __restrict__ dalpha) {
  __shared__ float red[256];
  if (static_cast<int64_t>(blockIdx.x) < nbc) {                       // block-uniform
    const int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (q >= count) return;
    // Chunks in order, eight loads out before their sums (indices past the
    // last chunk clamped, their values dropped).
    float s = 0.0f;
    for (int ch = 0; ch < nch; ch += 8) {
      const int nb = (nch - ch < 8) ? nch - ch : 8;
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = part[static_cast<int64_t>(ch + (u < nb ? u : 0)) * count + q];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < nb) s += w[u];
    }
    out[q] = s;
    return;
  }
  const int col = static_cast<int>(blockIdx.x - nbc);
  const float* c = pg + static_cast<int64_t>(col) * Tpad;
  float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
  int64_t t = threadIdx.x;
  // Four rounds' sixteen loads out before their sums, added in the order the
  // round-by-round loop below adds them.
  for (; t + 3 * 1024 + 768 < Tpad; t += 4096) {
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = c[t + 256 * u];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      s0 += v[4 * k];
      s1 += v[4 * k + 1];
      s2 += v[4 * k + 2];
      s3 += v[4 * k + 3];
    }
  }
  for (; t + 768 < Tpad; t += 1024) {
    s0 += c[t];
    s1 += c[t + 256];
    s2 += c[t + 512];
    s3 += c[t + 768];
  }
  for (; t < Tpad; t += 256) s0 += c[t];
  red[threadIdx.x] = (s0 + s1) + (s2 + s3);
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (col < m) dbias[col] = red[0];
    else dalpha[col - m] = red[0];
  }
}

int64_t kblocks_of(int64_t K) { return (K + APPLY_THREADS - 1) / APPLY_THREADS; }

// Workspace layout of mhc_pre_bwd (each part 256-byte aligned).
struct BwdLayout {
  size_t part, tok, gT, pg, dphi, total;
  int S, PW, SSO, nch;
  int64_t tchunk, Tpad;
};

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

BwdLayout bwd_layout(int64_t T, int n, int d, int dtype) {
  BwdLayout L{};
  const int m = num_maps(n);
  const int64_t K = static_cast<int64_t>(n) * d;
  L.S = pre_num_slices(d);
  L.PW = pre_part_width(n, true);
  L.SSO = pre_part_ss_offset(n, true);
  L.Tpad = (T + 31) / 32 * 32;
  // Token chunks of launch C.  bf16 (MFMA form): one workgroup per slice and
  // chunk, ~256 workgroups (one round: a workgroup fills a compute unit's
  // LDS; measured 6% faster than two rounds of 512, and half the dphi
  // partials), chunks a multiple of 32 tokens.  fp32: blocks of 256
  // positions, ~2048 blocks, chunks of at least 64 tokens.
  int64_t nch, unit;
  if (dtype == MHC_BF16) {
    nch = (256 + L.S - 1) / L.S;
    unit = 32;
  } else {
    const int64_t kblocks = kblocks_of(K);
    nch = (2048 + kblocks - 1) / kblocks;
    unit = APPLY_CH;
  }
  const int64_t max_ch = (T + unit - 1) / unit;
  if (nch > max_ch) nch = max_ch;
  if (nch < 1) nch = 1;
  L.tchunk = (T + nch - 1) / nch;
  L.tchunk = (L.tchunk + unit - 1) / unit * unit;
  if (L.tchunk < unit) L.tchunk = unit;
  L.nch = static_cast<int>((T + L.tchunk - 1) / L.tchunk);
  if (L.nch < 1) L.nch = 1;
  size_t off = 0;
  L.part = off;
  off = align256(off + pre_partial_bytes(T, n, d, true));
  L.tok = off;
  off = align256(off + static_cast<size_t>(T) * tok_width(n) * sizeof(float));
  L.gT = off;
  off = align256(off + static_cast<size_t>(L.Tpad) * 32 * sizeof(float));
  L.pg = off;
  off = align256(off + static_cast<size_t>(L.Tpad) * pg_width(n) * sizeof(float));
  L.dphi = off;
  off = align256(off + static_cast<size_t>(L.nch) * K * m * sizeof(float));
  L.total = off;
  return L;
}

template <typename ST, int N>
hipError_t launch_pre_bwd_t(const mhc_params& p, const void* X, const float* phi, const float* bias, const void* D,
                            const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                            void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  typedef typename ST::elem E;
  constexpr int M = num_maps(N);
  const BwdLayout L = bwd_layout(p.T, N, p.d, p.dtype);
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part);
  float* tok = reinterpret_cast<float*>(ws + L.tok);
  float* gT = reinterpret_cast<float*>(ws + L.gT);
  float* pg = reinterpret_cast<float*>(ws + L.pg);
  float* dphi_part = reinterpret_cast<float*>(ws + L.dphi);
  const int64_t K = static_cast<int64_t>(N) * p.d;
  if (p.T == 0) {                            // sums over no tokens
    const int64_t count = K * M;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, stream,
                       count, dphi);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, stream, static_cast<int64_t>(M), dbias);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, stream, static_cast<int64_t>(3), dalpha);
    return hipGetLastError();
  }

  hipError_t err = launch_pre_partial_with_d(p, X, D, phi, part, dev, stream);
  if (err != hipSuccess) return err;

  const int64_t tblocks = (L.Tpad + 3) / 4;
  if (tblocks > 0x7FFFFFFF || kblocks_of(K) > 0x7FFFFFFF) return hipErrorInvalidValue;
  const size_t lds = static_cast<size_t>(2 * (p.t_max > 0 ? p.t_max : 1)) * 64 * sizeof(float);
  if (tblocks > 0) {
    constexpr int TW4 = token_waves(true);
    if (p.t_max <= kRegTmax)
      hipLaunchKernelGGL((pre_bwd_token_kernel<N, true>), dim3(static_cast<unsigned>((tblocks + TW4 - 1) / TW4)),
                         dim3(64 * TW4), 0, stream,
                         p.T, L.Tpad, p.d, L.S, L.PW, L.SSO, static_cast<const float*>(part), bias, p.alpha_pre,
                         p.alpha_res, p.alpha_post, p.eps, p.t_max, dH, tok, gT, pg);
    else
      hipLaunchKernelGGL((pre_bwd_token_kernel<N, false>), dim3(static_cast<unsigned>(tblocks)), dim3(64), lds, stream,
                         p.T, L.Tpad, p.d, L.S, L.PW, L.SSO, static_cast<const float*>(part), bias, p.alpha_pre,
                         p.alpha_res, p.alpha_post, p.eps, p.t_max, dH, tok, gT, pg);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }

  if (std::is_same<ST, BF16>::value) {
    if (G != nullptr)
      hipLaunchKernelGGL((pre_bwd_apply_mfma_kernel<N, true>), dim3(static_cast<unsigned>(L.S), static_cast<unsigned>(L.nch)),
                         dim3(AM_THREADS), 0, stream, p.T, p.d, L.tchunk, static_cast<const uint16_t*>(X),
                         static_cast<const uint16_t*>(D), phi, static_cast<const float*>(tok),
                         static_cast<const float*>(gT), static_cast<const uint16_t*>(G), static_cast<uint16_t*>(dX),
                         dphi_part);
    else
      hipLaunchKernelGGL((pre_bwd_apply_mfma_kernel<N, false>), dim3(static_cast<unsigned>(L.S), static_cast<unsigned>(L.nch)),
                         dim3(AM_THREADS), 0, stream, p.T, p.d, L.tchunk, static_cast<const uint16_t*>(X),
                         static_cast<const uint16_t*>(D), phi, static_cast<const float*>(tok),
                         static_cast<const float*>(gT), static_cast<const uint16_t*>(nullptr),
                         static_cast<uint16_t*>(dX), dphi_part);
  } else {
    const int64_t kblocks = kblocks_of(K);
    hipLaunchKernelGGL((pre_bwd_apply_kernel<ST, N>), dim3(static_cast<unsigned>(kblocks), static_cast<unsigned>(L.nch)),
                       dim3(APPLY_THREADS), 0, stream, p.T, p.d, L.tchunk, static_cast<const E*>(X),
                       static_cast<const E*>(D), phi, static_cast<const float*>(tok), static_cast<const E*>(G),
                       static_cast<E*>(dX), dphi_part);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int64_t count = K * M;
  const int64_t nbc = (count + 255) / 256;
  if (nbc + pg_width(N) > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(reduce_grads_kernel, dim3(static_cast<unsigned>(nbc + pg_width(N))), dim3(256), 0, stream, count,
                     L.nch, nbc, static_cast<const float*>(dphi_part), dphi, L.Tpad, M, static_cast<const float*>(pg),
                     dbias, dalpha);
  return hipGetLastError();
}

template <typename ST>
hipError_t launch_pre_bwd_n(const mhc_params& p, const void* X, const float* phi, const float* bias, const void* D,
                            const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                            void* ws, const DeviceInfo& dev, hipStream_t stream) {
  switch (p.n) {
    case 1: return launch_pre_bwd_t<ST, 1>(p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, ws, dev, stream);
    case 2: return launch_pre_bwd_t<ST, 2>(p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, ws, dev, stream);
    case 4: return launch_pre_bwd_t<ST, 4>(p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, ws, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_post_bwd(const mhc_params& p, const void* X, const void* Y, const float* H, const void* G, void* dX,
                           void* dY, float* dH, void* workspace, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const bool bf = p.dtype == MHC_BF16;
  switch (p.n) {
    case 1: return bf ? launch_post_bwd_t<BF16, 1>(p, X, Y, H, G, dX, dY, dH, workspace, stream)
                      : launch_post_bwd_t<F32, 1>(p, X, Y, H, G, dX, dY, dH, workspace, stream);
    case 2: return bf ? launch_post_bwd_t<BF16, 2>(p, X, Y, H, G, dX, dY, dH, workspace, stream)
                      : launch_post_bwd_t<F32, 2>(p, X, Y, H, G, dX, dY, dH, workspace, stream);
    case 4: return bf ? launch_post_bwd_t<BF16, 4>(p, X, Y, H, G, dX, dY, dH, workspace, stream)
                      : launch_post_bwd_t<F32, 4>(p, X, Y, H, G, dX, dY, dH, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

int pre_bwd_max_tmax() { return kBwdMaxTmax; }

size_t pre_bwd_workspace_bytes(int64_t T, int n, int d, int dtype) { return bwd_layout(T, n, d, dtype).total; }

hipError_t launch_pre_bwd(const mhc_params& p, const void* X, const float* phi, const float* bias, const void* D,
                          const float* dH, const void* G, void* dX, float* dphi, float* dbias, float* dalpha,
                          void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  if (p.dtype == MHC_BF16)
    return launch_pre_bwd_n<BF16>(p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, workspace, dev, stream);
  return launch_pre_bwd_n<F32>(p, X, phi, bias, D, dH, G, dX, dphi, dbias, dalpha, workspace, dev, stream);
}

}  // namespace mhc
