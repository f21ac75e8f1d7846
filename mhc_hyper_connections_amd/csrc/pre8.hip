// mhc_pre for n = 8 streams: m = n^2 + 2n = 80 maps per token and a 64-entry
// Sinkhorn-Knopp.  Same method as pre.hip ("mHC" notes on DeepSeek-V4, eqs.
// dsv4-mhc-rmsnorm, a/b/c-tilde, sinkhorn-init, sinkhorn, gate; Dubrov,
// "DeepSeek mHC: Manifold-Constrained Hyper-Connections", Eq. 3 and section
// "Kernmechanismen" for the unconstrained HC maps), in two passes:
//  1. pre_partial8_kernel -- persistent split-K projection.  At n = 8 a
//     lane cannot hold its rows of phi for all 80 columns and all streams
//     (8 streams x 5 column blocks x hi/lo = 320 registers), so a slice is
//     512 positions of one stream (512 rows of the contraction, 164 KiB of
//     phi operands) and a workgroup's eight waves split it: wave w takes
//     positions 64 w .. 64 w + 63 of the slice and keeps those rows of phi
//     for all 80 columns in registers (80).  A slice of one stream rather
//     than 64 positions of every stream makes each load instruction one
//     token's contiguous 1 KiB of X (the 128-byte pieces of the other form
//     read X at about half the rate).  The eight waves' partials are added
//     in LDS in wave order and written as per-token records (m partials,
//     fp64 sum of squares); slices are numbered stream by stream.
//  2. pre_finish8_kernel -- one token per wave, one Sinkhorn entry per lane:
//     sums the slices in order (fp64), forms r, the logits, the gates and
//     Sinkhorn (column sums over lanes e ^ 8, 16, 32; row sums over e ^ 1,
//     2, 4), writes H and streams h = H_pre . X.
#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

constexpr int P8_N = 8;
constexpr int P8_M = num_maps(P8_N);          // 80
constexpr int P8_CB = P8_M / 16;              // 16-column blocks
constexpr int P8_WAVES = 8;
constexpr int P8_THREADS = P8_WAVES * 64;
constexpr int P8_SLICE = 64 * P8_WAVES;       // positions of one stream per slice
// Token record of one slice: 80 partials, 2 words of padding, the fp64 sum
// of squares at word 82; 84 words keep every record 16-byte aligned.
constexpr int P8_SSO = P8_M + 2;
constexpr int P8_PW = P8_SSO + 2;
constexpr size_t kP8TrashBytes = P8_THREADS * 16;   // write-only slots after the records

// MB: 16-token row blocks per tile (2 for bf16 state: 32 tokens a step).
// DB: two tile buffers in flight (bf16 state); fp32 state keeps one buffer.
// Either way a buffer is reloaded as soon as it has been multiplied.
template <typename ST, int MB, bool DB>
__global__ __launch_bounds__(P8_THREADS) void pre_partial8_kernel(int64_t T, int d, int S, int64_t ntiles,
                                                                  const typename ST::elem* X,
                                                                  const float* __restrict__ phi,
                                                                  float* __restrict__ part) {
  constexpr int N = P8_N, M = P8_M;
  constexpr int R = 16 * MB;                  // tokens per tile
  constexpr bool GRAM = std::is_same<ST, BF16>::value;
  __shared__ f32x4 red[P8_WAVES][R][M / 4];
  __shared__ double red_ss[P8_WAVES][R];
  // bf16: the tile arrives with each load instruction covering one token's
  // 1 KiB of the slice, goes through LDS and is read back in the MFMA A
  // layout; 16 bytes of padding per token keep the 16 tokens of a read on
  // distinct banks.
  constexpr bool STAGE = GRAM;
  static_assert(!STAGE || MB == 2, "the staged layout gives each wave 4 of the tile's 32 tokens");
  constexpr int STS = P8_SLICE * 2 + 16;
  __shared__ __attribute__((aligned(16))) unsigned char stage_l[STAGE ? R * STS : 16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int s = blockIdx.x % S;
  const int64_t ntg = gridDim.x / S;
  float* const trash = part + static_cast<int64_t>(S) * T * P8_PW;
  const int bps = S / N;                      // slices per stream
  const int si = s / bps;                     // the slice's stream
  const int p0 = (s - si * bps) * P8_SLICE;   // its first position
  // K block q of this lane: positions p0 + 64 w + 32 q + 8 g .. +7.
  int jq[2];
  bool jvq[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = p0 + 64 * w + 32 * q + 8 * g;
    jvq[q] = j < d;
    jq[q] = jvq[q] ? j : 0;
  }

  // This lane's rows of phi: rows si*d + jq[q] .. +7 of column 16 b + r16,
  // every column block b.
  PhiOp<ST> bop[2][P8_CB];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
#pragma unroll
    for (int b = 0; b < P8_CB; ++b) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = jvq[q] ? phi[(static_cast<int64_t>(si) * d + jq[q] + e) * M + 16 * b + r16] : 0.0f;
      bop[q][b] = make_phi_op(f, ST{});
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // Unconditional loads from valid addresses: tokens past T read token 0,
  // lanes past d read position 0 (zero phi rows; their squares are masked).
  // Staged load layout: load k of wave w covers token 4 w + k of the tile
  // (2 mb + q), 8 positions at jls.
  const int jls0 = p0 + 8 * lane;
  const int jls = jls0 < d ? jls0 : 0;
  auto load_tile = [&](int64_t tile, Raw8<ST> (&x)[MB][2]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if constexpr (STAGE) {
          const int64_t t = tile * R + 4 * w + 2 * mb + q;
          const int64_t tt = t < T ? t : 0;
          x[mb][q] = load_raw8<ST, true>(X + (tt * N + si) * d + jls);   // non-temporal: 6 us less at T = 16384
        } else {
          const int64_t t = tile * R + mb * 16 + r16;
          const int64_t tt = t < T ? t : 0;
          x[mb][q] = load_raw8<ST>(X + (tt * N + si) * d + jq[q]);
        }
      }
    }
  };

  auto step = [&](int64_t tile, Raw8<ST> (&cur)[MB][2], int64_t next) {
    if constexpr (STAGE) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
          *reinterpret_cast<u32x4*>(stage_l + (4 * w + 2 * mb + q) * STS + lane * 16) = cur[mb][q].v;
      }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
          cur[mb][q].v = *reinterpret_cast<const u32x4*>(stage_l + (mb * 16 + r16) * STS +
                                                         (64 * w + 32 * q + 8 * g) * 2);
      }
    }
    f32x4 acc[MB][P8_CB];
    double sq[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int b = 0; b < P8_CB; ++b) acc[mb][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      Raw8<ST> xm[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        xm[q] = jvq[q] ? cur[mb][q] : zero_raw8<ST>();
#pragma unroll
        for (int b = 0; b < P8_CB; ++b) acc[mb][b] = mfma_block(cur[mb][q], bop[q][b], acc[mb][b]);
      }
      if constexpr (GRAM) {
        // Token t's sum of squares over the wave's 2 x 32 values: entry (t, t)
        // of the Gram matrix (lane 16 (t / 4) + t, element t % 4); fp64 from
        // the registers if the fp32 sum is not finite.
        f32x4 gram = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int q = 0; q < 2; ++q) gram = mfma_block_gram(xm[q], gram);
        const int dv = r16 & 3;
        const float sqf = dv == 0 ? gram[0] : dv == 1 ? gram[1] : dv == 2 ? gram[2] : gram[3];
        double v = static_cast<double>(sqf);
        const bool ovf = g == (r16 >> 2) && !__builtin_isfinite(sqf);
        if (__any(ovf)) {            // wave-uniform: every lane takes part in the permutes
          double s64 = 0.0;
          for (int qq = 0; qq < 4; ++qq) {
            const int src = 16 * qq + r16;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              Raw8<ST> xq;
#pragma unroll
              for (int c = 0; c < 4; ++c)
                xq.v[c] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * src, static_cast<int>(xm[q].v[c])));
              float x[8];
              unpack8(xq, x);
#pragma unroll
              for (int e = 0; e < 8; ++e) s64 = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), s64);
            }
          }
          if (ovf) v = s64;
        }
        sq[mb] = v;
      } else {
        double v = 0.0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float x[8];
          unpack8(xm[q], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) v = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), v);
        }
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        sq[mb] = v;
      }
    }
    // The buffer is free once multiplied: the next tile's loads go out now.
    load_tile(next, cur);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int b = 0; b < P8_CB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[w][mb * 16 + 4 * g + v][(16 * b + r16) >> 2][r16 & 3] = acc[mb][b][v];
      if (GRAM ? (g == (r16 >> 2)) : (g == 0)) red_ss[w][mb * 16 + r16] = sq[mb];
    }
    __syncthreads();
    // Records out, 16 bytes a store: the eight waves' partials added in wave
    // order, a fixed number of stores per thread (items past the tile or past
    // T go to the write-only slots).
    constexpr int NF = R * (M / 4);
    constexpr int FPT = (NF + P8_THREADS - 1) / P8_THREADS;
#pragma unroll
    for (int k = 0; k < FPT; ++k) {
      const int q = threadIdx.x + k * P8_THREADS;
      const int qq = q < NF ? q : 0;
      const int tok = qq / (M / 4);
      const int c4 = qq - tok * (M / 4);
      f32x4 sum = red[0][tok][c4];
#pragma unroll
      for (int ww = 1; ww < P8_WAVES; ++ww) {
        const f32x4 y = red[ww][tok][c4];
        sum[0] += y[0];
        sum[1] += y[1];
        sum[2] += y[2];
        sum[3] += y[3];
      }
      const int64_t t = tile * R + tok;
      float* dst = (q < NF && t < T) ? part + (static_cast<int64_t>(s) * T + t) * P8_PW + 4 * c4
                                     : trash + 4 * threadIdx.x;
      *reinterpret_cast<f32x4*>(dst) = sum;
    }
    {
      const int tok = static_cast<int>(threadIdx.x) < R ? static_cast<int>(threadIdx.x) : 0;
      double sum = red_ss[0][tok];
#pragma unroll
      for (int ww = 1; ww < P8_WAVES; ++ww) sum += red_ss[ww][tok];
      const int64_t t = tile * R + tok;
      double* dst = (static_cast<int>(threadIdx.x) < R && t < T)
                        ? reinterpret_cast<double*>(part + (static_cast<int64_t>(s) * T + t) * P8_PW + P8_SSO)
                        : reinterpret_cast<double*>(trash) + threadIdx.x;
      *dst = sum;
    }
    __syncthreads();
  };

  // Every workgroup walks the same, even number of tiles; prefetches past
  // the end read token 0 and write nothing (see pre.hip).
  const int64_t tile0 = blockIdx.x / S;
  const int64_t per_wg = (ntiles + ntg - 1) / ntg;
  Raw8<ST> xa[MB][2];
  load_tile(tile0, xa);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (DB) {
    Raw8<ST> xb[MB][2];
    load_tile(tile0 + ntg, xb);
    __builtin_amdgcn_sched_barrier(0);
    int64_t k = 0;
    do {
      step(tile0 + k * ntg, xa, tile0 + (k + 2) * ntg);
      step(tile0 + (k + 1) * ntg, xb, tile0 + (k + 3) * ntg);
      k += 2;
    } while (k < per_wg);
  } else {
    int64_t k = 0;
    do {
      step(tile0 + k * ntg, xa, tile0 + (k + 1) * ntg);
      k += 1;
    } while (k < per_wg);
  }
}

// Sinkhorn-Knopp on one token's 8 x 8 map held by a whole wave: lane e owns
// entry (e / 8, e % 8).  Column sums add lanes e ^ 8, 16, 32, row sums
// e ^ 1, 2, 4 (a butterfly: every lane of a line holds the same bits).  The
// token's largest logit is subtracted first (unchanged iterates, finite exp).
__device__ __forceinline__ float sinkhorn64(float lr, int t_max) {
  float mx = lr;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (t_max == 0) mx = 0.0f;
  float mv = expf(lr - mx);
  for (int it = 0; it < t_max; ++it) {
    float cs = mv;
    cs += __shfl_xor(cs, 8);
    cs += __shfl_xor(cs, 16);
    cs += __shfl_xor(cs, 32);
    mv = mv / cs;
    float rs = mv;
    rs += __shfl_xor(rs, 1);
    rs += __shfl_xor(rs, 2);
    rs += __shfl_xor(rs, 4);
    mv = mv / rs;
  }
  return mv;
}

// One token per wave.  Lane e: residual entry e (column 8 + e); lanes e < 16
// also the gate of column e (pre) or 72 + e - 8 (post).
template <typename ST, bool HC>
__global__ __launch_bounds__(256) void pre_finish8_kernel(int64_t T, int d, int S, const typename ST::elem* __restrict__ X,
                                                          const float* __restrict__ part,
                                                          const float* __restrict__ bias, float a_pre, float a_res,
                                                          float a_post, float eps, int t_max,
                                                          typename ST::elem* __restrict__ h, float* __restrict__ H) {
  constexpr int N = P8_N, M = P8_M, NN = N * N;
  constexpr int PW = P8_PW;
  constexpr int SSO = P8_SSO;
  const int e = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;                                        // wave-uniform
  const int colr = N + e;
  const bool eg = e < 2 * N;
  const int colg = (e < N) ? e : (eg ? N + NN + (e - N) : 0);

  // Sums over the slices in order, 8 slices' loads at a time.
  double ss = 0.0, zr = 0.0, zg = 0.0;
  for (int s0 = 0; s0 < S; s0 += 8) {
    double pss[8];
    float pzr[8], pzg[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = s0 + k < S ? s0 + k : 0;
      const float* P = part + (static_cast<int64_t>(s) * T + t) * PW;
      pss[k] = *reinterpret_cast<const double*>(P + SSO);
      pzr[k] = P[colr];
      pzg[k] = P[colg];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (s0 + k < S) {
        ss += pss[k];
        zr += static_cast<double>(pzr[k]);
        zg += static_cast<double>(pzg[k]);
      }
    }
  }
  const double inv_r = inv_rms(ss, N * d, eps);
  float gv = 0.0f, mv;
  if constexpr (HC) {
    if (eg)
      gv = static_cast<float>(static_cast<double>(bias[colg]) +
                              static_cast<double>((e < N) ? a_pre : a_post) * tanh(zg * inv_r));
    mv = static_cast<float>(static_cast<double>(bias[colr]) + static_cast<double>(a_res) * tanh(zr * inv_r));
  } else {
    if (eg) {
      const float l = logit_of(zg, inv_r, (e < N) ? a_pre : a_post, bias[colg]);
      gv = (e < N) ? sigmoidf_(l) : 2.0f * sigmoidf_(l);
    }
    mv = sinkhorn64(logit_of(zr, inv_r, a_res, bias[colr]), t_max);
  }
  float* Ht = H + t * M;
  Ht[colr] = mv;
  if (eg) Ht[colg] = gv;
  float hp[N];
#pragma unroll
  for (int i = 0; i < N; ++i) hp[i] = __shfl(gv, i);

  // h = H_pre . X over passes of 64 lanes x 8 positions.
  const typename ST::elem* Xt = X + t * N * static_cast<int64_t>(d);
  typename ST::elem* ht = h + t * static_cast<int64_t>(d);
  for (int j = e * 8; j < d; j += 512) {
    Raw8<ST> x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = load_raw8<ST, true>(Xt + static_cast<int64_t>(i) * d + j);
    float o[8];
    {
      float v[8];
      unpack8(x[0], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = hp[0] * v[k];
    }
#pragma unroll
    for (int i = 1; i < N; ++i) {
      float v[8];
      unpack8(x[i], v);
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = fmaf(hp[i], v[k], o[k]);
    }
    store8<ST, true>(ht + j, o);
  }
}

int slices8(int d) { return P8_N * ((d + P8_SLICE - 1) / P8_SLICE); }

template <typename ST>
hipError_t launch_pre8_t(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                         void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  typedef typename ST::elem E;
  constexpr bool DB = sizeof(E) == 2;
  constexpr int MB = DB ? 2 : 1;
  const int S = slices8(p.d);
  const int64_t ntiles = (p.T + 16 * MB - 1) / (16 * MB);
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &occ, reinterpret_cast<const void*>(pre_partial8_kernel<ST, MB, DB>), P8_THREADS, 0) != hipSuccess ||
      occ < 1)
    occ = 1;
  int64_t groups = static_cast<int64_t>(dev.num_cus) * occ / S;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  float* part = static_cast<float*>(workspace);
  hipLaunchKernelGGL((pre_partial8_kernel<ST, MB, DB>), dim3(static_cast<unsigned>(groups * S)), dim3(P8_THREADS), 0,
                     stream, p.T, p.d, S, ntiles, static_cast<const E*>(X), phi, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 grid(static_cast<unsigned>((p.T + 3) / 4));
  if (p.maps == MHC_MAPS_HC)
    hipLaunchKernelGGL((pre_finish8_kernel<ST, true>), grid, dim3(256), 0, stream, p.T, p.d, S,
                       static_cast<const E*>(X), part, bias, p.alpha_pre, p.alpha_res, p.alpha_post, p.eps, p.t_max,
                       static_cast<E*>(h), H);
  else
    hipLaunchKernelGGL((pre_finish8_kernel<ST, false>), grid, dim3(256), 0, stream, p.T, p.d, S,
                       static_cast<const E*>(X), part, bias, p.alpha_pre, p.alpha_res, p.alpha_post, p.eps, p.t_max,
                       static_cast<E*>(h), H);
  return hipGetLastError();
}

}  // namespace

size_t pre8_workspace_bytes(int64_t T, int d) {
  return static_cast<size_t>(slices8(d)) * static_cast<size_t>(T) * static_cast<size_t>(P8_PW) * sizeof(float) +
         kP8TrashBytes;
}

hipError_t launch_pre8(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                       void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  if (p.dtype == MHC_BF16) return launch_pre8_t<BF16>(p, X, phi, bias, h, H, workspace, dev, stream);
  return launch_pre8_t<F32>(p, X, phi, bias, h, H, workspace, dev, stream);
}

}  // namespace mhc
