// mhc_pre on gfx950: RMSNorm + projection + gates + Sinkhorn-Knopp + aggregation.
//
// Method ("mHC" notes on DeepSeek-V4, eqs. dsv4-mhc-rmsnorm, dsv4-mhc-a-tilde /
// b-tilde / c-tilde, dsv4-mhc-sinkhorn-init, dsv4-mhc-sinkhorn, dsv4-mhc-gate;
// Dubrov, "DeepSeek mHC: Manifold-Constrained Hyper-Connections", sections
// "Sinkhorn-Knopp-projectie" and "Kernmechanismen", Eq. 3), per token t:
//   r = sqrt(sum_k x_k^2 / (n d) + eps)            x = vec(X_t), stream i at [i d, (i+1) d)
//   z = (x . phi) / r                               RMS division after the projection
//   l = alpha_blk z + bias
//   H_pre = sigmoid(l_pre), H_post = 2 sigmoid(l_post)
//   H_res = t_max x (normalise columns, then rows) of exp(Mat(l_res))
//   h = sum_i H_pre[i] X_t[i, :]
//
// Two launches:
//  1. pre_partial_kernel -- persistent split-K projection on MFMA.  The
//     hidden dimension is cut into slices of 256 positions (all n streams of
//     them: K-slice of 256 n rows of phi).  A workgroup owns one slice for its
//     whole life and keeps that slice of phi in registers as MFMA B operands
//     (bf16 state: phi = hi + lo, two bf16 halves, ~16 significant bits, above
//     the TF32 the pages name in table tbl-dsv4-mhc-mixed-precision; fp32
//     state: fp32 MFMA).  It then walks token tiles of 16*MB tokens, streaming
//     the X tile from HBM into registers (16-byte loads; the next tile is
//     prefetched while the current one is multiplied), and writes, per token,
//     the slice's 24 partial dot products and partial sum of squares.  No
//     atomics: every partial has its own slot.
//  2. pre_finish_kernel -- per token, sums the slices' partials in a fixed
//     order (sum of squares in fp64 throughout), forms the logits, gates and Sinkhorn (16 lanes per token, one
//     matrix entry per lane, column and row sums by lane shuffles), writes H
//     and forms h = H_pre . X from a second read of X.
#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

constexpr int PRE_WAVES = 8;                // waves per workgroup of the persistent form
constexpr int PRE_THREADS = PRE_WAVES * 64;
constexpr int SMALL_WAVES = 2;              // waves per workgroup of the small-T form
// Slices of d: 32 positions per wave (all n streams of them).
__host__ __device__ constexpr int slice_width(int waves) { return 32 * waves; }

// Write-only slots after the partial records that absorb the stores of
// items past the end (16 bytes per thread).
constexpr size_t kPartTrashBytes = PRE_THREADS * 16;

// MODE 0: the forward's projection partials of X.
// MODE 1: the backward's: also <D, X_i> per stream (Dg = D).
// MODE 2: the previous layer's mhc_post fused in front: X is X_l, Dg is
//         Y_l, Hin its maps; the tile's X_{l+1} = H_res X_l + H_post Y_l is
//         formed with mhc_post's arithmetic, stored to Xout, and its
//         projection partials (for the next layer) computed from the stored
//         values.
//
// PWV waves per workgroup, slices of 32 PWV positions.  ONE: every
// workgroup takes exactly one tile (blockIdx / S), with no prefetch: the
// small-T form, which spreads a few tiles over many workgroups; otherwise
// the workgroups are persistent and walk tiles with two in flight.
template <typename ST, int N, int MB, int MODE, int PWV = PRE_WAVES, bool ONE = false>
__global__ __launch_bounds__(PWV * 64) void pre_partial_kernel(int64_t T, int d, int S, int64_t ntiles,
                                                                  const typename ST::elem* X,
                                                                  const typename ST::elem* __restrict__ Dg,
                                                                  const float* __restrict__ phi,
                                                                  float* __restrict__ part,
                                                                  const float* __restrict__ Hin,
                                                                  typename ST::elem* Xout) {
  constexpr bool WITH_D = MODE == 1;
  constexpr bool FUSE_POST = MODE == 2;
  constexpr int M = num_maps(N);
  constexpr int NB = (M + 15) / 16;
  constexpr int R = 16 * MB;
  constexpr int ND = WITH_D ? N : 0;
  constexpr int NX = N + ((WITH_D || FUSE_POST) ? 1 : 0);   // chunks per token row: streams, then D or Y
  constexpr int HV = FUSE_POST ? M / 4 : 1;                 // the maps row of the previous layer, as f32x4
  constexpr int PW = part_width(N, WITH_D);
  constexpr int SSO = ss_offset(N, WITH_D);
  constexpr int NT = PWV * 64;                              // threads
  // Staged loads (bf16, persistent form): the tile arrives with each load
  // instruction covering 2 token rows x 512 bytes (wave w: tokens 2w, 2w+1 of
  // a 16-token block, lane = 16-byte chunk of the slice), goes through LDS and
  // is read back in the MFMA A layout.  On MI355X that streams ~18% faster
  // than loading the A layout directly (16 rows x 64 bytes per instruction).
  constexpr bool STAGE = std::is_same<ST, BF16>::value && !ONE && PWV == PRE_WAVES;
  constexpr int NSTG = FUSE_POST ? N : NX;                  // chunks staged (the fused post stages X_{l+1})
  constexpr int STS = NSTG * 512 + 16;                      // LDS bytes per token: 16 B of padding keeps the
                                                            // A-layout reads of 16 tokens on distinct banks
  __shared__ float red[PWV][R][M + ND];
  __shared__ double red_ss[PWV][R];
  __shared__ __attribute__((aligned(16))) unsigned char stage_l[STAGE ? R * STS : 16];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int s = blockIdx.x % S;
  const int64_t ntg = gridDim.x / S;
  float* const trash = part + static_cast<int64_t>(S) * T * PW;     // kPartTrashBytes of write-only slots
  const int j0 = s * slice_width(PWV) + 32 * w + 8 * g;
  const bool jv = j0 < d;
  // Load layout of the staged form: token row trow of each 16-token block,
  // 8 positions at jl0.
  const int trow = 2 * w + (lane >> 5);
  const int jl0 = s * slice_width(PWV) + 8 * (lane & 31);
  const bool jvl = jl0 < d;

  // This lane's rows of phi: rows i*d + j0 .. +7 of column 16 nb + r16.
  PhiOp<ST> bop[N][NB];
#pragma unroll
  for (int i = 0; i < N; ++i) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int col = 16 * nb + r16;
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        f[e] = (jv && col < M) ? phi[static_cast<int64_t>(i * d + j0 + e) * M + col] : 0.0f;
      bop[i][nb] = make_phi_op(f, ST{});
    }
  }
  __builtin_amdgcn_sched_barrier(0);     // finish the phi operands before the first tile's loads

  Raw8<ST> xa[MB][NX], xb[MB][NX];             // chunk N: D (backward) or Y (fused post)
  f32x4 ha[MB][HV], hb[MB][HV];                // the previous layer's maps (fused post only)
  // Every lane loads every chunk from a valid address, with no branch and no
  // select on the data (either would make the compiler wait for the load on
  // the spot): tokens past T read token 0 (their rows are never written) and
  // lanes past d read position 0 (their phi rows are zero and their squares
  // are dropped below).  The backward's pass (WITH_D) reads X and D
  // non-temporally: the apply pass reads them again only after the token
  // pass, and at T = 16384, n = 4, d = 4096 that took 12 us off mhc_pre_bwd
  // (in the forward's modes non-temporal loads measured no faster, so they
  // stay cached).
  const int jl = STAGE ? (jvl ? jl0 : 0) : (jv ? j0 : 0);
  auto load_tile = [&](int64_t tile, Raw8<ST> (&x)[MB][NX], f32x4 (&hv)[MB][HV]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t t = tile * R + mb * 16 + (STAGE ? trow : r16);
      const int64_t tt = t < T ? t : 0;
#pragma unroll
      for (int i = 0; i < N; ++i) x[mb][i] = load_raw8<ST, WITH_D>(X + (tt * N + i) * d + jl);
      if constexpr (WITH_D || FUSE_POST) x[mb][N] = load_raw8<ST, WITH_D>(Dg + tt * d + jl);
      if constexpr (FUSE_POST) {
#pragma unroll
        for (int v = 0; v < HV; ++v) hv[mb][v] = *reinterpret_cast<const f32x4*>(Hin + tt * M + 4 * v);
      }
    }
  };

  // One tile: partials of `cur` while the other buffer streams in; once
  // `cur` is consumed it is refilled with the tile after next.  Two buffers,
  // prefetch distance two, the loop unrolled by two so the buffers keep
  // their registers (copying a buffer that is still being loaded would wait
  // for it and serialise the prefetch).
  auto step = [&](int64_t tile, Raw8<ST> (&cur)[MB][NX], f32x4 (&hv)[MB][HV]) {
    if constexpr (FUSE_POST) {
      // X_{l+1} = H_res X_l + H_post Y_l, term order as in mhc_post; the
      // stored (rounded) values replace X_l for the projection below.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        float mix[N * N + N];
#pragma unroll
        for (int q = 0; q < N * N + N; ++q) mix[q] = hv[mb][(N + q) >> 2][(N + q) & 3];
        float x[N][8], y[8];
#pragma unroll
        for (int i = 0; i < N; ++i) unpack8(cur[mb][i], x[i]);
        unpack8(cur[mb][N], y);
        const int64_t t = tile * R + mb * 16 + (STAGE ? trow : r16);
        const bool pv = STAGE ? jvl : jv;
        const int pj = STAGE ? jl0 : j0;
        Raw8<ST> nx[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float o[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float a = mix[i * N] * x[0][e];
#pragma unroll
            for (int j = 1; j < N; ++j) a = fmaf(mix[i * N + j], x[j][e], a);
            o[e] = fmaf(mix[N * N + i], y[e], a);
          }
          nx[i] = pack8(o, ST{});
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
          typename ST::elem* dst = (t < T && pv) ? Xout + (t * N + i) * d + pj
                                                 : reinterpret_cast<typename ST::elem*>(trash) + threadIdx.x * 8;
          store_raw8<true>(dst, nx[i]);
          cur[mb][i] = nx[i];
        }
      }
    }

    if constexpr (STAGE) {
      // Through LDS into the A layout: lane (r16, g) takes 8 positions of
      // token r16 from each staged chunk.
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int c = 0; c < NSTG; ++c)
          *reinterpret_cast<u32x4*>(stage_l + (mb * 16 + trow) * STS + c * 512 + (lane & 31) * 16) = cur[mb][c].v;
      }
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int c = 0; c < NSTG; ++c)
          cur[mb][c].v = *reinterpret_cast<const u32x4*>(stage_l + (mb * 16 + r16) * STS + c * 512 + (32 * w + 8 * g) * 2);
      }
    }

    // Sum of squares.  bf16 state: the diagonal of the tile's 16 x 16 Gram
    // matrix on MFMA (bf16 products are exact in fp32; fp32 accumulation
    // over the wave's 32 positions x n streams), redone in fp64 for a token
    // whose fp32 sum overflows; entry (t, t) sits in lane 16 (t / 4) + t,
    // element t % 4, and covers the wave's 4 lane groups.  fp32 state: fp64
    // per lane, added over the 4 groups below.  Either never overflows for
    // a finite state.  <D, X_i> (with D): bf16, the diagonal of X_i D^T on
    // MFMA (fp32 accumulation); fp32, per lane.
    constexpr bool GRAM = std::is_same<ST, BF16>::value;
    double ss[MB];
    float dd[MB][ND > 0 ? ND : 1];
    f32x4 acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      double sq = 0.0;
      if constexpr (GRAM) {
        f32x4 gram = {0.0f, 0.0f, 0.0f, 0.0f};
        Raw8<ST> xm[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
          xm[i] = jv ? cur[mb][i] : zero_raw8<ST>();   // lanes past d hold position 0's values
          gram = mfma_block_gram(xm[i], gram);
        }
        const int dv = r16 & 3;
        const float sqf = dv == 0 ? gram[0] : dv == 1 ? gram[1] : dv == 2 ? gram[2] : gram[3];
        sq = static_cast<double>(sqf);
        const bool ovf = g == (r16 >> 2) && !__builtin_isfinite(sqf);
        if (__any(ovf)) {            // wave-uniform: every lane takes part in the permutes
          double s64 = 0.0;
          for (int q = 0; q < 4; ++q) {
            const int src = 16 * q + r16;
#pragma unroll
            for (int i = 0; i < N; ++i) {
              Raw8<ST> xq;
#pragma unroll
              for (int c = 0; c < 4; ++c)
                xq.v[c] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * src, static_cast<int>(xm[i].v[c])));
              float x[8];
              unpack8(xq, x);
#pragma unroll
              for (int e = 0; e < 8; ++e) s64 = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), s64);
            }
          }
          if (ovf) sq = s64;
        }
        ss[mb] = (g == (r16 >> 2)) ? sq : 0.0;
        if constexpr (WITH_D) {
          // <D, X_i> over the wave's 32 positions: the diagonal of the 16 x 16
          // product X_i D^T on MFMA (D's A-layout registers are the B operand
          // of D^T), entry (t, t) in lane 16 (t / 4) + t, element t % 4, like
          // the sum of squares; lanes past d hold zeros in xm.
          const bf16x8 dvb = __builtin_bit_cast(bf16x8, cur[mb][N].v);
#pragma unroll
          for (int i = 0; i < N; ++i) {
            const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xm[i].v), dvb,
                                                                     f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const int dvi = r16 & 3;
            const float dg = dvi == 0 ? c[0] : dvi == 1 ? c[1] : dvi == 2 ? c[2] : c[3];
            dd[mb][i] = (g == (r16 >> 2)) ? dg : 0.0f;
          }
        }
      } else {
        float dv[8];
        if (WITH_D) unpack8(cur[mb][N], dv);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float x[8];
          unpack8(cur[mb][i], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) sq = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), sq);
          if (WITH_D) {
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(dv[e], x[e], a);
            dd[mb][i] = jv ? a : 0.0f;
          }
        }
        ss[mb] = jv ? sq : 0.0;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < N; ++i) a = mfma_block(cur[mb][i], bop[i][nb], a);
        acc[mb][nb] = a;
      }
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 16 * nb + r16;
        if (col < M) {
#pragma unroll
          for (int v = 0; v < 4; ++v) red[w][mb * 16 + 4 * g + v][col] = acc[mb][nb][v];
        }
      }
      if constexpr (GRAM) {
        if (g == (r16 >> 2)) red_ss[w][mb * 16 + r16] = ss[mb];
      } else {
        double sq = ss[mb];
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        if (g == 0) red_ss[w][mb * 16 + r16] = sq;
      }
      if (WITH_D) {
#pragma unroll
        for (int i = 0; i < ND; ++i) {
          if constexpr (GRAM) {
            if (g == (r16 >> 2)) red[w][mb * 16 + r16][M + i] = dd[mb][i];
          } else {
            float a = dd[mb][i];
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            if (g == 0) red[w][mb * 16 + r16][M + i] = a;
          }
        }
      }
    }
    __syncthreads();
    // Partial records out: a fixed number of stores per thread and no branch
    // (stores share the load counter; an unknown count would make the next
    // tile's wait drain the prefetch).  Items past the tile or past T go to
    // the trash slots after the records.
    constexpr int NF = R * (M + ND);
    constexpr int FPT = (NF + NT - 1) / NT;
#pragma unroll
    for (int k = 0; k < FPT; ++k) {
      const int q = threadIdx.x + k * NT;
      const int qq = q < NF ? q : 0;
      const int tok = qq / (M + ND);
      const int col = qq - tok * (M + ND);
      float sum = 0.0f;
#pragma unroll
      for (int ww = 0; ww < PWV; ++ww) sum += red[ww][tok][col];
      const int64_t t = tile * R + tok;
      float* dst = (q < NF && t < T) ? part + (static_cast<int64_t>(s) * T + t) * PW + col : trash + threadIdx.x;
      *dst = sum;
    }
    {
      const int tok = static_cast<int>(threadIdx.x) < R ? static_cast<int>(threadIdx.x) : 0;
      double sum = 0.0;
#pragma unroll
      for (int ww = 0; ww < PWV; ++ww) sum += red_ss[ww][tok];
      const int64_t t = tile * R + tok;
      double* dst = (static_cast<int>(threadIdx.x) < R && t < T)
                        ? reinterpret_cast<double*>(part + (static_cast<int64_t>(s) * T + t) * PW + SSO)
                        : reinterpret_cast<double*>(trash) + threadIdx.x;
      *dst = sum;
    }
    if constexpr (!ONE) {
      __syncthreads();
      load_tile(tile + 2 * ntg, cur, hv);
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch here: the scheduler would sink it to its use
    }
  };

  if constexpr (ONE) {
    const int64_t tile = blockIdx.x / S;
    load_tile(tile, xa, ha);
    step(tile, xa, ha);
    return;
  }

  // Every workgroup walks the same number of tiles, an even number, and
  // every prefetch is issued unconditionally (tiles past the end read token
  // 0, which stays in cache, and write nothing).  With no branch around a
  // load, the compiler counts the loads in flight exactly and waits only for
  // the buffer it is about to use; a conditional prefetch made it wait for
  // both buffers, which halved the loads in flight.
  const int64_t tile0 = blockIdx.x / S;
  const int64_t per_wg = (ntiles + ntg - 1) / ntg;
  load_tile(tile0, xa, ha);
  __builtin_amdgcn_sched_barrier(0);     // all of the first buffer's loads before the second's
  load_tile(tile0 + ntg, xb, hb);
  __builtin_amdgcn_sched_barrier(0);
  // do-while: at least one pair runs (T >= 1), and without the zero-trip
  // guard the compiler cannot sink the prologue's loads below a branch.
  int64_t k = 0;
  do {
    step(tile0 + k * ntg, xa, ha);
    step(tile0 + (k + 1) * ntg, xb, hb);
    k += 2;
  } while (k < per_wg);
}

// One token per wave.  The token's X streams in passes of 64 lanes x 8
// positions, two passes in flight; the first two are issued before the
// partials are summed (they do not depend on the maps).  All four 16-lane
// groups compute the same maps (Sinkhorn is a few hundred instructions);
// group 0 writes H.  Lanes past d work on the last chunk again and store
// the same values to the same place, so no load or store sits behind a
// branch and the compiler keeps both passes in flight.
// SPG: slices per 16-lane group held in registers (the group sums slices
// q, q+4, ...; S <= 4 SPG take no further loop).  With few tokens the
// token's passes are split over `ppp`-pass parts (grid y): every part's wave
// forms the same maps, part 0 writes H.
template <typename ST, int N, bool HC, int SPG>
__global__ __launch_bounds__(256) void pre_finish_kernel(int64_t T, int d, int S, int ppp,
                                                         const typename ST::elem* __restrict__ X,
                                                         const float* __restrict__ part,
                                                         const float* __restrict__ bias, float a_pre,
                                                         float a_res, float a_post, float eps, int t_max,
                                                         typename ST::elem* __restrict__ h,
                                                         float* __restrict__ H) {
  constexpr int M = num_maps(N);
  constexpr int NN = N * N;
  constexpr int PW = part_width(N);
  constexpr int SSO = ss_offset(N);
  const int lane = threadIdx.x & 63;
  const int e = lane & 15;          // Sinkhorn entry (i, j) = (e / N, e % N) when e < N*N
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;               // wave-uniform
  const int colr = N + e;                                  // residual column of entry e
  const int colg = (e < N) ? e : (N + NN + (e - N));       // gate column: pre for e < n, post for n <= e < 2n

  const typename ST::elem* Xt = X + t * N * static_cast<int64_t>(d);
  typename ST::elem* ht = h + t * static_cast<int64_t>(d);
  const int p_first = static_cast<int>(blockIdx.y) * ppp;      // this part's passes: p_first .. + npass - 1
  const int npass_all = (d + 511) / 512;
  const int npass = (npass_all - p_first < ppp) ? npass_all - p_first : ppp;
  auto pos = [&](int p) {
    const int j = (p_first + p) * 512 + lane * 8;
    return j < d ? j : d - 8;
  };
  Raw8<ST> xa[N], xb[N];
  auto load_pass = [&](int p, Raw8<ST> (&x)[N]) {
    const int j = pos(p < npass ? p : npass - 1);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = load_raw8<ST, true>(Xt + static_cast<int64_t>(i) * d + j);
  };

  // The slices' partials, summed in a fixed order (16-lane group q takes
  // slices q, q+4, ..., then the four groups are added); RMS and logits in
  // fp64 (a handful of values per token), everything after in fp32.  The
  // first slices' loads are issued before the X prefetch (load completions
  // are counted in order, so waiting for them must not wait for X).
  const int q = lane >> 4;
  const bool er = e < NN, eg = e < 2 * N;
  const int cr = er ? colr : 0, cg = eg ? colg : 0;
  double pss[SPG];
  float pzr[SPG], pzg[SPG];
#pragma unroll
  for (int k = 0; k < SPG; ++k) {
    const int s = q + 4 * k;
    const float* P = part + (static_cast<int64_t>(s < S ? s : 0) * T + t) * PW;
    pss[k] = *reinterpret_cast<const double*>(P + SSO);
    pzr[k] = P[cr];
    pzg[k] = P[cg];
  }
  const float bias_r = bias[cr], bias_g = bias[cg];
  load_pass(0, xa);
  load_pass(1, xb);
  __builtin_amdgcn_sched_barrier(0);
  double ss = 0.0, zr = 0.0, zg = 0.0;
#pragma unroll
  for (int k = 0; k < SPG; ++k) {
    const bool sv = q + 4 * k < S;
    ss += sv ? pss[k] : 0.0;
    zr += sv ? static_cast<double>(pzr[k]) : 0.0;
    zg += sv ? static_cast<double>(pzg[k]) : 0.0;
  }
  for (int s = q + 4 * SPG; s < S; s += 4) {     // more slices than the registers hold (large d)
    const float* P = part + (static_cast<int64_t>(s) * T + t) * PW;
    ss += *reinterpret_cast<const double*>(P + SSO);
    zr += P[cr];
    zg += P[cg];
  }
  ss += __shfl_xor(ss, 16);
  zr += __shfl_xor(zr, 16);
  zg += __shfl_xor(zg, 16);
  ss += __shfl_xor(ss, 32);
  zr += __shfl_xor(zr, 32);
  zg += __shfl_xor(zg, 32);
  if (!er) zr = 0.0;
  if (!eg) zg = 0.0;
  const double inv_r = inv_rms(ss, N * d, eps);

  float gv = 0.0f;
  float mv = 0.0f;
  if constexpr (HC) {
    // The unconstrained HC form: bias + alpha_blk * tanh(z), in fp64 per value.
    if (e < 2 * N) gv = static_cast<float>(static_cast<double>(bias_g) +
                                           static_cast<double>((e < N) ? a_pre : a_post) * tanh(zg * inv_r));
    if (e < NN) mv = static_cast<float>(static_cast<double>(bias_r) + static_cast<double>(a_res) * tanh(zr * inv_r));
  } else {
    if (e < 2 * N) {
      const float l = logit_of(zg, inv_r, (e < N) ? a_pre : a_post, bias_g);
      gv = (e < N) ? sigmoidf_(l) : 2.0f * sigmoidf_(l);
    }
    float lr = -INFINITY;
    if (e < NN) lr = logit_of(zr, inv_r, a_res, bias_r);
    mv = sinkhorn16<N>(lr, e, t_max);
  }
  if (lane < 16 && blockIdx.y == 0) {
    float* Ht = H + t * M;
    if (e < NN) Ht[colr] = mv;
    if (e < 2 * N) Ht[colg] = gv;
  }
  float hp[N];
#pragma unroll
  for (int i = 0; i < N; ++i) hp[i] = __shfl(gv, i);

  auto emit = [&](int p, Raw8<ST> (&x)[N]) {
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
    store8<ST, true>(ht + pos(p < npass ? p : npass - 1), o);
  };
  // Prefetch two passes ahead while passes remain; the last one or two
  // passes are emitted after the loop (a prefetch past the end would read
  // the state again, and these loads bypass the caches).
  int p = 0;
  for (; p + 2 < npass; p += 2) {
    emit(p, xa);
    load_pass(p + 2, xa);
    __builtin_amdgcn_sched_barrier(0);
    emit(p + 1, xb);
    load_pass(p + 3, xb);
    __builtin_amdgcn_sched_barrier(0);
  }
  emit(p, xa);
  if (p + 1 < npass) emit(p + 1, xb);
}

int num_slices(int d, int waves = PRE_WAVES) { return (d + slice_width(waves) - 1) / slice_width(waves); }

// The forward's small-T form: when the persistent form would launch fewer
// than 128 workgroups (32-token tiles x slices of 256), slices of 64
// positions and one 16-token tile per workgroup.  A function of T and d
// only, so the workspace size is too.
bool small_t_form(int64_t T, int d) { return ((T + 31) / 32) * num_slices(d) < 128; }
int forward_slices(int64_t T, int d) { return small_t_form(T, d) ? num_slices(d, SMALL_WAVES) : num_slices(d); }

// The finishing pass, in the form of the maps p asks for.
template <typename ST, int N, bool HC>
hipError_t launch_finish_t(const mhc_params& p, int S, const void* X, const float* part, const float* bias, void* h,
                           float* H, hipStream_t stream) {
  typedef typename ST::elem E;
  // Parts per token: enough waves for the device (~1024) when T is small.
  const int npass = (p.d + 511) / 512;
  int64_t want = (1024 + p.T - 1) / p.T;
  if (want > npass) want = npass;
  if (want < 1) want = 1;
  const int ppp = static_cast<int>((npass + want - 1) / want);
  const int parts = (npass + ppp - 1) / ppp;                  // every part has at least one pass
  const dim3 grid(static_cast<unsigned>((p.T + 3) / 4), static_cast<unsigned>(parts));
  if (S <= 16)
    hipLaunchKernelGGL((pre_finish_kernel<ST, N, HC, 4>), grid, dim3(256), 0, stream, p.T, p.d, S, ppp,
                       static_cast<const E*>(X), part, bias, p.alpha_pre, p.alpha_res, p.alpha_post, p.eps, p.t_max,
                       static_cast<E*>(h), H);
  else
    hipLaunchKernelGGL((pre_finish_kernel<ST, N, HC, 16>), grid, dim3(256), 0, stream, p.T, p.d, S, ppp,
                       static_cast<const E*>(X), part, bias, p.alpha_pre, p.alpha_res, p.alpha_post, p.eps, p.t_max,
                       static_cast<E*>(h), H);
  return hipGetLastError();
}

// The finishing pass over S slices' records, in the form of the maps p asks for.
template <typename ST, int N>
hipError_t launch_finish(const mhc_params& p, int S, const void* X, const float* part, const float* bias, void* h,
                         float* H, hipStream_t stream) {
  return p.maps == MHC_MAPS_HC ? launch_finish_t<ST, N, true>(p, S, X, part, bias, h, H, stream)
                               : launch_finish_t<ST, N, false>(p, S, X, part, bias, h, H, stream);
}

template <typename ST, int N>
hipError_t launch_pre_t(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                        void* workspace, const DeviceInfo& dev, hipStream_t stream) {
  typedef typename ST::elem E;
  float* part = static_cast<float*>(workspace);
  if (small_t_form(p.T, p.d)) {
    // Few tokens: one 16-token tile per workgroup, slices of 64 positions.
    constexpr int MB = 1;
    const int S = num_slices(p.d, SMALL_WAVES);
    const int64_t ntiles = (p.T + 16 * MB - 1) / (16 * MB);
    hipLaunchKernelGGL((pre_partial_kernel<ST, N, MB, 0, SMALL_WAVES, true>), dim3(static_cast<unsigned>(S * ntiles)),
                       dim3(SMALL_WAVES * 64), 0, stream, p.T, p.d, S, ntiles, static_cast<const E*>(X),
                       static_cast<const E*>(nullptr), phi, part, static_cast<const float*>(nullptr),
                       static_cast<E*>(nullptr));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_finish<ST, N>(p, S, X, part, bias, h, H, stream);
  }
  constexpr int MB = 2;                  // 32-token tiles: two in flight fit the registers
  constexpr int R = 16 * MB;
  const int S = num_slices(p.d);
  const int64_t ntiles = (p.T + R - 1) / R;
  int64_t groups = dev.num_cus / S;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  const int64_t grid = groups * S;
  hipLaunchKernelGGL((pre_partial_kernel<ST, N, MB, 0>), dim3(static_cast<unsigned>(grid)), dim3(PRE_THREADS), 0,
                     stream, p.T, p.d, S, ntiles, static_cast<const E*>(X), static_cast<const E*>(nullptr), phi, part,
                     static_cast<const float*>(nullptr), static_cast<E*>(nullptr));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_finish<ST, N>(p, S, X, part, bias, h, H, stream);
}

// mhc_post of the previous layer fused into the partial pass (MODE 2), then
// the finishing pass on the new state.  16-token tiles: a tile buffer also
// holds Y and the previous layer's maps.
template <typename ST, int N>
hipError_t launch_post_pre_t(const mhc_params& p, const void* X, const void* Y, const float* Hprev, void* Xout,
                             const float* phi, const float* bias, void* h, float* H, void* workspace,
                             const DeviceInfo& dev, hipStream_t stream) {
  typedef typename ST::elem E;
  constexpr int MB = 1;
  constexpr int R = 16 * MB;
  float* part = static_cast<float*>(workspace);
  if (small_t_form(p.T, p.d)) {
    // The small-T form, as mhc_pre takes it: the same slices and records, so
    // the results stay bitwise those of the separate calls.
    const int S = num_slices(p.d, SMALL_WAVES);
    const int64_t ntiles = (p.T + R - 1) / R;
    hipLaunchKernelGGL((pre_partial_kernel<ST, N, MB, 2, SMALL_WAVES, true>), dim3(static_cast<unsigned>(S * ntiles)),
                       dim3(SMALL_WAVES * 64), 0, stream, p.T, p.d, S, ntiles, static_cast<const E*>(X),
                       static_cast<const E*>(Y), phi, part, Hprev, static_cast<E*>(Xout));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_finish<ST, N>(p, S, Xout, part, bias, h, H, stream);
  }
  const int S = num_slices(p.d);
  const int64_t ntiles = (p.T + R - 1) / R;
  int64_t groups = dev.num_cus / S;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  const int64_t grid = groups * S;
  hipLaunchKernelGGL((pre_partial_kernel<ST, N, MB, 2>), dim3(static_cast<unsigned>(grid)), dim3(PRE_THREADS), 0,
                     stream, p.T, p.d, S, ntiles, static_cast<const E*>(X), static_cast<const E*>(Y), phi, part,
                     Hprev, static_cast<E*>(Xout));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_finish<ST, N>(p, S, Xout, part, bias, h, H, stream);
}

template <typename ST>
hipError_t launch_pre_n(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                        void* ws, const DeviceInfo& dev, hipStream_t stream) {
  switch (p.n) {
    case 1: return launch_pre_t<ST, 1>(p, X, phi, bias, h, H, ws, dev, stream);
    case 2: return launch_pre_t<ST, 2>(p, X, phi, bias, h, H, ws, dev, stream);
    case 4: return launch_pre_t<ST, 4>(p, X, phi, bias, h, H, ws, dev, stream);
    case 8: return launch_pre8(p, X, phi, bias, h, H, ws, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename ST, int N>
hipError_t launch_partial_d_t(const mhc_params& p, const void* X, const void* D, const float* phi, float* part,
                              const DeviceInfo& dev, hipStream_t stream) {
  typedef typename ST::elem E;
  // 16-token tiles: twice the tiles of the forward's 32, each with fewer
  // registers live (174 against 226); at T = 16384, n = 4, d = 4096 that
  // took another 11 us off mhc_pre_bwd, with the same bits.
  constexpr int MB = 1;
  constexpr int R = 16 * MB;
  const int S = num_slices(p.d);
  const int64_t ntiles = (p.T + R - 1) / R;
  int64_t groups = dev.num_cus / S;
  if (groups < 1) groups = 1;
  if (groups > ntiles) groups = ntiles;
  const int64_t grid = groups * S;
  hipLaunchKernelGGL((pre_partial_kernel<ST, N, MB, 1>), dim3(static_cast<unsigned>(grid)), dim3(PRE_THREADS), 0,
                     stream, p.T, p.d, S, ntiles, static_cast<const E*>(X), static_cast<const E*>(D), phi, part,
                     static_cast<const float*>(nullptr), static_cast<E*>(nullptr));
  return hipGetLastError();
}

}  // namespace

int pre_num_slices(int d) { return num_slices(d); }
int pre_part_width(int n, bool with_d) { return part_width(n, with_d); }
int pre_part_ss_offset(int n, bool with_d) { return ss_offset(n, with_d); }

hipError_t launch_pre_partial_with_d(const mhc_params& p, const void* X, const void* D, const float* phi, float* part,
                                     const DeviceInfo& dev, hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const bool bf = p.dtype == MHC_BF16;
  switch (p.n) {
    case 1: return bf ? launch_partial_d_t<BF16, 1>(p, X, D, phi, part, dev, stream)
                      : launch_partial_d_t<F32, 1>(p, X, D, phi, part, dev, stream);
    case 2: return bf ? launch_partial_d_t<BF16, 2>(p, X, D, phi, part, dev, stream)
                      : launch_partial_d_t<F32, 2>(p, X, D, phi, part, dev, stream);
    case 4: return bf ? launch_partial_d_t<BF16, 4>(p, X, D, phi, part, dev, stream)
                      : launch_partial_d_t<F32, 4>(p, X, D, phi, part, dev, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t pre_partial_bytes(int64_t T, int n, int d, bool with_d) {
  return static_cast<size_t>(num_slices(d)) * static_cast<size_t>(T) * static_cast<size_t>(part_width(n, with_d)) *
             sizeof(float) + kPartTrashBytes;
}

hipError_t launch_post_pre(const mhc_params& p, const void* X, const void* Y, const float* Hprev, void* Xout,
                           const float* phi, const float* bias, void* h, float* H, void* workspace, size_t ws_bytes,
                           int algo, int* used, const DeviceInfo& dev, hipStream_t stream) {
  if (used) *used = MHC_PRE_TWO_PASS;
  if (p.T == 0) return hipSuccess;
  // The single pass recomputes from X_l when its waits run out, so it needs
  // X_{l+1} in a buffer of its own.  MHC_PRE_AUTO takes it when X_{l+1} is
  // separate and each team gets at least kAutoTilesPostPre[S] tiles (on
  // MI355X at T = 16384, n = 4, d = 4096: 265-272 us against 326-329 us for
  // the two-pass form), else the two-pass form.
  const bool separate = Xout != X;
  if (algo == MHC_PRE_AUTO && separate && pre_fused_preferred(p, dev, true)) {
    if (launch_post_pre_fused(p, X, Y, Hprev, Xout, phi, bias, h, H, workspace, ws_bytes, false, dev, stream) ==
        hipSuccess) {
      if (used) *used = MHC_PRE_ONE_PASS;
      return hipSuccess;
    }
    (void)hipGetLastError();                 // refused: the two-pass form below
  }
  if (algo == MHC_PRE_ONE_PASS || algo == MHC_PRE_ONE_PASS_FALLBACK_TEST) {
    if (!separate) return hipErrorNotSupported;
    const hipError_t e = launch_post_pre_fused(p, X, Y, Hprev, Xout, phi, bias, h, H, workspace, ws_bytes,
                                               algo == MHC_PRE_ONE_PASS_FALLBACK_TEST, dev, stream);
    if (e == hipSuccess) {
      if (used) *used = MHC_PRE_ONE_PASS;
      return hipSuccess;
    }
    (void)hipGetLastError();                 // clear a refused launch
    return e;
  }
  const bool bf = p.dtype == MHC_BF16;
  void* body = static_cast<char*>(workspace) + kPreHeaderBytes;
  switch (p.n) {
    case 2: return bf ? launch_post_pre_t<BF16, 2>(p, X, Y, Hprev, Xout, phi, bias, h, H, body, dev, stream)
                      : launch_post_pre_t<F32, 2>(p, X, Y, Hprev, Xout, phi, bias, h, H, body, dev, stream);
    case 4: return bf ? launch_post_pre_t<BF16, 4>(p, X, Y, Hprev, Xout, phi, bias, h, H, body, dev, stream)
                      : launch_post_pre_t<F32, 4>(p, X, Y, Hprev, Xout, phi, bias, h, H, body, dev, stream);
    default: {   // n = 1 (m = 3 maps per token) and n = 8: the two entry points one after the other
      hipError_t e = launch_post(p, X, Y, Hprev, Xout, stream);
      if (e != hipSuccess) return e;
      int u = 0;
      return launch_pre(p, Xout, phi, bias, h, H, workspace, ws_bytes, MHC_PRE_TWO_PASS, &u, dev, stream);
    }
  }
}

size_t pre_workspace_bytes(int64_t T, int n, int d) {
  // [header][body]: the header is the single pass's alone (its error word,
  // sequence number and the current call's tag); every other form keeps its
  // records in the body, so it never disturbs them.
  size_t body = 0;
  if (n == 8) {
    body = pre8_workspace_bytes(T, d);
  } else {
    body = pre_partial_bytes(T, n, d, false);   // persistent form (also mhc_post_pre's)
    if (small_t_form(T, d)) {
      const size_t small = static_cast<size_t>(num_slices(d, SMALL_WAVES)) * static_cast<size_t>(T) *
                               static_cast<size_t>(part_width(n)) * sizeof(float) + kPartTrashBytes;
      if (small > body) body = small;
    }
    const size_t one_pass = pre_fused_body_bytes(n, d);
    if (one_pass > body) body = one_pass;
  }
  return kPreHeaderBytes + body;
}

hipError_t launch_pre(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h, float* H,
                      void* workspace, size_t ws_bytes, int algo, int* used, const DeviceInfo& dev,
                      hipStream_t stream) {
  if (used) *used = MHC_PRE_TWO_PASS;
  if (p.T == 0) return hipSuccess;
  if (algo == MHC_PRE_AUTO && pre_fused_preferred(p, dev, false)) {
    if (launch_pre_fused(p, X, phi, bias, h, H, workspace, ws_bytes, false, dev, stream) == hipSuccess) {
      if (used) *used = MHC_PRE_ONE_PASS;
      return hipSuccess;
    }
    (void)hipGetLastError();                 // refused: the two-pass form below
  }
  if (algo == MHC_PRE_ONE_PASS || algo == MHC_PRE_ONE_PASS_FALLBACK_TEST) {
    const hipError_t e = launch_pre_fused(p, X, phi, bias, h, H, workspace, ws_bytes,
                                          algo == MHC_PRE_ONE_PASS_FALLBACK_TEST, dev, stream);
    if (e == hipSuccess) {
      if (used) *used = MHC_PRE_ONE_PASS;
      return hipSuccess;
    }
    (void)hipGetLastError();                 // clear a refused launch
    return e;
  }
  void* body = static_cast<char*>(workspace) + kPreHeaderBytes;
  if (p.dtype == MHC_BF16) return launch_pre_n<BF16>(p, X, phi, bias, h, H, body, dev, stream);
  return launch_pre_n<F32>(p, X, phi, bias, h, H, body, dev, stream);
}

}  // namespace mhc
