// mhc_pre in ONE pass over the state (bf16), for 8 <= ceil(d / 256) <= 16.
//
// Same method as pre.hip ("mHC" notes on DeepSeek-V4, eqs. dsv4-mhc-rmsnorm,
// a/b/c-tilde, sinkhorn-init, sinkhorn, gate; Dubrov, "DeepSeek mHC:
// Manifold-Constrained Hyper-Connections", Eq. 3 for h = H_pre . X).
//
// Why one pass is hard: H_pre needs the reduction over all n*d values of a
// token before h = H_pre . X can be formed, and phi (n*d x 24, 1.5 MiB at
// d = 4096) is too large for one CU.  Here teams of S workgroups (one per CU)
// split d: member s keeps its 256-position slice of phi in LDS and, for every
// 32-token tile, streams its slice of X from HBM into registers once.
//   1. MFMA partial dot products + fp64 partial sum of squares of the tile,
//      reduced over the 8 waves in LDS, then posted to the team as tagged
//      64-bit words (value | tile tag << 32, device-scope stores: no fence,
//      no wait on the writer's side).
//   2. One tile later, every member reads the posted pre-columns and sums of
//      squares of all S members (device-scope loads, issued BEFORE the next
//      prefetch so the in-order wait covers only data that is due anyway),
//      forms H_pre of the 32 tokens and h for its slice from the X tile it
//      still holds in registers.  The tile never travels from HBM twice.
//   3. Member s also reads all 24 columns of its ceil(32 / S) tokens and runs
//      the gates + Sinkhorn for them (16 lanes per token), writing H.  No one
//      in the kernel waits for these rows, so Sinkhorn is off the critical path.
// The team's tiles are pipelined: X of tile k+1 streams in while tile k's
// partials are posted and tile k-1's h is formed.  Slots in the exchange
// area form a ring of 4 (a member can be at most about one tile ahead of the
// slowest, see the slot-reuse note in the launcher).  Every sum runs in a
// fixed order: results are bitwise reproducible.  All waits are bounded; a
// wait that runs out records an error word in the workspace header instead
// of hanging.  The launch is cooperative (all workgroups co-resident).
#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

constexpr int FW = 8;                  // waves per workgroup
constexpr int FT = FW * 64;            // threads per workgroup
constexpr int FSLICE = FW * 32;        // positions of d per team member
constexpr int FMB = 2;                 // 16-token blocks per tile
constexpr int FR = 16 * FMB;           // tokens per tile
constexpr int FSLOTS = 4;              // exchange ring depth
constexpr int FS_MIN = 8;              // team size range (ceil(d / FSLICE))
constexpr int FS_MAX = 16;
constexpr int FTPR_MAX = (FR + FS_MIN - 1) / FS_MIN;   // tokens whose maps one member forms
constexpr size_t FHDR = 256;           // workspace header: error word
constexpr unsigned kSpinLimit = 1u << 14;   // ~tens of ms per word; far beyond any legitimate wait

struct FusedArgs {
  int64_t T;
  int d, S, tpx, teams, tpr;
  int64_t ntiles;
  const uint16_t* X;
  const float* phi;
  const float* bias;
  float a_pre, a_res, a_post, eps;
  int t_max;
  uint16_t* h;
  float* H;
  unsigned long long* xch;
  unsigned* err;
};

__device__ __forceinline__ unsigned long long xword(float v, unsigned tag) {
  return (static_cast<unsigned long long>(tag) << 32) | static_cast<unsigned long long>(__float_as_uint(v));
}
__device__ __forceinline__ void xstore(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long xload(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int N>
__global__ __launch_bounds__(FT) void pre_fused_kernel(FusedArgs a) {
  constexpr int M = num_maps(N);
  constexpr int NB = (M + 15) / 16;
  constexpr int NN = N * N;
  constexpr int W = M + 2;             // words per token record: m partials, sum of squares (hi, lo)
  constexpr int WA = N + 2;            // pre columns + sum of squares, read for every token
  constexpr int WB = M - N;            // residual + post columns, read for the member's own tokens
  constexpr int KMAX = (FS_MAX * FR * WA + FS_MAX * FTPR_MAX * WB + FT - 1) / FT;   // words per thread

  __shared__ u32x4 phi_l[FW][N][2][4][M];    // MFMA B operands: [wave][stream][hi/lo][lane group][column]
  __shared__ float red[FW][FR][M];
  __shared__ double red_ss[FW][FR];
  __shared__ float xin[FS_MAX * FR * WA + FS_MAX * FTPR_MAX * WB];   // part a: [member][tok][WA], then part b
  float (*xin_a)[FR][WA] = reinterpret_cast<float (*)[FR][WA]>(xin);
  float (*xin_b)[FTPR_MAX][WB] = reinterpret_cast<float (*)[FTPR_MAX][WB]>(xin + FS_MAX * FR * WA);
  __shared__ float hp[FR][N];

  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int idx = wg >> 3;
  if (idx >= a.tpx * a.S) return;            // not part of a team (cooperative grid of one workgroup per CU)
  const int S = a.S;
  const int team = xcd * a.tpx + idx / S;    // teams live inside one XCD (workgroup w runs on XCD w % 8)
  const int s = idx - (idx / S) * S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int d = a.d;
  const int j0 = s * FSLICE + 32 * wave + 8 * g;
  const bool jv = j0 < d;
  const int64_t T = a.T;
  const int64_t J = (a.ntiles > team) ? (a.ntiles - team + a.teams - 1) / a.teams : 0;

  // This member's slice of phi into LDS as bf16 hi / lo operand halves.
  for (int q = tid; q < FW * N * 4 * M; q += FT) {
    const int col = q % M;
    const int gg = (q / M) & 3;
    const int i = (q / (4 * M)) % N;
    const int ww = q / (4 * M * N);
    const int jj = s * FSLICE + 32 * ww + 8 * gg;
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (jj < d) ? a.phi[static_cast<int64_t>(i * d + jj + e) * M + col] : 0.0f;
    const PhiOp<BF16> op = make_phi_op(f, BF16{});
    phi_l[ww][i][0][gg][col] = __builtin_bit_cast(u32x4, op.hi);
    phi_l[ww][i][1][gg][col] = __builtin_bit_cast(u32x4, op.lo);
  }
  __syncthreads();

  auto tile_of = [&](int64_t jt) -> int64_t { return team + jt * a.teams; };
  // Unconditional loads from always-valid addresses (no branch, no select on
  // the data, either of which would make the compiler wait for the load on
  // the spot): tokens past T read token 0 (never written back), lanes past d
  // read position 0 (zero phi rows; squares dropped; h not stored).
  const int jl = jv ? j0 : 0;
  auto load_tile = [&](int64_t jt, Raw8<BF16> (&x)[FMB][N]) {
    const int64_t t0 = tile_of(jt) * FR;
#pragma unroll
    for (int mb = 0; mb < FMB; ++mb) {
      const int64_t t = t0 + mb * 16 + r16;
      const int64_t tt = t < T ? t : 0;
#pragma unroll
      for (int i = 0; i < N; ++i) x[mb][i] = load_raw8<BF16, true>(a.X + (tt * N + i) * d + jl);
    }
  };
  auto xrec = [&](int64_t jt, int member, int tok) -> unsigned long long* {
    return a.xch + ((static_cast<int64_t>(team) * FSLOTS + (jt % FSLOTS)) * S + member) * (FR * W) + tok * W;
  };

  Raw8<BF16> b0[FMB][N], b1[FMB][N], b2[FMB][N];
  if (J > 0) load_tile(0, b0);
  if (J > 1) load_tile(1, b1);
  const int tpr = a.tpr;
  bool broken = false;                 // a wait ran out: stop waiting (results are invalid, the error word is set)
  // Word q of a tile's reads, laid out for the largest team so that the
  // decomposition uses constants only: part a = [member < FS_MAX][token][WA],
  // part b = [member < FS_MAX][own token < FTPR_MAX][WB].  Returns the word's
  // offset in the tile's slot, or -1 when the word does not exist; lds is
  // its index in xin.
  constexpr int QA = FS_MAX * FR * WA;
  constexpr int QTOT = QA + FS_MAX * FTPR_MAX * WB;
  auto word_of = [&](int q, int& lds) -> int {
    lds = q;
    if (q < QA) {
      const int member = q / (FR * WA);
      const int rem = q - member * (FR * WA);
      const int tok = rem / WA;
      const int c = rem - tok * WA;
      if (member >= S) return -1;
      return member * (FR * W) + tok * W + ((c < N) ? c : M + (c - N));
    }
    const int qb = q - QA;
    const int member = qb / (FTPR_MAX * WB);
    const int rem = qb - member * (FTPR_MAX * WB);
    const int qq = rem / WB;
    const int cb = rem - qq * WB;
    const int tok = s * tpr + qq;
    if (member >= S || qq >= tpr || tok >= FR) return -1;
    return member * (FR * W) + tok * W + N + cb;
  };

  unsigned long long wv[KMAX];           // the team's words of the previous tile, in flight between rounds

  // One round, for tile jt: its partials from `xc` are posted; then tile
  // jt - 1's exchange words (read at the end of the previous round) are
  // checked, its H_pre and h (from `xh`) formed and its maps written; then
  // the reads of tile jt's words are issued and tile jt + 2 starts streaming
  // into `xh`, free by now.  Every wait therefore covers only operations
  // older than the prefetch in flight.  The rounds are unrolled by three so
  // the buffers rotate roles without register copies.
  auto round = [&](int64_t jt, Raw8<BF16> (&xh)[FMB][N], Raw8<BF16> (&xc)[FMB][N]) {
    const int64_t p = jt - 1;
    if (jt < J) {
      // 1. Partials of tile jt over this member's slice.
      double ssq[FMB];
      f32x4 acc[FMB][NB];
#pragma unroll
      for (int mb = 0; mb < FMB; ++mb) {
        double sq = 0.0;
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float x[8];
          unpack8(xc[mb][i], x);
#pragma unroll
          for (int e = 0; e < 8; ++e) sq = fma(static_cast<double>(x[e]), static_cast<double>(x[e]), sq);
        }
        ssq[mb] = jv ? sq : 0.0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int i = 0; i < N; ++i) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = 16 * nb + r16;
          PhiOp<BF16> b;
          const u32x4 zero = {0u, 0u, 0u, 0u};
          b.hi = __builtin_bit_cast(bf16x8, col < M ? phi_l[wave][i][0][g][col] : zero);
          b.lo = __builtin_bit_cast(bf16x8, col < M ? phi_l[wave][i][1][g][col] : zero);
#pragma unroll
          for (int mb = 0; mb < FMB; ++mb) acc[mb][nb] = mfma_block(xc[mb][i], b, acc[mb][nb]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < FMB; ++mb) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int col = 16 * nb + r16;
          if (col < M) {
#pragma unroll
            for (int v = 0; v < 4; ++v) red[wave][mb * 16 + 4 * g + v][col] = acc[mb][nb][v];
          }
        }
        double sq = ssq[mb];
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        if (g == 0) red_ss[wave][mb * 16 + r16] = sq;
      }
      __syncthreads();
      // 2. Post the tile's record: m partial dot products, sum of squares as hi + lo.
      const unsigned tag = static_cast<unsigned>(jt + 1);
      unsigned long long* mine = xrec(jt, s, 0);
      for (int q = tid; q < FR * W; q += FT) {
        const int tok = q / W;
        const int col = q - tok * W;
        float v;
        if (col < M) {
          v = 0.0f;
#pragma unroll
          for (int ww = 0; ww < FW; ++ww) v += red[ww][tok][col];
        } else {
          double sd = 0.0;
#pragma unroll
          for (int ww = 0; ww < FW; ++ww) sd += red_ss[ww][tok];
          const float hi = static_cast<float>(sd);
          v = (col == M) ? hi : static_cast<float>(sd - static_cast<double>(hi));
        }
        xstore(mine + q, xword(v, tag));
      }
      __syncthreads();
    }

    if (jt >= 1) {
      // In the last round no barrier has passed since the previous round's
      // step 6 (wave FW-1 may still read xin): wait for it before overwriting.
      if (jt == J) __syncthreads();
      // 3. Check the tags of tile jt - 1's words (re-reading any not yet posted).
      const unsigned want = static_cast<unsigned>(p + 1);
      const unsigned long long* slot = xrec(p, 0, 0);
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int q = tid + k * FT;
        int lds = 0;
        const int off = (q < QTOT) ? word_of(q, lds) : -1;
        if (off >= 0) {
          unsigned long long v = wv[k];
          unsigned spins = 0;
          while (!broken && static_cast<unsigned>(v >> 32) != want) {
            if (++spins > kSpinLimit) {
              atomicOr(a.err, 1u);
              broken = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
            v = xload(slot + off);
          }
          xin[lds] = __uint_as_float(static_cast<unsigned>(v));
        }
      }
      __syncthreads();
      // 4. H_pre of the tile's tokens (every member, identical arithmetic).
      if (tid < FR * N) {
        const int tok = tid / N;
        const int i = tid - tok * N;
        double z = 0.0, ss = 0.0;
        for (int m2 = 0; m2 < S; ++m2) {
          z += static_cast<double>(xin_a[m2][tok][i]);
          ss += static_cast<double>(xin_a[m2][tok][N]) + static_cast<double>(xin_a[m2][tok][N + 1]);
        }
        const double inv_r = inv_rms(ss, N * d, a.eps);
        hp[tok][i] = sigmoidf_(logit_of(z, inv_r, a.a_pre, a.bias[i]));
      }
      __syncthreads();
      // 5. h = H_pre . X for this member's slice, from the tile still in registers.
      const int64_t t0 = tile_of(p) * FR;
#pragma unroll
      for (int mb = 0; mb < FMB; ++mb) {
        const int tok = mb * 16 + r16;
        const int64_t t = t0 + tok;
        if (jv && t < T) {
          float o[8];
          {
            float x[8];
            unpack8(xh[mb][0], x);
            const float w0 = hp[tok][0];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = w0 * x[e];
          }
#pragma unroll
          for (int i = 1; i < N; ++i) {
            float x[8];
            unpack8(xh[mb][i], x);
            const float wi = hp[tok][i];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(wi, x[e], o[e]);
          }
          store8<BF16, true>(a.h + t * d + j0, o);
        }
      }
      // 6. Gates + Sinkhorn for this member's tokens; nothing here waits for them.
      if (wave == FW - 1) {
        const int qq = lane >> 4;
        const int e = lane & 15;
        const int tok = s * tpr + qq;
        const bool tv = qq < tpr && tok < FR && t0 + tok < T;
        const int tk = tok < FR ? tok : 0;
        const int qc = qq < FTPR_MAX ? qq : 0;
        double ss = 0.0, zr = 0.0, zg = 0.0;
        for (int m2 = 0; m2 < S; ++m2) {
          ss += static_cast<double>(xin_a[m2][tk][N]) + static_cast<double>(xin_a[m2][tk][N + 1]);
          if (e < NN) zr += static_cast<double>(xin_b[m2][qc][e]);
          if (e < N) zg += static_cast<double>(xin_a[m2][tk][e]);
          else if (e < 2 * N) zg += static_cast<double>(xin_b[m2][qc][NN + (e - N)]);
        }
        const double inv_r = inv_rms(ss, N * d, a.eps);
        const int colg = (e < N) ? e : (N + NN + (e - N));
        float gv = 0.0f;
        if (e < 2 * N) {
          const float l = logit_of(zg, inv_r, (e < N) ? a.a_pre : a.a_post, a.bias[colg]);
          gv = (e < N) ? sigmoidf_(l) : 2.0f * sigmoidf_(l);
        }
        float lr = -INFINITY;
        if (e < NN) lr = logit_of(zr, inv_r, a.a_res, a.bias[N + e]);
        const float mv = sinkhorn16<N>(lr, e, a.t_max);
        if (tv) {
          float* Ht = a.H + (t0 + tok) * M;
          if (e < NN) Ht[N + e] = mv;
          if (e < 2 * N) Ht[colg] = gv;
        }
      }
    }
    // 7. Issue the reads of tile jt's words, then stream tile jt + 2 into xh.
    if (jt < J) {
      const unsigned long long* slot = xrec(jt, 0, 0);
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int q = tid + k * FT;
        int lds;
        const int off = (q < QTOT) ? word_of(q, lds) : -1;
        wv[k] = (off >= 0) ? xload(slot + off) : 0ull;
      }
    }
    asm volatile("" ::: "memory");
    if (jt + 2 < J) load_tile(jt + 2, xh);
    __builtin_amdgcn_sched_barrier(0);
  };

  for (int64_t jt = 0; jt <= J; jt += 3) {
    round(jt, b2, b0);
    if (jt + 1 <= J) round(jt + 1, b0, b1);
    if (jt + 2 <= J) round(jt + 2, b1, b2);
  }
}

__global__ __launch_bounds__(256) void clear_words_kernel(unsigned long long* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = 0ull;
}

int fused_slices(int d) { return (d + FSLICE - 1) / FSLICE; }

size_t fused_exchange_words(int teams, int S, int n) {
  return static_cast<size_t>(teams) * FSLOTS * S * FR * (num_maps(n) + 2);
}

template <int N>
const void* fused_kernel_ptr() {
  return reinterpret_cast<const void*>(&pre_fused_kernel<N>);
}

}  // namespace

// Bytes the fused form may need: header + exchange ring, for devices with up
// to 48 CUs per XCD.
size_t pre_fused_workspace_bytes(int64_t /*T*/, int n, int d) {
  const int S = fused_slices(d);
  if (S < FS_MIN || S > FS_MAX) return 0;
  const int teams = 8 * (48 / S);
  return FHDR + fused_exchange_words(teams, S, n) * sizeof(unsigned long long);
}

// Launch the single-pass form when it applies; returns hipErrorNotSupported
// (without launching anything) when it does not, so the caller can fall back.
hipError_t launch_pre_fused(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, size_t ws_bytes, const DeviceInfo& dev, hipStream_t stream) {
  if (p.dtype != MHC_BF16 || (p.n != 4 && p.n != 2 && p.n != 1) || p.maps != MHC_MAPS_MHC)
    return hipErrorNotSupported;
  const int S = fused_slices(p.d);
  if (S < FS_MIN || S > FS_MAX || !dev.cooperative || dev.num_cus % 8 != 0) return hipErrorNotSupported;
  const int per_xcd = dev.num_cus / 8;
  const int tpx = per_xcd / S;
  if (tpx < 1) return hipErrorNotSupported;
  const int teams = 8 * tpx;
  const int64_t ntiles = (p.T + FR - 1) / FR;
  if (ntiles < 2 * static_cast<int64_t>(teams)) return hipErrorNotSupported;   // too little work to fill the teams
  const size_t words = fused_exchange_words(teams, S, p.n);
  if (FHDR + words * sizeof(unsigned long long) > ws_bytes) return hipErrorNotSupported;
  const void* fn = nullptr;
  switch (p.n) {
    case 1: fn = fused_kernel_ptr<1>(); break;
    case 2: fn = fused_kernel_ptr<2>(); break;
    default: fn = fused_kernel_ptr<4>(); break;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, FT, 0) != hipSuccess || occ < 1)
    return hipErrorNotSupported;

  char* base = static_cast<char*>(workspace);
  unsigned long long* xch = reinterpret_cast<unsigned long long*>(base + FHDR);
  // Clear the header and the ring: tags of an earlier call must never match.
  const int64_t nclear = static_cast<int64_t>(words + FHDR / sizeof(unsigned long long));
  hipLaunchKernelGGL(clear_words_kernel, dim3(1024), dim3(256), 0, stream, reinterpret_cast<unsigned long long*>(base),
                     nclear);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  FusedArgs fa;
  fa.T = p.T;
  fa.d = p.d;
  fa.S = S;
  fa.tpx = tpx;
  fa.teams = teams;
  fa.tpr = (FR + S - 1) / S;
  fa.ntiles = ntiles;
  fa.X = static_cast<const uint16_t*>(X);
  fa.phi = phi;
  fa.bias = bias;
  fa.a_pre = p.alpha_pre;
  fa.a_res = p.alpha_res;
  fa.a_post = p.alpha_post;
  fa.eps = p.eps;
  fa.t_max = p.t_max;
  fa.h = static_cast<uint16_t*>(h);
  fa.H = H;
  fa.xch = xch;
  fa.err = reinterpret_cast<unsigned*>(base);
  void* args[] = {&fa};
  return hipLaunchCooperativeKernel(fn, dim3(dev.num_cus), dim3(FT), args, 0, stream);
}

}  // namespace mhc
