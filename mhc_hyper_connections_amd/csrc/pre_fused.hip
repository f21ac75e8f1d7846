// mhc_pre in ONE pass over the state (bf16): X travels from HBM once.
//
// Same method as pre.hip ("mHC" notes on DeepSeek-V4, eqs. dsv4-mhc-rmsnorm,
// a/b/c-tilde, sinkhorn-init, sinkhorn, gate; Dubrov, "DeepSeek mHC:
// Manifold-Constrained Hyper-Connections", Eq. 3 for h = H_pre . X, and the
// section "Kernmechanismen" for the unconstrained HC maps).
//
// Why one pass is hard: H_pre needs the reduction over all n*d values of a
// token before h = H_pre . X can be formed, and phi (n*d x 24, 1.5 MiB at
// d = 4096) is too large for one CU.  So the hidden dimension is split over a
// team of S = ceil(d / 256) workgroups (8 <= S <= 16), one per CU, all on one
// XCD: they exchange per-token sums through that XCD's L2.  Member s owns
// positions [256 s, 256 s + 256) of every stream; the team walks 16-token
// tiles.  Workgroups are dispatched to the XCDs round-robin, not always
// starting at XCD 0 (after a HIP graph has been captured in the process the
// start moved): a workgroup takes its team from its hardware XCD id and its
// place on that XCD from its index / 8.  Were the placement ever not a
// rotation, a team's members would sit on different XCDs, their exchange
// words would not meet in one L2, and the bounded waits would report it.
// A workgroup runs eleven waves with fixed roles:
//  * waves 0-7 stream.  Wave w holds positions 32 w .. 32 w + 31 of the
//    member's slice for a tile's 16 tokens in registers (lane = token row
//    and 8 positions, the MFMA A layout; one 16-byte load per stream).  In
//    step k it forms tile k's m partial dot products with phi on MFMA (phi
//    as bf16 hi + lo halves, kept in LDS) and the partial sums of squares
//    (the diagonal of the tile's 16 x 16 Gram matrix, also on MFMA) into an
//    LDS ring; sums its eighth of tile k-1's record over the
//    8 waves (wave order) and posts it with one 16-byte store; and, once
//    tile k-OD's H_pre has come back, forms h = H_pre . X for its positions
//    from the registers that still hold that tile, and stores it.  These
//    waves issue no memory operation but their X loads, the record store and
//    the h store, a fixed number per step (masked lanes use out-of-range
//    buffer offsets, which move no data), so the in-order completion count
//    only ever makes them wait for their oldest tile.
//  * waves 8-9 exchange, tiles alternating between them.  For tile j, once
//    the member's waves have posted its record:
//      B  reduce-scatter: member s owns tokens s and s + S of the tile.  It
//         reads every member's record of them, sums them by a fixed tree
//         over the members (fp64), forms r, the logits and the gates, posts
//         H_pre and hands the residual logits to wave 10.
//      C  broadcast: reads H_pre of all 16 tokens into LDS for the
//         streaming waves.
//  * wave 10 runs Sinkhorn-Knopp for the member's own tokens (two tiles per
//    pass) and writes H.
// Exchange words are tagged 64-bit values (value | tag << 32) moved in
// 16-byte pairs: written with plain stores (through the CU's L1 into the
// XCD's L2), read with sc1 buffer loads (which skip the L1); a pair whose tag
// is not yet the tile's is read again.  Each member clears its own slots
// before any wave posts, and the team meets on words stamped with the call's
// sequence number, so words of earlier calls never match.  Every sum runs in
// a fixed order: results are bitwise reproducible.  All waits are bounded;
// one that runs out marks the workgroup broken (no further waits; its
// results are garbage, its writes stay in bounds) and the call's sequence
// number is stored into the workspace's error word.
// The launch is an ordinary one of one workgroup per CU, which on an idle
// device makes every team resident together; a cooperative launch would
// guarantee it but costs about 16 us more per call on MI355X.  The guarantee
// is replaced by a fallback: the two-pass form is launched behind the single
// pass, each of its kernels gated on the error word holding this call's
// sequence number, so it recomputes every output when a wait ran out and
// otherwise returns at once (about 3 us for the two launches).
// The exchange and Sinkhorn waves run at a raised issue priority: the
// streaming waves have slack, the exchange is on every tile's critical path.
#include <atomic>
#include <cstdlib>

#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

typedef unsigned long long u64;

constexpr int OW = 8;                   // streaming waves
constexpr int OX = 2;                   // exchange waves (tiles alternate between them)
constexpr int OT = (OW + OX + 1) * 64;  // + the exchange waves + the Sinkhorn wave
constexpr int OSLICE = OW * 32;         // positions of d per member
constexpr int OR = 16;                  // tokens per tile
constexpr int OS_MIN = 8;               // team size range (ceil(d / OSLICE))
constexpr int OS_MAX = 16;
constexpr int OTPR = (OR + OS_MIN - 1) / OS_MIN;   // most tokens a member owns per tile
constexpr int OSLOTS = 5;               // exchange ring depth (tiles); see below
constexpr int ORR = 3;                  // LDS ring of partials (tiles)
constexpr int OMR = 5;                  // LDS ring of H_pre (tiles; a slot is rewritten once its tile's h is out)
constexpr int OKR = 4;                  // LDS ring of Sinkhorn inputs (tiles; taken two at a time)
constexpr int OD = 5;                   // tiles between a tile's partials and its h; see below
constexpr int OP = 2;                   // X tiles in flight ahead of the one being multiplied
constexpr int ONB = OD + OP;            // X tile buffers per lane
constexpr size_t OHDR = kOnePassHeaderBytes;   // workspace header: the error word
constexpr int OXCD = 8;                 // XCDs of the device (MI355X)
constexpr unsigned kLdsSpin = 1u << 20; // bounded waits: far beyond any legitimate one
constexpr unsigned kMemSpin = 1u << 16;
constexpr unsigned kStartSpin = 1u << 12; // the team's meeting: members start within microseconds of each other
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every range: loads read 0, stores drop

// Progress and slot reuse.  In step k a streaming wave writes tile k's
// partials, posts its share of tile k-1's record, then emits tile k-OD,
// which waits for that tile's H_pre.  An exchange wave handles tile j once
// every streaming wave of its member has posted tile j's record: B (read the
// members' records of the owned tokens, post H_pre) and C (read all owners'
// H_pre).  Nothing waits for a later step, so every wait ends.
// A member posts tile k's record after finishing step k, hence after
// emitting tile k-OD, hence after its C of every tile <= k-OD, which came
// after every owner's B of those tiles.  Tile k's record and H_pre words
// overwrite those of tile k-OSLOTS, which is therefore read by then when
// OSLOTS >= OD; tile k's H_pre goes into LDS slot k % OMR, whose previous
// tile, k-OMR, has been emitted when OMR >= OD.
static_assert(OSLOTS >= OD, "exchange words of a tile are rewritten only after every member has read them");
static_assert(OMR >= OD, "an H_pre slot in LDS is rewritten only after its tile has been emitted");
static_assert(OD >= 2, "a tile's H_pre needs the next step's record post");

struct OneArgs {
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
  u64* hdr;        // [0] error word
  u64* start;      // [team][OS_MAX] start words
  u64* ring;       // [team][OSLOTS][slot words]
  int64_t slotw;   // words per slot: S * OR * record words, then OR * n H_pre words
  u64 epoch;       // sequence number of the call (never 0)
  int xbytes, hbytes;
  int force_break; // testing aid: every workgroup starts broken, so the call falls back
};

__device__ __forceinline__ u64 xword(uint32_t v, uint32_t tag) {
  return (static_cast<u64>(tag) << 32) | static_cast<u64>(v);
}
__device__ __forceinline__ u64 agent_load(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Flags in LDS, shared by the workgroup's waves.  Atomic accesses (never
// cached in registers, never merged) on the variables themselves, so the
// compiler keeps them LDS operations: a generic (flat) access would also
// count as a vector memory operation, and waiting for it would wait for
// every X load in flight.
__device__ __forceinline__ int flag_get(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_set(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// LDS writes issued so far have completed: a wave that then sees a flag
// written after this point also sees them.
__device__ __forceinline__ void lds_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Wait (wave-uniform) until *flag >= want.  false when the workgroup is or
// becomes broken.
__device__ __forceinline__ bool wait_ge(int* flag, int want, int* broken) {
  unsigned n = 0;
  while (flag_get(flag) < want) {
    if (flag_get(broken)) return false;
    if (++n > kLdsSpin) {
      flag_set(broken, 1);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Wait (wave-uniform) until flags[w] >= want for every w < OW; lane w
// reads flag w.
__device__ __forceinline__ bool wait_all_ge(int* flags, int want, int* broken, int lane) {
  unsigned n = 0;
  while (true) {
    const int v = (lane < OW) ? flag_get(&flags[lane < OW ? lane : 0]) : 0x7fffffff;
    if (__all(v >= want)) return true;
    if (flag_get(broken)) return false;
    if (++n > kLdsSpin) {
      flag_set(broken, 1);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Sum over the 16 lanes of a row in fp64, the same bits on every lane: quad
// butterfly (partners e^1, e^2), then partners e^8 (rotation by 8), then the
// other pair of quads (rotation by 4: either direction reaches a lane of the
// same pair, so every lane adds the same two values).
template <int CTRL>
__device__ __forceinline__ double dpp64(double v) {
  const u64 b = __builtin_bit_cast(u64, v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false));
  return __builtin_bit_cast(double, (static_cast<u64>(hi) << 32) | lo);
}
__device__ __forceinline__ double row16_sum(double v) {
  v = v + dpp64<0xB1>(v);
  v = v + dpp64<0x4E>(v);
  v = v + dpp64<0x128>(v);
  v = v + dpp64<0x124>(v);
  return v;
}

template <int N, bool HC>
__global__ __launch_bounds__(OT) void pre_one_pass_kernel(OneArgs a) {
  constexpr int M = num_maps(N);
  constexpr int NB = (M + 15) / 16;
  constexpr int NN = N * N;
  constexpr int SSO = (M + 1) & ~1;     // word of the sum of squares in a token record (even)
  constexpr int W = SSO + 2;            // words per token record (even: records are 16-byte pairs)
  constexpr int NP = W / 2;             // word pairs per token record
  constexpr int NRB = (NP + 3) / 4;     // reduce-scatter loads per owned token (a pair per 16-lane row)
  constexpr int PHE = 4 * M;            // phi operand entries per (wave, stream, half)
  constexpr int MP = (M + 3) / 4;       // 4-column groups per token in the partials ring
  constexpr int SHARE = (OR * NP + OW - 1) / OW;   // record pairs each streaming wave posts per tile
  static_assert(SHARE <= 64, "one pair per lane");

  __shared__ u32x4 phi_l[OW][N][2][PHE];   // MFMA B operands, entry nb*64 + g*cn + r (cn = columns of block nb)
  __shared__ f32x4 red[ORR][OW][OR][MP];   // per wave and token: m partials (padded to 4s)
  __shared__ double red_ss[ORR][OW][OR];
  __shared__ double xs[OX][OTPR][W];       // an owned token's column sums over the team, per exchange wave
  __shared__ float maps[OMR][OR][N];
  __shared__ float2 skin[OKR][OTPR][16];   // (residual logit or HC value, gate value) per entry
  __shared__ int64_t sktok[OKR][OTPR];     // global token, or -1
  __shared__ int part_ready[OW];           // wave w has written the partials of tiles < part_ready[w]
  __shared__ int posted[OW];               // wave w has posted its record share of tiles < posted[w]
  __shared__ int maps_tag[OMR];            // H_pre of tile t is in slot t % OMR once maps_tag[slot] > t
  __shared__ int sk_tag[OKR];              // likewise for the Sinkhorn inputs
  __shared__ int sk_free, broken;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int* const vbroken = &broken;

  // Team membership: the team from the hardware XCD id, the place on the
  // XCD from the workgroup index (round-robin dispatch puts workgroups b,
  // b + 8, b + 16, ... on one XCD, whichever XCD the rotation starts at).
  __shared__ int xcc_l;
  if (tid == 0) {
    xcc_l = static_cast<int>(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7);   // HW_REG_XCC_ID
    for (int q = 0; q < OMR; ++q) maps_tag[q] = 0;
    for (int q = 0; q < OKR; ++q) {
      sk_tag[q] = 0;
      for (int o = 0; o < OTPR; ++o) sktok[q][o] = -1;
    }
    sk_free = 0;
    broken = a.force_break;
  }
  if (tid < OW) {
    part_ready[tid] = 0;
    posted[tid] = 0;
  }
  __syncthreads();
  const int S = a.S;
  const int idx = static_cast<int>(blockIdx.x) / OXCD;
  if (idx >= a.tpx * S) return;   // not part of a team (whole workgroup)
  const int team = xcc_l * a.tpx + idx / S;
  const int s = idx % S;
  const int d = a.d;
  const int64_t T = a.T;
  const int teams = a.teams;
  const int J = (a.ntiles > team) ? static_cast<int>((a.ntiles - team + teams - 1) / teams) : 0;

  // Streaming lanes: lane = (token row r16, position group g) of wave w.
  const int w = wave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int j0 = s * OSLICE + 32 * w + 8 * g;
  const bool jv = wave < OW && j0 < d;
  const __amdgpu_buffer_rsrc_t xrx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X), 0, a.xbytes, 0x00020000);
  auto load_tile = [&](int jt, u32x4 (&x)[N]) {
    const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + r16;
    const bool ok = jt < J && t < T && jv;
    const uint32_t o0 = ok ? static_cast<uint32_t>((t * N * d + j0) * 2) : kOob;
    const uint32_t st = ok ? static_cast<uint32_t>(d * 2) : 0u;
#pragma unroll
    for (int i = 0; i < N; ++i)
      x[i] = __builtin_amdgcn_raw_buffer_load_b128(xrx, static_cast<int>(o0 + i * st), 0, 2);
  };
  // The first X tiles go out before the set-up below, which they overlap.
  u32x4 xb[ONB][N];
  if (wave < OW) {
#pragma unroll
    for (int p = 0; p < OP; ++p) {
      load_tile(p, xb[p]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // This member's slice of phi into LDS as bf16 hi / lo operand halves: the
  // slice's rows of each stream are contiguous in phi, read in 16-byte
  // pieces (all issued before any is used), and each value goes to element
  // e of operand entry (wave, stream, column) for its position 32 w + 8 g + e.
  {
    constexpr int G = (M % 4 == 0) ? 4 : 1;            // floats per load
    constexpr int PER = OSLICE * M / G;                  // loads per stream
    constexpr int KPHI = (N * PER + OT - 1) / OT;
    float pv[KPHI][G];
#pragma unroll
    for (int k = 0; k < KPHI; ++k) {
      const int q = tid + k * OT;
      const int i = q / PER;
      const int f = (q - i * PER) * G;
      const int row = f / M;
      const int j = s * OSLICE + row;
      const bool ok = q < N * PER && j < d;
      const float* src = a.phi + (static_cast<int64_t>(i) * d + j) * M + (f - row * M);
      if constexpr (G == 4) {
        const f32x4 v = ok ? *reinterpret_cast<const f32x4*>(src) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) pv[k][c] = v[c];
      } else {
        pv[k][0] = ok ? *src : 0.0f;
      }
    }
#pragma unroll
    for (int k = 0; k < KPHI; ++k) {
      const int q = tid + k * OT;
      if (q < N * PER) {
        const int i = q / PER;
        const int f = (q - i * PER) * G;
        const int row = f / M;
        const int ww = row >> 5, gg = (row >> 3) & 3, e = row & 7;
#pragma unroll
        for (int c = 0; c < G; ++c) {
          const int col = f - row * M + c;
          const int nb = col >> 4;
          const int cn = (M - 16 * nb < 16) ? M - 16 * nb : 16;
          const int ent = 64 * nb + gg * cn + (col & 15);
          const __bf16 hi = static_cast<__bf16>(pv[k][c]);
          const __bf16 lo = static_cast<__bf16>(pv[k][c] - static_cast<float>(hi));
          reinterpret_cast<__bf16*>(&phi_l[ww][i][0][ent])[e] = hi;
          reinterpret_cast<__bf16*>(&phi_l[ww][i][1][ent])[e] = lo;
        }
      }
    }
  }

  // Clear this member's words of every ring slot (its records, the H_pre
  // words of the tokens it owns) before any wave posts into them; the team
  // then meets on the start words, so no member reads a slot before its
  // writer has cleared it.
  u64* const tring = a.ring + static_cast<int64_t>(team) * OSLOTS * a.slotw;
  const int64_t recw = static_cast<int64_t>(S) * OR * W;   // record words per slot
  for (int q = tid; q < OSLOTS * OR * W; q += OT)
    tring[(q / (OR * W)) * a.slotw + static_cast<int64_t>(s) * OR * W + q % (OR * W)] = 0ull;
  for (int q = tid; q < OSLOTS * OTPR * N; q += OT) {
    const int sl = q / (OTPR * N);
    const int r = q - sl * (OTPR * N);
    const int tok = s + (r / N) * S;
    if (r / N < a.tpr && tok < OR) tring[sl * a.slotw + recw + tok * N + r % N] = 0ull;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  const int ring_bytes = static_cast<int>(OSLOTS * a.slotw * 8);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(tring, 0, ring_bytes, 0x00020000);
  constexpr int kOff = 0x7FFFFFF0;       // past the ring
  auto rec_off = [&](int jt, int m, int tok, int word) -> int {
    return static_cast<int>(((jt % OSLOTS) * a.slotw + (m * OR + tok) * W + word) * 8);
  };

  if (wave < OW) {
    // ---------------------------------------------------------------- streaming
    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(a.h, 0, a.hbytes, 0x00020000);

    // Tile jt's partials over this wave's 32 positions into the LDS ring.
    // Sum of squares: with A = B = the tile (16 tokens x 32 positions), the
    // MFMA's diagonal entry (t, t) is token t's sum of squares over the
    // wave's positions; bf16 products are exact in fp32, the accumulation
    // over the 4 streams' 128 values is fp32, the sums across waves and
    // members fp64.  Entry (t, t) sits in lane 16 (t / 4) + t, element t % 4.
    auto partials = [&](int jt, const u32x4 (&x)[N]) {
      f32x4 gram = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const bf16x8 xv = __builtin_bit_cast(bf16x8, x[i]);
        gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int cn = (M - 16 * nb < 16) ? M - 16 * nb : 16;
          // A block narrower than 16 columns (the last one) repeats valid
          // entries in its unused columns: output column c depends only on
          // B column c, and columns >= m are never written out.
          const int ent = 64 * nb + g * cn + (r16 < cn ? r16 : r16 - cn);
          PhiOp<BF16> b;
          b.hi = __builtin_bit_cast(bf16x8, phi_l[w][i][0][ent]);
          b.lo = __builtin_bit_cast(bf16x8, phi_l[w][i][1][ent]);
          acc[nb] = mfma_block(Raw8<BF16>{x[i]}, b, acc[nb]);
        }
        __builtin_amdgcn_sched_barrier(0);   // read phi per stream, next to its MFMAs (registers)
      }
      const int dv = r16 & 3;
      const float sqf = dv == 0 ? gram[0] : dv == 1 ? gram[1] : dv == 2 ? gram[2] : gram[3];
      double sq = static_cast<double>(sqf);
      const bool ovf = g == (r16 >> 2) && !__builtin_isfinite(sqf);
      if (__any(ovf)) {
        // fp32 overflow (|x| beyond ~1e18): the token's sum again in fp64
        // from the 4 lanes that hold its positions (lane 16 q + t holds
        // positions 8 q .. 8 q + 7).  Wave-uniform branch: every lane
        // takes part in the permutes.
        double s64 = 0.0;
        for (int q = 0; q < 4; ++q) {
          const int src = 16 * q + r16;
#pragma unroll
          for (int i = 0; i < N; ++i) {
            u32x4 xq;
#pragma unroll
            for (int c = 0; c < 4; ++c)
              xq[c] = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * src, static_cast<int>(x[i][c])));
            float v[8];
            unpack8(Raw8<BF16>{xq}, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) s64 = fma(static_cast<double>(v[e]), static_cast<double>(v[e]), s64);
          }
        }
        if (ovf) sq = s64;
      }
      const int slot = jt % ORR;
      wait_all_ge(posted, jt - ORR + 1, vbroken, lane);   // every wave has posted the slot's last tile
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 16 * nb + r16;
        if (col < M) {
#pragma unroll
          for (int v = 0; v < 4; ++v) red[slot][w][4 * g + v][col >> 2][col & 3] = acc[nb][v];
        }
      }
      if (g == (r16 >> 2)) red_ss[slot][w][r16] = sq;
      lds_done();
      if (lane == 0) flag_set(&part_ready[w], jt + 1);
    };

    // This wave's share of tile jp's record: pairs SHARE w .. SHARE w + SHARE-1
    // of the 16 tokens x NP pairs, each the 8 waves' partials added in wave
    // order, posted with one 16-byte store (lanes without a pair store out of
    // range, which moves no data).
    auto post_share = [&](int jp) {
      const bool have = jp >= 0 && jp < J;
      if (have) wait_all_ge(part_ready, jp + 1, vbroken, lane);
      const int q = SHARE * w + lane;
      const bool qv = have && lane < SHARE && q < OR * NP;
      const int qq = qv ? q : 0;
      const int tok = qq / NP;
      const int p = qq - tok * NP;
      const int rs = (have ? jp : 0) % ORR;
      uint32_t v0 = 0u, v1 = 0u;
      if (qv) {
        if (2 * p == SSO) {
          double sd = red_ss[rs][0][tok];
#pragma unroll
          for (int ww = 1; ww < OW; ++ww) sd += red_ss[rs][ww][tok];
          const u64 b = __builtin_bit_cast(u64, sd);
          v0 = static_cast<uint32_t>(b);
          v1 = static_cast<uint32_t>(b >> 32);
        } else {
          // columns 2p and 2p + 1: one 8-byte read per wave
          const float2* r2 = reinterpret_cast<const float2*>(&red[rs][0][tok][0]) + p;
          constexpr int WS = OR * MP * 2;                 // float2 stride between waves
          float2 x = r2[0];
#pragma unroll
          for (int ww = 1; ww < OW; ++ww) {
            const float2 y = r2[ww * WS];
            x.x += y.x;
            x.y += y.y;
          }
          v0 = __float_as_uint(x.x);
          v1 = __float_as_uint(x.y);
        }
      }
      const uint32_t tag = static_cast<uint32_t>(jp + 1);
      const int off = qv ? rec_off(jp, s, tok, 2 * p) : kOff;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{v0, tag, v1, tag}, xr, off, 0, 0);
      lds_done();
      if (have && lane == 0) flag_set(&posted[w], jp + 1);
    };

    auto emit = [&](int jt, const u32x4 (&x)[N]) {
      const bool have = jt >= 0 && jt < J;
      float hp[N];
#pragma unroll
      for (int i = 0; i < N; ++i) hp[i] = 0.0f;
      if (have) {
        wait_ge(&maps_tag[jt % OMR], jt + 1, vbroken);
#pragma unroll
        for (int i = 0; i < N; ++i) hp[i] = maps[jt % OMR][r16][i];
      }
      const u32x4 (&y)[N] = x;
      float o[8];
      {
        float v[8];
        unpack8(Raw8<BF16>{y[0]}, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = hp[0] * v[e];
      }
#pragma unroll
      for (int i = 1; i < N; ++i) {
        float v[8];
        unpack8(Raw8<BF16>{y[i]}, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(hp[i], v[e], o[e]);
      }
      const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + r16;
      const bool ok = have && t < T && jv;
      const uint32_t ho = ok ? static_cast<uint32_t>((t * d + j0) * 2) : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(pack8(o, BF16{}).v, hr, static_cast<int>(ho), 0, 2);
    };

    // Tile k lives in buffer k % ONB; the buffer of tile k - OD, emitted in
    // step k, then receives tile k + OP.  Every step issues N loads and two
    // stores, with no branch around any of them.
    const int kend = ((J + OD + ONB - 1) / ONB) * ONB;
    for (int k0 = 0; k0 < kend; k0 += ONB) {
#pragma unroll
      for (int u = 0; u < ONB; ++u) {
        const int k = k0 + u;
        if (k < J) partials(k, xb[u]);
        post_share(k - 1);
        emit(k - OD, xb[(u + OP) % ONB]);
        load_tile(k + OP, xb[(u + OP) % ONB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (wave < OW + OX) {
    // ---------------------------------------------------------------- exchange
    // Exchange wave x takes the tiles t with t % OX == x.  Meet the team
    // first: every member's slots are clear once its start word holds this
    // call's sequence number.
    __builtin_amdgcn_s_setprio(2);
    const int xw = wave - OW;
    u64* st = a.start + static_cast<int64_t>(team) * OS_MAX;
    if (lane == 0 && xw == 0) st[s] = a.epoch;
    if (lane < S) {
      unsigned n = 0;
      while (agent_load(st + lane) != a.epoch) {
        if (flag_get(vbroken)) break;
        if (++n > kStartSpin) {
          flag_set(vbroken, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }

    const int tpr = a.tpr;
    // Loads carry sc1: they skip the CU's L1 and read the XCD's L2.  Few,
    // wide memory instructions: this wave shares the CU's memory pipeline
    // with the streaming waves and would otherwise queue behind their loads.
    auto ld2 = [&](int off) -> u32x4 { return __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 16); };
    // Reduce-scatter reads: load r of owned token o covers word pairs 4 r ..
    // 4 r + 3, one per 16-lane row; lane m of a row reads member m's pair.
    const int rq = lane >> 4;
    const int rm = lane & 15;
    auto rs_off = [&](int jt, int o, int r) -> int {
      const int p = 4 * r + rq;
      const int tok = s + o * S;
      if (o >= tpr || tok >= OR || p >= NP || rm >= S) return kOff;
      return rec_off(jt, rm, tok, 2 * p);
    };
    auto bc_off = [&](int jt) -> int {
      return (2 * lane < OR * N) ? static_cast<int>(((jt % OSLOTS) * a.slotw + recw + 2 * lane) * 8) : kOff;
    };
    // Wait until both words of a pair carry `tag` (reading it again as needed).
    auto settle = [&](u32x4 v, int off, uint32_t tag) -> u32x4 {
      unsigned n = 0;
      while (off != kOff && (v.y != tag || v.w != tag)) {
        if (flag_get(vbroken)) break;
        if (++n > kMemSpin) {
          flag_set(vbroken, 1);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        asm volatile("" ::: "memory");
        v = ld2(off);
      }
      return v;
    };
    u32x4 rsv[OTPR][NRB];
    // Lane (o, e) of the maps: entry e of owned token o.  Its bias values are
    // fixed per lane: loaded once, not behind the streaming loads every tile.
    const int o = lane >> 4;
    const int e = lane & 15;
    const int colr = N + e;
    const int colg = (e < N) ? e : (N + NN + (e - N));
    const int cr = e < NN ? colr : 0, cg = e < 2 * N ? colg : 0;
    const float bias_r = a.bias[cr], bias_g = a.bias[cg];
    const float alpha_g = (e < N) ? a.a_pre : a.a_post;
    // Tile jb: once this member's waves have posted their record of it (the
    // other members post theirs at about the same time), the reduce-scatter
    // (B) and then the broadcast of the owners' H_pre (C).
    for (int jb = xw; jb < J; jb += OX) {
      wait_all_ge(posted, jb + 1, vbroken, lane);
#pragma unroll
      for (int o = 0; o < OTPR; ++o) {
        if (o < tpr) {
#pragma unroll
          for (int r = 0; r < NRB; ++r) rsv[o][r] = ld2(rs_off(jb, o, r));
        }
      }
      const uint32_t tag = static_cast<uint32_t>(jb + 1);
      // B: the team's sums for the tokens this member owns: a fixed tree over
      // the members across each 16-lane row, in fp64.
#pragma unroll
      for (int o = 0; o < OTPR; ++o) {
        if (o < tpr) {
#pragma unroll
          for (int r = 0; r < NRB; ++r) {
            const int off = rs_off(jb, o, r);
            const u32x4 v = settle(rsv[o][r], off, tag);
            const int p = 4 * r + rq;
            double d0 = 0.0, d1 = 0.0;
            if (off != kOff) {
              if (2 * p == SSO) {
                d0 = __builtin_bit_cast(double, (static_cast<u64>(v.z) << 32) | v.x);
              } else {
                d0 = static_cast<double>(__uint_as_float(v.x));
                d1 = static_cast<double>(__uint_as_float(v.z));
              }
            }
            d0 = row16_sum(d0);
            d1 = row16_sum(d1);
            if (rm == 0 && p < NP) {
              xs[xw][o][2 * p] = d0;
              xs[xw][o][2 * p + 1] = d1;
            }
          }
        }
      }
      lds_done();
      const int tok = s + o * S;
      const bool own = o < tpr && tok < OR;
      const int oo = o < OTPR ? o : 0;
      const double ss = xs[xw][oo][SSO];
      const double zr = xs[xw][oo][cr];
      const double zg = xs[xw][oo][cg];
      const double inv_r = inv_rms(ss, N * d, a.eps);
      float gv = 0.0f, rv = -INFINITY;
      if constexpr (HC) {
        if (e < 2 * N)
          gv = static_cast<float>(static_cast<double>(bias_g) + static_cast<double>(alpha_g) * tanh(zg * inv_r));
        rv = (e < NN) ? static_cast<float>(static_cast<double>(bias_r) +
                                           static_cast<double>(a.a_res) * tanh(zr * inv_r))
                      : 0.0f;
      } else {
        if (e < 2 * N) {
          const float l = logit_of(zg, inv_r, alpha_g, bias_g);
          gv = (e < N) ? sigmoidf_(l) : 2.0f * sigmoidf_(l);
        }
        if (e < NN) rv = logit_of(zr, inv_r, a.a_res, bias_r);
      }
      u64* slot = tring + (jb % OSLOTS) * a.slotw;
      if (own && e < N) slot[recw + tok * N + e] = xword(__float_as_uint(gv), tag);
      // C's read goes out now; the other owners post at about the same time.
      const int boff = bc_off(jb);
      u32x4 bcv = ld2(boff);
      // Hand the token's values to the Sinkhorn wave.
      wait_ge(&sk_free, jb - OKR + 1, vbroken);
      const int ks = jb % OKR;
      if (o < OTPR) {
        skin[ks][o][e] = make_float2(rv, gv);
        const int64_t t = (team + static_cast<int64_t>(jb) * teams) * OR + tok;
        if (e == 0) sktok[ks][o] = (own && t < T) ? t : -1;
      }
      lds_done();
      if (lane == 0) flag_set(&sk_tag[ks], jb + 1);
      // C: H_pre of the tile's 16 tokens, for the streaming waves.
      bcv = settle(bcv, boff, tag);
      if (boff != kOff) {
        const int w0 = 2 * lane;
        maps[jb % OMR][w0 / N][w0 % N] = __uint_as_float(bcv.x);
        maps[jb % OMR][(w0 + 1) / N][(w0 + 1) % N] = __uint_as_float(bcv.z);
      }
      lds_done();
      if (lane == 0) flag_set(&maps_tag[jb % OMR], jb + 1);
    }
    if (flag_get(vbroken) && lane == 0) __hip_atomic_store(a.hdr, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    // ----------------------------------------------------------------- Sinkhorn
    // Two tiles per pass: lanes 32 q .. 32 q + 31 take tile jt + q, 16 lanes
    // per owned token.
    __builtin_amdgcn_s_setprio(2);
    const int q = lane >> 5;
    const int o = (lane >> 4) & 1;
    const int e = lane & 15;
    const int colg = (e < N) ? e : (N + NN + (e - N));
    for (int jt = 0; jt < J; jt += 2) {
      const int jn = (jt + 2 < J) ? jt + 2 : J;
      wait_ge(&sk_tag[jt % OKR], jt + 1, vbroken);
      if (jt + 1 < J) wait_ge(&sk_tag[(jt + 1) % OKR], jt + 2, vbroken);
      const int tj = jt + q;
      const bool tv = tj < J;
      const int ks = (tv ? tj : jt) % OKR;
      const float2 in = skin[ks][o][e];
      const int64_t t = tv ? sktok[ks][o] : -1;
      lds_done();
      if (lane == 0) flag_set(&sk_free, jn);
      float mv = in.x;
      if constexpr (!HC) mv = sinkhorn16<N>(e < NN ? in.x : -INFINITY, e, a.t_max);
      if (t >= 0 && t < a.T) {             // (a broken workgroup may read a slot before it is written)
        float* Ht = a.H + t * M;
        if (e < NN) Ht[N + e] = mv;
        if (e < 2 * N) Ht[colg] = in.y;
      }
    }
  }
}

int one_pass_slices(int d) { return (d + OSLICE - 1) / OSLICE; }

// Token record: m partials, padding to an even word, the fp64 sum of squares.
int record_words(int n) { return ((num_maps(n) + 1) & ~1) + 2; }
int64_t slot_words(int S, int n) { return static_cast<int64_t>(S) * OR * record_words(n) + OR * n; }

int max_teams(int S) { return OXCD * (48 / S); }   // devices with up to 48 CUs per XCD

template <int N, bool HC>
const void* one_pass_kernel_ptr() {
  return reinterpret_cast<const void*>(&pre_one_pass_kernel<N, HC>);
}

std::atomic<u64> g_epoch{0};

}  // namespace

// Bytes the single-pass form needs: header, start words and the exchange
// ring, for devices with up to 48 CUs per XCD.
size_t pre_fused_workspace_bytes(int64_t /*T*/, int n, int d) {
  const int S = one_pass_slices(d);
  if (S < OS_MIN || S > OS_MAX) return 0;
  const int teams = max_teams(S);
  return OHDR + static_cast<size_t>(teams) * OS_MAX * sizeof(u64) +
         static_cast<size_t>(teams) * OSLOTS * static_cast<size_t>(slot_words(S, n)) * sizeof(u64);
}

// Whether MHC_PRE_AUTO takes the single pass: measured faster on MI355X for
// n = 4 when the teams fill whole XCDs and each gets at least 40 tiles (at
// T = 16384, d = 4096: 194 us against 227 us); for n <= 2 a tile carries too
// little data to hide the exchange.
bool pre_fused_preferred(const mhc_params& p, const DeviceInfo& dev) {
  if (p.dtype != MHC_BF16 || p.n != 4 || dev.num_cus % OXCD != 0) return false;
  const int S = one_pass_slices(p.d);
  const int per_xcd = dev.num_cus / OXCD;
  if (S < OS_MIN || S > OS_MAX || per_xcd % S != 0) return false;
  const int64_t teams = static_cast<int64_t>(OXCD) * (per_xcd / S);
  return (p.T + OR - 1) / OR >= 40 * teams;
}

// Launch the single-pass form when it applies; returns hipErrorNotSupported
// (without launching anything) when it does not, so the caller can fall back.
hipError_t launch_pre_fused(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, size_t ws_bytes, const DeviceInfo& dev, hipStream_t stream) {
  if (p.dtype != MHC_BF16 || (p.n != 4 && p.n != 2 && p.n != 1)) return hipErrorNotSupported;
  // Not under stream capture: a graph replays the captured call's sequence
  // number, so words left by the previous replay would pass for this one's.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone)
    return hipErrorNotSupported;
  const int S = one_pass_slices(p.d);
  if (S < OS_MIN || S > OS_MAX || dev.num_cus % OXCD != 0) return hipErrorNotSupported;
  const int per_xcd = dev.num_cus / OXCD;
  const int tpx = per_xcd / S;
  if (tpx < 1) return hipErrorNotSupported;
  const int teams = OXCD * tpx;
  if (teams > max_teams(S)) return hipErrorNotSupported;
  const int64_t ntiles = (p.T + OR - 1) / OR;
  if (ntiles < teams) return hipErrorNotSupported;   // too little work to give every team a tile
  // Buffer ranges are 31-bit byte counts.
  const int64_t xbytes = p.T * p.n * static_cast<int64_t>(p.d) * 2;
  const int64_t hbytes = p.T * static_cast<int64_t>(p.d) * 2;
  if (xbytes >= (int64_t{1} << 31) || p.T < 1) return hipErrorNotSupported;
  if (pre_fused_workspace_bytes(p.T, p.n, p.d) > ws_bytes) return hipErrorNotSupported;
  const bool hc = p.maps == MHC_MAPS_HC;
  const void* fn = nullptr;
  switch (p.n) {
    case 1: fn = hc ? one_pass_kernel_ptr<1, true>() : one_pass_kernel_ptr<1, false>(); break;
    case 2: fn = hc ? one_pass_kernel_ptr<2, true>() : one_pass_kernel_ptr<2, false>(); break;
    default: fn = hc ? one_pass_kernel_ptr<4, true>() : one_pass_kernel_ptr<4, false>(); break;
  }
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, OT, 0) != hipSuccess || occ < 1)
    return hipErrorNotSupported;

  char* base = static_cast<char*>(workspace);
  OneArgs a;
  a.T = p.T;
  a.d = p.d;
  a.S = S;
  a.tpx = tpx;
  a.teams = teams;
  a.tpr = (OR + S - 1) / S;
  a.ntiles = ntiles;
  a.X = static_cast<const uint16_t*>(X);
  a.phi = phi;
  a.bias = bias;
  a.a_pre = p.alpha_pre;
  a.a_res = p.alpha_res;
  a.a_post = p.alpha_post;
  a.eps = p.eps;
  a.t_max = p.t_max;
  a.h = static_cast<uint16_t*>(h);
  a.H = H;
  a.hdr = reinterpret_cast<u64*>(base);
  a.start = reinterpret_cast<u64*>(base + OHDR);
  a.ring = a.start + static_cast<size_t>(max_teams(S)) * OS_MAX;
  a.slotw = slot_words(S, p.n);
  a.epoch = ++g_epoch;
  a.xbytes = static_cast<int>(xbytes);
  a.hbytes = static_cast<int>(hbytes);
  const char* fb = std::getenv("MHC_TEST_ONE_PASS_FALLBACK");
  a.force_break = (fb != nullptr && fb[0] == '1') ? 1 : 0;
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3(dev.num_cus), dim3(OT), args, 0, stream);
  if (e != hipSuccess) return e;
  // The fallback: the two-pass form, gated on this call's sequence number in
  // the error word, so it runs only if a wait of the single pass ran out.
  return launch_pre_gated(p, X, phi, bias, h, H, base + OHDR, dev, a.hdr, a.epoch, stream);
}

}  // namespace mhc
