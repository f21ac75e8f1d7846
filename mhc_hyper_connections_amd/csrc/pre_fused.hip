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
//  * waves 0-7 stream.  Wave w holds line w % 4 of the member's slice (64
//    positions, 128 bytes of every stream row) for tokens 8 (w / 4) .. + 7
//    of a tile in registers (lane = token and 8 positions of all n streams;
//    each load and store covers whole 128-byte lines).  In step k it forms
//    tile k's m partial dot products with phi on MFMA (phi as bf16 hi + lo
//    halves, kept in LDS; the A operand's rows 0..7 hold the line's first
//    32 positions, rows 8..15 its last 32) and the partial sums of squares
//    (the diagonal of a 16 x 16 Gram matrix, also on MFMA) into an LDS ring;
//    once tile k-OD's H_pre has come back, forms h = H_pre . X for its
//    positions from the registers that still hold that tile, and stores it;
//    prefetches tile k+OP; and last sums its eighth of tile k's record over
//    the token's rows (position order) and posts it with one 16-byte store
//    (by then the other waves have written tile k's partials).  These
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
// before any wave posts, and the team meets on start words stamped with the
// call's tag, so words of earlier calls never match.  The tag comes from a
// sequence number kept in the workspace's header, which the kernel after the
// single pass advances; nothing on the host counts calls, so a call captured
// into a HIP graph gets a fresh tag at every replay.  Every sum runs in a
// fixed order: results are bitwise reproducible.  All waits are bounded; one
// that runs out marks the workgroup broken (no further waits; its results are
// garbage, its writes stay in bounds) and the call's tag, XORed with a fixed
// pattern, is stored into the header's error word (the pattern keeps a header
// whose words all hold the same initial bytes from reading as a failure).
// The launch is an ordinary one of one workgroup per CU, which on an idle
// device makes every team resident together; a cooperative launch would
// guarantee it but costs about 16 us more per call on MI355X.  The guarantee
// is replaced by a fallback: pre_one_pass_fallback_kernel follows the single
// pass on the stream.  Its workgroups return at once unless the error word
// holds this call's tag; then they recompute every output with the single
// pass's own arithmetic and summation order but no exchange (each workgroup
// takes whole tiles and walks the members' slices itself), so the results
// are bitwise those of an undisturbed single pass.
// The exchange and Sinkhorn waves run at a raised issue priority: the
// streaming waves have slack, the exchange is on every tile's critical path.
#include "launch.hpp"
#include "pre_common.hpp"

namespace mhc {
namespace {

typedef unsigned long long u64;

constexpr int OW = 8;                   // streaming waves
constexpr int OX = 2;                   // exchange waves (tiles alternate between them; three measured the same)
constexpr int OT = (OW + OX + 1) * 64;  // + the exchange waves + the Sinkhorn wave
constexpr int OTP = OT + 64;            // with the previous layer's mhc_post fused in: + the maps loader wave
constexpr int OHR = 4;                  // LDS ring of the previous layer's mixing maps (tiles)
constexpr int OSLICE = OW * 32;         // positions of d per member
constexpr int OR = 16;                  // tokens per tile
constexpr int OS_MIN = 8;               // team size range (ceil(d / OSLICE))
constexpr int OS_MAX = 16;
constexpr int OTPR = (OR + OS_MIN - 1) / OS_MIN;   // most tokens a member owns per tile
constexpr int OSLOTS = 5;               // exchange ring depth (tiles); see below
constexpr int ORR = 3;                  // LDS ring of partials (tiles)
constexpr int OMR = 5;                  // LDS ring of H_pre (tiles; a slot is rewritten once its tile's h is out)
constexpr int OKR = 4;                  // LDS ring of Sinkhorn inputs (tiles; taken two at a time)
constexpr int OD = 4;                   // tiles between a tile's partials and its h; see below
constexpr int OP = 2;                   // X tiles in flight ahead of the one being multiplied
// Both forms fit the streaming waves in 168 registers (3 waves per SIMD)
// without spilling.  The plain form's also hold three phi operands in flight
// (see partials); with the previous layer's post fused in, a step holds a
// chunk of Y and the mix's maps and temporaries instead, and one tile fewer
// is in flight.
constexpr int OD_POST = 4;
constexpr int OP_POST = 1;
constexpr size_t OHDR = kPreHeaderBytes;       // workspace header (error word, sequence number, current tag)
constexpr u64 kTagBit = 1ull << 63;     // set in every call's tag: a cleared or zeroed word never matches one
constexpr u64 kErrFlip = 0x5555555555555555ull;   // error word = tag ^ kErrFlip: never the raw sequence word
constexpr int OXCD = 8;                 // XCDs of the device (MI355X)
constexpr unsigned kLdsSpin = 1u << 20; // bounded waits: far beyond any legitimate one
constexpr unsigned kMemSpin = 1u << 16;
constexpr unsigned kStartSpin = 1u << 12; // the team's meeting: members start within microseconds of each other
constexpr uint32_t kOob = 0x80000000u;  // buffer offset past every range: loads read 0, stores drop

// Progress and slot reuse.  In step k a streaming wave writes tile k's
// partials, emits tile k-OD (which waits for that tile's H_pre), prefetches
// tile k+OP and then posts its share of tile k's record (which waits until
// every streaming wave has written tile k's partials).  An exchange wave handles tile j once
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
static_assert(OD >= 2, "a tile's H_pre comes back from the exchange at least a step after its record");
static_assert(OD_POST >= 2 && OD_POST <= OD && OP_POST >= 1, "the fused form's ring use is the plain form's");
// The partials ring needs no wait of its own: a wave writes tile k into slot
// k % ORR in step k after its post of tile k-1, which waited until every
// wave had written tile k-1's partials, so every wave had finished step k-2,
// including its post (the last read) of tile k-2 and of tile k-ORR <= k-2.
static_assert(ORR >= 2, "a partials slot is rewritten only after every wave has posted its tile");

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
  u64* hdr;        // [0] error word, [1] sequence number, [2] the current call's tag
  u64* start;      // [team][OS_MAX] start words
  u64* ring;       // [team][OSLOTS][slot words]
  int64_t slotw;   // words per slot: S * OR * record words, then OR * n H_pre words
  int nstart;      // start words in the workspace (max_teams(S) * OS_MAX)
  int xbytes, hbytes;
  int force_break; // testing aid: every workgroup starts broken, so the call falls back
  // With the previous layer's mhc_post fused in front (X is then X_l):
  const uint16_t* Y;   // [T, d] layer l's sublayer output
  const float* Hp;     // [T, m] layer l's maps
  uint16_t* Xo;        // [T, n, d] X_{l+1}, which the rest of the pass reads in place of X
};

__device__ __forceinline__ u64 xword(uint32_t v, uint32_t tag) {
  return (static_cast<u64>(tag) << 32) | static_cast<u64>(v);
}
__device__ __forceinline__ u64 agent_load(const u64* p) {
  return __hip_atomic_load(const_cast<u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The call's tag: the header's sequence number (advanced by the kernel that
// follows the single pass) with the top bit set.
__device__ __forceinline__ u64 call_tag(const OneArgs& a) { return agent_load(a.hdr + 1) | kTagBit; }
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

// mhc_post of one chunk (8 positions of all n streams of a token), in place:
// X_{l+1}[i] = sum_j H_res[i][j] X_l[j] + H_post[i] Y, each output value
// accumulated in fp32 in the order j = 0 .. n-1 and then the Y term, and
// rounded to bf16 (nearest, ties to even): mhc_post's arithmetic, so the bits
// are those mhc_post stores.
template <int N, bool RELOAD, typename Maps>
__device__ __forceinline__ void post_mix(u32x4 (&x)[N], const u32x4& y, const Maps& maps) {
  // Word c of every stream holds the same two positions: all n outputs of
  // them are formed from the n inputs, then written over those inputs.
  // maps(i, j) is H_res[i][j] and maps(i, n) H_post[i]; with RELOAD they are
  // fetched again for every word (from LDS), so that only one row is held.
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (RELOAD) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);   // one word at a time: the scheduler would unpack all 16 ahead
    }
    float xv[N][2];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      xv[j][0] = bf16_lo(x[j][c]);
      xv[j][1] = bf16_hi(x[j][c]);
    }
    const float y0 = bf16_lo(y[c]), y1 = bf16_hi(y[c]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float r0 = maps(i, 0);
      float o0 = r0 * xv[0][0];
      float o1 = r0 * xv[0][1];
#pragma unroll
      for (int j = 1; j < N; ++j) {
        const float rj = maps(i, j);
        o0 = fmaf(rj, xv[j][0], o0);
        o1 = fmaf(rj, xv[j][1], o1);
      }
      const float pi = maps(i, N);
      o0 = fmaf(pi, y0, o0);
      o1 = fmaf(pi, y1, o1);
      x[i][c] = pack_bf16(o0, o1);
    }
  }
}

template <int N, bool HC, bool POST>
__global__ __launch_bounds__(POST ? OTP : OT) void pre_one_pass_kernel(OneArgs a) {
  constexpr int NTHR = POST ? OTP : OT;
  constexpr int OD = POST ? OD_POST : ::mhc::OD;   // see OD_POST
  constexpr int OP = POST ? OP_POST : ::mhc::OP;
  constexpr int ONB = OD + OP;                      // X tile buffers per lane
  constexpr int M = num_maps(N);
  constexpr int NB = (2 * M + 15) / 16;   // column blocks: the m columns of a line's first half, then its second's
  constexpr int NN = N * N;
  constexpr int SSO = (M + 1) & ~1;     // word of the sum of squares in a token record (even)
  constexpr int W = SSO + 2;            // words per token record (even: records are 16-byte pairs)
  constexpr int NP = W / 2;             // word pairs per token record
  constexpr int NRB = (NP + 3) / 4;     // reduce-scatter loads per owned token (a pair per 16-lane row)
  constexpr int PHE = 64 * NB;          // phi operand entries per (line, stream, bf16 part)
  constexpr int MP = (M + 3) / 4;       // 4-column groups per token in the partials ring
  constexpr int SHARE = (OR * NP + OW - 1) / OW;   // record pairs each streaming wave posts per tile
  static_assert(SHARE <= 64, "one pair per lane");

  __shared__ u32x4 phi_l[4][N][2][PHE];    // MFMA B operands per line: entry 64 nb + 16 g + c
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
  constexpr int HF = N * N + N;            // a token's H_res and H_post (maps row words n .. m-1)
  __shared__ float hmix[POST ? OHR : 1][OR][HF];   // the previous layer's maps of a tile's tokens
  __shared__ int hmix_tag[OHR];             // slot t % OHR holds tile t's once hmix_tag[slot] > t

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
    for (int q = 0; q < OHR; ++q) hmix_tag[q] = 0;
    for (int q = 0; q < OKR; ++q) {
      sk_tag[q] = 0;
      for (int o = 0; o < OTPR; ++o) sktok[q][o] = -1;
    }
    sk_free = 0;
    broken = a.force_break;
    if (blockIdx.x == 0)   // the tag the fallback kernel compares the error word with
      __hip_atomic_store(a.hdr + 2, call_tag(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

  // Streaming lanes.  Wave w takes line L = w % 4 of the member's slice (64
  // positions: 128 bytes of every stream row) for tokens 8 (w / 4) .. + 7 of
  // a tile.  Lane 16 g + k holds token k % 8 at chunk g + 4 (k / 8) of the
  // line (8 positions), so every load and store covers 8 whole 128-byte
  // lines (16 rows of 64 bytes, half lines, ran 13% slower on reads alone).
  // Read as an MFMA A operand (row = lane % 16, K group = lane / 16), rows
  // 0..7 hold the line's first 32 positions of the 8 tokens and rows 8..15
  // its last 32: row 8 h + k carries exactly what row 8 (w / 4) + k of the
  // 32-position block 2 L + h did when a wave took a 16 x 32 block.
  static_assert(OW == 8 && OSLICE == 256 && OR == 16, "4 lines x 2 token halves per member");
  const int w = wave;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int L = w & 3;
  const int tk = 8 * (w >> 2) + (lane & 7);   // token within the tile
  const int j0 = s * OSLICE + 64 * L + 8 * (g + 4 * (r16 >> 3));
  const bool jv = wave < OW && j0 < d;
  const __amdgpu_buffer_rsrc_t xrx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.X), 0, a.xbytes, 0x00020000);
  auto load_tile = [&](int jt, u32x4 (&x)[N]) {
    const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + tk;
    const bool ok = jt < J && t < T && jv;
    const uint32_t o0 = ok ? static_cast<uint32_t>((t * N * d + j0) * 2) : kOob;
    const uint32_t st = ok ? static_cast<uint32_t>(d * 2) : 0u;
#pragma unroll
    for (int i = 0; i < N; ++i)
      x[i] = __builtin_amdgcn_raw_buffer_load_b128(xrx, static_cast<int>(o0 + i * st), 0, 2);
  };
  // X (and Y) are read with non-temporal loads: each instruction covers
  // whole 128-byte lines, so nothing is fetched twice, and X is not left in
  // the caches for the next kernel (in a model the sublayer runs between
  // this call and mhc_post).
  // The first X tiles go out before the set-up below, which they overlap.
  u32x4 xb[ONB][N];
  // With the previous layer's post fused in: the chunk of Y_l of the tile to
  // be mixed next (loaded one step ahead of its use).
  const __amdgpu_buffer_rsrc_t yrx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(POST ? a.Y : a.X), 0, a.hbytes, 0x00020000);
  auto load_y = [&](int jt) -> u32x4 {
    const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + tk;
    const bool ok = jt < J && t < T && jv;
    const uint32_t o0 = ok ? static_cast<uint32_t>((t * d + j0) * 2) : kOob;
    return __builtin_amdgcn_raw_buffer_load_b128(yrx, static_cast<int>(o0), 0, 2);
  };
  u32x4 yb = {0u, 0u, 0u, 0u};
  if (wave < OW) {
#pragma unroll
    for (int p = 0; p < OP; ++p) {
      load_tile(p, xb[p]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (POST) yb = load_y(0);
  }

  // This member's slice of phi into LDS as bf16 hi / lo operand parts: the
  // slice's rows of each stream are contiguous in phi, read in 16-byte
  // pieces (all issued before any is used).  Line L's operand column
  // q = 16 nb + c is map column q of the line's first 32 positions for
  // q < m and map column q - m of its last 32 for q >= m (zero past 2 m);
  // position 64 L + 32 h + 8 g + e is element e of entry 64 nb + 16 g + c.
  {
    constexpr int G = (M % 4 == 0) ? 4 : 1;            // floats per load
    constexpr int PER = OSLICE * M / G;                  // loads per stream
    constexpr int KPHI = (N * PER + NTHR - 1) / NTHR;
    float pv[KPHI][G];
#pragma unroll
    for (int k = 0; k < KPHI; ++k) {
      const int q = tid + k * NTHR;
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
    if constexpr (2 * M < 16 * NB) {
      for (int q = tid; q < 4 * N * 2 * PHE; q += NTHR) {
        const int ent = q % PHE;
        if (16 * (ent >> 6) + (ent & 15) >= 2 * M) (&phi_l[0][0][0][0])[q] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < KPHI; ++k) {
      const int q = tid + k * NTHR;
      if (q < N * PER) {
        const int i = q / PER;
        const int f = (q - i * PER) * G;
        const int row = f / M;
        const int ln = row >> 6, hh = (row >> 5) & 1, gg = (row >> 3) & 3, e = row & 7;
#pragma unroll
        for (int c = 0; c < G; ++c) {
          const int col = hh * M + f - row * M + c;
          const int ent = 64 * (col >> 4) + 16 * gg + (col & 15);
          const __bf16 hi = static_cast<__bf16>(pv[k][c]);
          const __bf16 lo = static_cast<__bf16>(pv[k][c] - static_cast<float>(hi));
          reinterpret_cast<__bf16*>(&phi_l[ln][i][0][ent])[e] = hi;
          reinterpret_cast<__bf16*>(&phi_l[ln][i][1][ent])[e] = lo;
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
  for (int q = tid; q < OSLOTS * OR * W; q += NTHR)
    tring[(q / (OR * W)) * a.slotw + static_cast<int64_t>(s) * OR * W + q % (OR * W)] = 0ull;
  for (int q = tid; q < OSLOTS * OTPR * N; q += NTHR) {
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

    // Tile jt's partials over this wave's 64 positions into the LDS ring, one
    // row per (token, half line): row 8 h + k is token 8 (w / 4) + k over
    // positions 32 h .. 32 h + 31 of the line.  Output column q of a block
    // is valid in the rows of the half that operand column q belongs to
    // (rows 0..7 for q < m, 8..15 for q >= m); the other half's entries
    // there are discarded.
    // Sum of squares: with A = B = the tile, the MFMA's diagonal entry
    // (rho, rho) is row rho's sum of squares; bf16 products are exact in
    // fp32, the accumulation over the 4 streams' 128 values is fp32, the sums
    // across rows, waves and members fp64.  Entry (rho, rho) sits in lane
    // 16 (rho / 4) + rho, element rho % 4.
    auto partials = [&](int jt, const u32x4 (&x)[N]) {
      f32x4 gram = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      // phi operands come from LDS.  The plain form keeps three (stream,
      // block) operands in flight ahead of the MFMAs, so the LDS latency is
      // met once per tile rather than once per stream (7 us less at
      // T = 16384, n = 4, d = 4096); the fused form has no registers for
      // that and reads each stream's operands next to its MFMAs.
      auto read_phi = [&](int q, PhiOp<BF16>& o) {
        const int i = q / NB, nb = q % NB;
        o.hi = __builtin_bit_cast(bf16x8, phi_l[L][i][0][64 * nb + lane]);
        o.lo = __builtin_bit_cast(bf16x8, phi_l[L][i][1][64 * nb + lane]);
      };
      if constexpr (!POST) {
        constexpr int QN = N * NB;
        constexpr int DP = QN < 3 ? QN : 3;
        PhiOp<BF16> bq[DP];
#pragma unroll
        for (int q = 0; q < DP; ++q) read_phi(q, bq[q]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < QN; ++q) {
          const int i = q / NB, nb = q % NB;
          if (nb == 0) {
            const bf16x8 xv = __builtin_bit_cast(bf16x8, x[i]);
            gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
          }
          acc[nb] = mfma_block(Raw8<BF16>{x[i]}, bq[q % DP], acc[nb]);
          if (q + DP < QN) read_phi(q + DP, bq[q % DP]);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const bf16x8 xv = __builtin_bit_cast(bf16x8, x[i]);
          gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, xv, gram, 0, 0, 0);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            PhiOp<BF16> b;
            read_phi(i * NB + nb, b);
            acc[nb] = mfma_block(Raw8<BF16>{x[i]}, b, acc[nb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int dv = r16 & 3;
      const float sqf = dv == 0 ? gram[0] : dv == 1 ? gram[1] : dv == 2 ? gram[2] : gram[3];
      double sq = static_cast<double>(sqf);
      const bool ovf = g == (r16 >> 2) && !__builtin_isfinite(sqf);
      if (__any(ovf)) {
        // fp32 overflow (|x| beyond ~1e18): the row's sum again in fp64
        // from the 4 lanes that hold its positions (lane 16 q + rho holds
        // row rho's 8 positions of K group q).  Wave-uniform branch: every
        // lane takes part in the permutes.
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
      const int slot = jt % ORR;   // free: see the static_assert on ORR
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int q = 16 * nb + r16;              // rows 4 g .. 4 g + 3 lie in half g / 2
        const int col = q - (g >> 1) * M;
        if (col >= 0 && col < M) {
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
      // Token tok's rows: row 8 h + tok % 8 of waves 4 (tok / 8) .. + 3, added
      // in position order (block 2 L + h for line L, half h).
      const int t8 = tok & 7, wb = 4 * (tok >> 3);
      if (qv) {
        if (2 * p == SSO) {
          double sd = red_ss[rs][wb][t8];
          sd += red_ss[rs][wb][8 + t8];
#pragma unroll
          for (int l4 = 1; l4 < 4; ++l4) {
            sd += red_ss[rs][wb + l4][t8];
            sd += red_ss[rs][wb + l4][8 + t8];
          }
          const u64 b = __builtin_bit_cast(u64, sd);
          v0 = static_cast<uint32_t>(b);
          v1 = static_cast<uint32_t>(b >> 32);
        } else {
          // columns 2p and 2p + 1: one 8-byte read per row
          const float2* r2 = reinterpret_cast<const float2*>(&red[rs][wb][t8][0]) + p;
          constexpr int WS = OR * MP * 2;                 // float2 stride between waves
          constexpr int HS = 8 * MP * 2;                  // and between the two halves of a line
          float2 x = r2[0];
          {
            const float2 y = r2[HS];
            x.x += y.x;
            x.y += y.y;
          }
#pragma unroll
          for (int l4 = 1; l4 < 4; ++l4) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const float2 y = r2[l4 * WS + hf * HS];
              x.x += y.x;
              x.y += y.y;
            }
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
        for (int i = 0; i < N; ++i) hp[i] = maps[jt % OMR][tk][i];
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
      const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + tk;
      const bool ok = have && t < T && jv;
      const uint32_t ho = ok ? static_cast<uint32_t>((t * d + j0) * 2) : kOob;
      // A plain store (whole lines; with half lines from two waves the L2 had
      // to merge them, which non-temporal stores defeated).
      __builtin_amdgcn_raw_buffer_store_b128(pack8(o, BF16{}).v, hr, static_cast<int>(ho), 0, 0);
    };

    // The previous layer's mhc_post of tile jt, in place: X_l in x becomes
    // X_{l+1} = H_res X_l + H_post Y_l with mhc_post's arithmetic and
    // rounding, which is stored and from here on is the tile.  Its N stores
    // are issued whether or not the tile exists (then out of range).
    const __amdgpu_buffer_rsrc_t xor_ = __builtin_amdgcn_make_buffer_rsrc(POST ? a.Xo : a.h, 0,
                                                                          POST ? a.xbytes : a.hbytes, 0x00020000);
    auto mix = [&](int jt, u32x4 (&x)[N], const u32x4& y) {
      const bool have = jt < J;
      const int sl = jt % OHR;
      if (have) wait_ge(&hmix_tag[sl], jt + 1, vbroken);
      // (a tile past the end mixes whatever the slot holds; its stores are
      // out of range and it is never used)
      const float* hm = &hmix[sl][tk][0];
      post_mix<N, true>(x, y, [&](int i, int j) { return j < N ? hm[i * N + j] : hm[N * N + i]; });
      const int64_t t = (team + static_cast<int64_t>(jt) * teams) * OR + tk;
      const bool ok = have && t < T && jv;
      const uint32_t o0 = ok ? static_cast<uint32_t>((t * N * d + j0) * 2) : kOob;
      const uint32_t st = ok ? static_cast<uint32_t>(d * 2) : 0u;
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(x[i], xor_, static_cast<int>(o0 + i * st), 0, 0);   // plain: as h's
    };

    // Tile k lives in buffer k % ONB; the buffer of tile k - OD, emitted in
    // step k, then receives tile k + OP.  Every step issues N loads and two
    // stores (with the post fused in: N + 1 loads and N + 2 stores), with no
    // branch around any of them.
    const int kend = ((J + OD + ONB - 1) / ONB) * ONB;
    for (int k0 = 0; k0 < kend; k0 += ONB) {
#pragma unroll
      for (int u = 0; u < ONB; ++u) {
        const int k = k0 + u;
        if constexpr (POST) {
          mix(k, xb[u], yb);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (k < J) partials(k, xb[u]);
        emit(k - OD, xb[(u + OP) % ONB]);
        if constexpr (POST) yb = load_y(k + 1);
        load_tile(k + OP, xb[(u + OP) % ONB]);
        __builtin_amdgcn_sched_barrier(0);
        post_share(k);
      }
    }
  } else if (wave < OW + OX) {
    // ---------------------------------------------------------------- exchange
    // Exchange wave x takes the tiles t with t % OX == x.  Meet the team
    // first: every member's slots are clear once its start word holds this
    // call's sequence number.
    __builtin_amdgcn_s_setprio(2);
    const int xw = wave - OW;
    const u64 tag = call_tag(a);
    u64* st = a.start + static_cast<int64_t>(team) * OS_MAX;
    if (lane == 0 && xw == 0) st[s] = tag;
    if (lane < S) {
      unsigned n = 0;
      while (agent_load(st + lane) != tag) {
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
    if (flag_get(vbroken) && lane == 0)
      __hip_atomic_store(a.hdr, tag ^ kErrFlip, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (wave == OW + OX) {
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
  } else if constexpr (POST) {
    // ------------------------------------------------- previous layer's maps
    // Tile j's H_res and H_post rows into LDS slot j % OHR, once every
    // streaming wave has mixed tile j - OHR (its partials of that tile are
    // written after the mix).  Tokens past T read as 0.
    constexpr int HW = OR * HF;
    for (int j = 0; j < J; ++j) {
      const int sl = j % OHR;
      if (j >= OHR && !wait_all_ge(part_ready, j - OHR + 1, vbroken, lane)) break;
      float v[(HW + 63) / 64];
#pragma unroll
      for (int k = 0; k < (HW + 63) / 64; ++k) {
        const int q = lane + 64 * k;
        const int tok = q / HF;
        const int64_t t = (team + static_cast<int64_t>(j) * teams) * OR + tok;
        v[k] = (q < HW && t < T) ? a.Hp[t * M + N + (q - tok * HF)] : 0.0f;
      }
#pragma unroll
      for (int k = 0; k < (HW + 63) / 64; ++k) {
        const int q = lane + 64 * k;
        if (q < HW) hmix[sl][q / HF][q % HF] = v[k];
      }
      lds_done();
      if (lane == 0) flag_set(&hmix_tag[sl], j + 1);
    }
  }
}

// The single pass's fallback, and the bookkeeping that follows every call.
// Workgroup 0 advances the header's sequence number (the next call's tag)
// and clears the start words.  Every workgroup then compares the error word
// with the current call's tag and returns unless a wait of the single pass ran
// out; if one did, the workgroups take whole 16-token tiles and recompute h
// and H with the single pass's arithmetic in its order:
//  - member slice s, wave w: positions 256 s + 32 w .. +31, the same MFMA
//    sequence (per stream: the Gram diagonal, then phi hi and lo per
//    16-column block) on the same operands (phi split into bf16 halves the
//    same way), the same fp64 redo of an overflowing sum of squares;
//  - the member's record: the 8 waves' partials added in wave order (fp32;
//    the sum of squares in fp64);
//  - the team's sums: the same fixed tree over 16 lanes (member = lane % 16,
//    members past S add 0) in fp64;
//  - logits, gates, Sinkhorn and h = H_pre . X by the same functions;
//  - with the previous layer's post fused in, X_{l+1} by the same mix,
//    stored, and read back for h.
// No exchange, so nothing here waits for another workgroup.
template <int N, bool HC, bool POST>
__global__ __launch_bounds__(OW * 64) void pre_one_pass_fallback_kernel(OneArgs a) {
  constexpr int M = num_maps(N);
  constexpr int NB = (M + 15) / 16;
  constexpr int NN = N * N;
  constexpr int NWD = M + 1;                 // team sums per token: m projections, then the sum of squares
  constexpr int NTH = OW * 64;
  __shared__ float fred[OW][OR][M];
  __shared__ double fred_ss[OW][OR];
  __shared__ float mrec[OS_MAX][OR][M];
  __shared__ double mss[OS_MAX][OR];
  __shared__ double team[OR][NWD];
  __shared__ float fmaps[OR][N];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const u64 err = agent_load(a.hdr);
  const u64 cur = agent_load(a.hdr + 2);
  if (blockIdx.x == 0) {
    if (tid == 0) {
      const u64 next = ((agent_load(a.hdr + 1) & ~kTagBit) + 1) & ~kTagBit;
      __hip_atomic_store(a.hdr + 1, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int q = tid; q < a.nstart; q += NTH) a.start[q] = 0ull;
  }
  if (err != (cur ^ kErrFlip)) return;

  const int S = a.S;
  const int d = a.d;
  const int64_t T = a.T;
  for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int64_t t = tile * OR + r16;
    const bool tv = t < T;
    for (int s = 0; s < S; ++s) {
      const int j0 = s * OSLICE + 32 * w + 8 * g;
      const bool jv = j0 < d;
      u32x4 x[N];
#pragma unroll
      for (int i = 0; i < N; ++i)
        x[i] = (tv && jv) ? *reinterpret_cast<const u32x4*>(a.X + (t * N + i) * d + j0) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (POST) {
        float res[N][N], post[N];
        const float* Hr = a.Hp + (tv ? t : 0) * M;
#pragma unroll
        for (int i = 0; i < N; ++i) {
#pragma unroll
          for (int j = 0; j < N; ++j) res[i][j] = tv ? Hr[N + i * N + j] : 0.0f;
          post[i] = tv ? Hr[N + NN + i] : 0.0f;
        }
        const u32x4 y = (tv && jv) ? *reinterpret_cast<const u32x4*>(a.Y + t * d + j0) : u32x4{0u, 0u, 0u, 0u};
        post_mix<N, false>(x, y, [&](int i, int j) { return j < N ? res[i][j] : post[i]; });
        if (tv && jv) {
#pragma unroll
          for (int i = 0; i < N; ++i) *reinterpret_cast<u32x4*>(a.Xo + (t * N + i) * d + j0) = x[i];
        }
      }
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
          const int col = 16 * nb + r16 % cn;
          float f[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) f[e] = jv ? a.phi[static_cast<int64_t>(i * d + j0 + e) * M + col] : 0.0f;
          acc[nb] = mfma_block(Raw8<BF16>{x[i]}, make_phi_op(f, BF16{}), acc[nb]);
        }
      }
      const int dv = r16 & 3;
      const float sqf = dv == 0 ? gram[0] : dv == 1 ? gram[1] : dv == 2 ? gram[2] : gram[3];
      double sq = static_cast<double>(sqf);
      const bool ovf = g == (r16 >> 2) && !__builtin_isfinite(sqf);
      if (__any(ovf)) {
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
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int col = 16 * nb + r16;
        if (col < M) {
#pragma unroll
          for (int v = 0; v < 4; ++v) fred[w][4 * g + v][col] = acc[nb][v];
        }
      }
      if (g == (r16 >> 2)) fred_ss[w][r16] = sq;
      __syncthreads();
      for (int q = tid; q < OR * M; q += NTH) {
        const int tok = q / M;
        const int c = q - tok * M;
        float v = fred[0][tok][c];
#pragma unroll
        for (int ww = 1; ww < OW; ++ww) v += fred[ww][tok][c];
        mrec[s][tok][c] = v;
      }
      if (tid < OR) {
        double sd = fred_ss[0][tid];
#pragma unroll
        for (int ww = 1; ww < OW; ++ww) sd += fred_ss[ww][tid];
        mss[s][tid] = sd;
      }
      __syncthreads();
    }
    // The team's sums: one (token, word) per 16-lane row.
    for (int base = 4 * w; base < OR * NWD; base += 4 * OW) {
      const int pi = base + (lane >> 4);
      const int rm = lane & 15;
      const bool pv = pi < OR * NWD;
      const int tok = pv ? pi / NWD : 0;
      const int wd = pv ? pi - tok * NWD : 0;
      double v = 0.0;
      if (pv && rm < S) v = wd < M ? static_cast<double>(mrec[rm][tok][wd]) : mss[rm][tok];
      v = row16_sum(v);
      if (pv && rm == 0) team[tok][wd] = v;
    }
    __syncthreads();
    // Maps: 16 lanes per token, four tokens per wave.
    if (w < OR / 4) {
      const int tok = 4 * w + (lane >> 4);
      const int e = lane & 15;
      const int colr = N + e;
      const int colg = (e < N) ? e : (N + NN + (e - N));
      const int cr = e < NN ? colr : 0, cg = e < 2 * N ? colg : 0;
      const float bias_r = a.bias[cr], bias_g = a.bias[cg];
      const float alpha_g = (e < N) ? a.a_pre : a.a_post;
      const double inv_r = inv_rms(team[tok][M], N * d, a.eps);
      const double zr = team[tok][cr];
      const double zg = team[tok][cg];
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
      float mv = rv;
      if constexpr (!HC) mv = sinkhorn16<N>(e < NN ? rv : -INFINITY, e, a.t_max);
      const int64_t tt = tile * OR + tok;
      if (tt < T) {
        float* Ht = a.H + tt * M;
        if (e < NN) Ht[N + e] = mv;
        if (e < 2 * N) Ht[colg] = gv;
      }
      if (e < N) fmaps[tok][e] = gv;
    }
    __syncthreads();
    // h = H_pre . X, from a second read of the tile.
    float hp[N];
#pragma unroll
    for (int i = 0; i < N; ++i) hp[i] = fmaps[r16][i];
    for (int s = 0; s < S; ++s) {
      const int j0 = s * OSLICE + 32 * w + 8 * g;
      if (!tv || j0 >= d) continue;
      const uint16_t* Xs = POST ? a.Xo : a.X;   // the pass's state: X_{l+1} as stored above
      u32x4 x[N];
#pragma unroll
      for (int i = 0; i < N; ++i) x[i] = *reinterpret_cast<const u32x4*>(Xs + (t * N + i) * d + j0);
      float o[8];
      {
        float v[8];
        unpack8(Raw8<BF16>{x[0]}, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = hp[0] * v[e];
      }
#pragma unroll
      for (int i = 1; i < N; ++i) {
        float v[8];
        unpack8(Raw8<BF16>{x[i]}, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(hp[i], v[e], o[e]);
      }
      *reinterpret_cast<u32x4*>(a.h + t * d + j0) = pack8(o, BF16{}).v;
    }
    __syncthreads();   // the next tile reuses the LDS arrays
  }
}

int one_pass_slices(int d) { return (d + OSLICE - 1) / OSLICE; }

// Token record: m partials, padding to an even word, the fp64 sum of squares.
int record_words(int n) { return ((num_maps(n) + 1) & ~1) + 2; }
int64_t slot_words(int S, int n) { return static_cast<int64_t>(S) * OR * record_words(n) + OR * n; }

int max_teams(int S) { return OXCD * (48 / S); }   // devices with up to 48 CUs per XCD

template <int N, bool HC, bool POST>
void one_pass_kernels(const void** fn, const void** fb) {
  *fn = reinterpret_cast<const void*>(&pre_one_pass_kernel<N, HC, POST>);
  *fb = reinterpret_cast<const void*>(&pre_one_pass_fallback_kernel<N, HC, POST>);
}

}  // namespace

// Body bytes the single-pass form needs after the header: start words and
// the exchange ring, for devices with up to 48 CUs per XCD.
size_t pre_fused_body_bytes(int n, int d) {
  const int S = one_pass_slices(d);
  if (n > 4 || S < OS_MIN || S > OS_MAX) return 0;
  const int teams = max_teams(S);
  return static_cast<size_t>(teams) * OS_MAX * sizeof(u64) +
         static_cast<size_t>(teams) * OSLOTS * static_cast<size_t>(slot_words(S, n)) * sizeof(u64);
}

// Whether MHC_PRE_AUTO takes the single pass: for n = 4 when the teams fill
// whole XCDs and each gets at least min_tiles tiles.  Measured on MI355X
// (single pass against two-pass form): mhc_pre 27.1 against 32.3 us at 6
// tiles per team (T = 1536, d = 4096) and 27.6 against 32.5 us (T = 3072,
// d = 2048), even at 4; mhc_post_pre 74.6 against 84.1 us at 16 tiles
// (T = 4096, d = 4096) and 76.7 against 90.5 us (T = 8192, d = 2048), even
// or slower at 8-12.  For n <= 2 a tile carries too little data to hide the
// exchange.
bool pre_fused_preferred(const mhc_params& p, const DeviceInfo& dev, bool post) {
  if (p.dtype != MHC_BF16 || p.n != 4 || dev.num_cus % OXCD != 0) return false;
  const int S = one_pass_slices(p.d);
  const int per_xcd = dev.num_cus / OXCD;
  if (S < OS_MIN || S > OS_MAX || per_xcd < S) return false;
  static_assert(OS_MAX - OS_MIN + 1 == 9, "one threshold per team size");
  const int min_tiles = post ? kAutoTilesPostPre[S - OS_MIN] : kAutoTilesPre[S - OS_MIN];
  const int64_t teams = static_cast<int64_t>(OXCD) * (per_xcd / S);
  return (p.T + OR - 1) / OR >= static_cast<int64_t>(min_tiles) * teams;
}

namespace {

// Launch the single-pass form (with the previous layer's post in front when
// Y is not null) and its fallback kernel when it applies; returns
// hipErrorNotSupported (without launching anything) when it does not, so
// the caller can take the two-pass form.
hipError_t launch_one_pass(const mhc_params& p, const void* X, const void* Y, const float* Hp, void* Xo,
                           const float* phi, const float* bias, void* h, float* H, void* workspace, size_t ws_bytes,
                           bool force_fallback, const DeviceInfo& dev, hipStream_t stream) {
  if (p.dtype != MHC_BF16 || (p.n != 4 && p.n != 2 && p.n != 1)) return hipErrorNotSupported;
  const bool post = Y != nullptr;
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
  if (OHDR + pre_fused_body_bytes(p.n, p.d) > ws_bytes) return hipErrorNotSupported;
  const bool hc = p.maps == MHC_MAPS_HC;
  const void* fn = nullptr;
  const void* fb = nullptr;
  if (post) {
    switch (p.n) {
      case 1: hc ? one_pass_kernels<1, true, true>(&fn, &fb) : one_pass_kernels<1, false, true>(&fn, &fb); break;
      case 2: hc ? one_pass_kernels<2, true, true>(&fn, &fb) : one_pass_kernels<2, false, true>(&fn, &fb); break;
      default: hc ? one_pass_kernels<4, true, true>(&fn, &fb) : one_pass_kernels<4, false, true>(&fn, &fb); break;
    }
  } else {
    switch (p.n) {
      case 1: hc ? one_pass_kernels<1, true, false>(&fn, &fb) : one_pass_kernels<1, false, false>(&fn, &fb); break;
      case 2: hc ? one_pass_kernels<2, true, false>(&fn, &fb) : one_pass_kernels<2, false, false>(&fn, &fb); break;
      default: hc ? one_pass_kernels<4, true, false>(&fn, &fb) : one_pass_kernels<4, false, false>(&fn, &fb); break;
    }
  }
  const int threads = post ? OTP : OT;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, threads, 0) != hipSuccess || occ < 1)
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
  a.nstart = max_teams(S) * OS_MAX;
  a.ring = a.start + a.nstart;
  a.slotw = slot_words(S, p.n);
  a.xbytes = static_cast<int>(xbytes);
  a.hbytes = static_cast<int>(hbytes);
  a.force_break = force_fallback ? 1 : 0;
  a.Y = static_cast<const uint16_t*>(Y);
  a.Hp = Hp;
  a.Xo = static_cast<uint16_t*>(Xo);
  void* args[] = {&a};
  hipError_t e = hipLaunchKernel(fn, dim3(dev.num_cus), dim3(threads), args, 0, stream);
  if (e != hipSuccess) return e;
  // Always launched: it advances the sequence number, and recomputes the
  // call only if a wait of the single pass ran out.
  return hipLaunchKernel(fb, dim3(dev.num_cus), dim3(OW * 64), args, 0, stream);
}

}  // namespace

hipError_t launch_pre_fused(const mhc_params& p, const void* X, const float* phi, const float* bias, void* h,
                            float* H, void* workspace, size_t ws_bytes, bool force_fallback, const DeviceInfo& dev,
                            hipStream_t stream) {
  return launch_one_pass(p, X, nullptr, nullptr, nullptr, phi, bias, h, H, workspace, ws_bytes, force_fallback, dev,
                         stream);
}

// The previous layer's mhc_post fused in front of the single pass: X is X_l,
// Xo receives X_{l+1} (Xo must not overlap X: the fallback recomputes from
// X_l).
hipError_t launch_post_pre_fused(const mhc_params& p, const void* X, const void* Y, const float* Hp, void* Xo,
                                 const float* phi, const float* bias, void* h, float* H, void* workspace,
                                 size_t ws_bytes, bool force_fallback, const DeviceInfo& dev, hipStream_t stream) {
  if (!Y || !Hp || !Xo) return hipErrorInvalidValue;
  return launch_one_pass(p, X, Y, Hp, Xo, phi, bias, h, H, workspace, ws_bytes, force_fallback, dev, stream);
}

}  // namespace mhc
