// Device pieces shared by the two forms of mhc_pre: the phi MFMA operands,
// the projection block, the per-token logits and the Sinkhorn-Knopp
// iteration on 16 lanes.
#pragma once

#include "device.hpp"

namespace mhc {

__host__ __device__ constexpr int num_maps(int n) { return n * n + 2 * n; }

// Per-token record of one slice of d in a split-K workspace: m fp32 partial
// dot products (then, for the backward, n more: <D, X_i> over the slice),
// then the partial sum of squares as an fp64 at an 8-byte aligned float offset.
__host__ __device__ constexpr int ss_offset(int n, bool with_d = false) {
  return (num_maps(n) + (with_d ? n : 0) + 1) & ~1;
}
__host__ __device__ constexpr int part_width(int n, bool with_d = false) { return ss_offset(n, with_d) + 2; }

// MFMA B operand for one (stream, 16-column block): 8 rows of phi per lane.
// bf16 state: phi = hi + lo, two bf16 halves (~16 significant bits); fp32
// state: phi itself for the fp32 MFMA.
template <typename ST> struct PhiOp;
template <> struct PhiOp<BF16> { bf16x8 hi, lo; };
template <> struct PhiOp<F32> { float v[8]; };

__device__ __forceinline__ PhiOp<BF16> make_phi_op(const float (&f)[8], BF16) {
  PhiOp<BF16> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 hi = static_cast<__bf16>(f[e]);
    o.hi[e] = hi;
    o.lo[e] = static_cast<__bf16>(f[e] - static_cast<float>(hi));
  }
  return o;
}
__device__ __forceinline__ PhiOp<F32> make_phi_op(const float (&f)[8], F32) {
  PhiOp<F32> o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o.v[e] = f[e];
  return o;
}

// acc += A . B for one 16 (tokens) x 32 (positions) x 16 (columns) block.
// A row = lane % 16 (token), positions 8 (lane / 16) .. +7 held by the lane;
// B column = lane % 16, same positions.  Output: lane holds rows
// 4 (lane / 16) .. +3 of column lane % 16.
__device__ __forceinline__ f32x4 mfma_block(const Raw8<BF16>& a, const PhiOp<BF16>& b, f32x4 acc) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a.v);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b.hi, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b.lo, acc, 0, 0, 0);
  return acc;
}
// acc += A . A^T for a 16 (tokens) x 32 (positions) bf16 block in the A
// layout above: entry (t, t) is token t's sum of squares over the block.
__device__ __forceinline__ f32x4 mfma_block_gram(const Raw8<BF16>& a, f32x4 acc) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a.v);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, av, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_block(const Raw8<F32>& a, const PhiOp<F32>& b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[e], b.v[e], acc, 0, 0, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[e], b.v[4 + e], acc, 0, 0, 0);
  return acc;
}

// 1 / r with r = sqrt(sum x^2 / K + eps), in fp64.
__device__ __forceinline__ double inv_rms(double ss, int K, float eps) {
  return 1.0 / sqrt(ss / static_cast<double>(K) + static_cast<double>(eps));
}

// logit = alpha * (z / r) + bias, formed in fp64 and rounded once to fp32.
__device__ __forceinline__ float logit_of(double z, double inv_r, float alpha, float bias) {
  return static_cast<float>(static_cast<double>(alpha) * (z * inv_r) + static_cast<double>(bias));
}

// Lane exchanges inside 16-lane rows without the LDS unit (DPP): quad
// permutes for partners e^1 and e^2, row rotations for partners at +-4 and 8
// (lanes e and e^8 are 8 apart either way).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp<0xB1>(v); }    // quad_perm [1,0,3,2]
__device__ __forceinline__ float lane_xor2(float v) { return dpp<0x4E>(v); }    // quad_perm [2,3,0,1]
__device__ __forceinline__ float lane_rot8(float v) { return dpp<0x128>(v); }   // row_ror:8 = partner e^8
__device__ __forceinline__ float lane_rot4(float v) { return dpp<0x124>(v); }   // row_ror:4

// Sum over the lanes of a Sinkhorn line, the same value on every lane of
// the line.  Rows (fixed i, j varies: the low lane bits): (v + v^1) + its ^2
// partner.  Columns (fixed j, i varies: the lane bits above log2 n): for
// n = 4, p = v + v^8 pairs rows i and i+2, then p + rot4(p) adds the other
// pair; every lane of the column adds the same two addends, so all hold the
// same bits whichever way the rotation runs.  For n = 2 a column is lanes
// {e, e^2}.
template <int N>
__device__ __forceinline__ float row_sum(float v) {
  if constexpr (N == 1) {
    return v;
  } else if constexpr (N == 2) {
    return v + lane_xor1(v);
  } else {
    const float q = v + lane_xor1(v);
    return q + lane_xor2(q);
  }
}
template <int N>
__device__ __forceinline__ float col_sum(float v) {
  if constexpr (N == 1) {
    return v;
  } else if constexpr (N == 2) {
    return v + lane_xor2(v);
  } else {
    const float p = v + lane_rot8(v);
    return p + lane_rot4(p);
  }
}

// Sinkhorn-Knopp on one token's n x n map held by 16 lanes: lane e (e = lane
// % 16) owns entry (e / n, e % n) for e < n*n and receives the residual logit
// `lr` (-inf on lanes e >= n*n).  Returns the entry of H_res after t_max
// passes of (normalise columns, then rows).  Every lane of the wave must
// call it (n = 1, 2, 4).
template <int N>
__device__ __forceinline__ float sinkhorn16(float lr, int e, int t_max) {
  static_assert(N == 1 || N == 2 || N == 4, "16-lane Sinkhorn covers n <= 4");
  constexpr int NN = N * N;
  // Subtracting the token's largest residual logit leaves every iterate
  // unchanged (the first column step divides it out) and keeps exp finite;
  // with no pass at all the map is exp(logits) itself.
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
  float mv = (e < NN) ? expf(lr - mx) : 0.0f;
  for (int it = 0; it < t_max; ++it) {
    mv = mv / col_sum<N>(mv);
    mv = mv / row_sum<N>(mv);
  }
  return mv;
}

}  // namespace mhc
