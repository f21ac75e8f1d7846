// Device-side helpers of libmhc for gfx950: storage chunks of 8 state values,
// bf16 conversions and the MFMA operand types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mhc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tags: the state (X, h, Y, X') is fp32 or bf16.  bf16 values travel
// as their 16-bit patterns.
struct F32 { typedef float elem; static constexpr int bytes = 4; };
struct BF16 { typedef uint16_t elem; static constexpr int bytes = 2; };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Round two floats to bf16 (nearest, ties to even; v_cvt_pk_bf16_f32) and pack
// them as lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
  const uint32_t b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
  return a | (b << 16);
}

__device__ __forceinline__ float round_to_bf16(float f) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f))) << 16);
}

// Raw storage of one chunk of 8 consecutive state values.
template <typename ST> struct Raw8;
template <> struct Raw8<BF16> { u32x4 v; };
template <> struct Raw8<F32> { f32x4 a, b; };

template <typename ST, bool NT = false>
__device__ __forceinline__ Raw8<ST> load_raw8(const typename ST::elem* p);

template <>
__device__ __forceinline__ Raw8<BF16> load_raw8<BF16, false>(const uint16_t* p) {
  return Raw8<BF16>{*reinterpret_cast<const u32x4*>(p)};
}
template <>
__device__ __forceinline__ Raw8<BF16> load_raw8<BF16, true>(const uint16_t* p) {
  return Raw8<BF16>{__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))};
}
template <>
__device__ __forceinline__ Raw8<F32> load_raw8<F32, false>(const float* p) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
  return Raw8<F32>{q[0], q[1]};
}
template <>
__device__ __forceinline__ Raw8<F32> load_raw8<F32, true>(const float* p) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p);
  return Raw8<F32>{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1)};
}

template <typename ST> __device__ __forceinline__ Raw8<ST> zero_raw8();
template <> __device__ __forceinline__ Raw8<BF16> zero_raw8<BF16>() { return Raw8<BF16>{u32x4{0, 0, 0, 0}}; }
template <> __device__ __forceinline__ Raw8<F32> zero_raw8<F32>() { return Raw8<F32>{f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}}; }

__device__ __forceinline__ void unpack8(const Raw8<BF16>& r, float (&x)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[2 * q] = bf16_lo(r.v[q]);
    x[2 * q + 1] = bf16_hi(r.v[q]);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<F32>& r, float (&x)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    x[q] = r.a[q];
    x[4 + q] = r.b[q];
  }
}

// Round 8 values to the storage form (bf16: nearest, ties to even) and store it.
__device__ __forceinline__ Raw8<BF16> pack8(const float (&x)[8], BF16) {
  return Raw8<BF16>{u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])}};
}
__device__ __forceinline__ Raw8<F32> pack8(const float (&x)[8], F32) {
  return Raw8<F32>{f32x4{x[0], x[1], x[2], x[3]}, f32x4{x[4], x[5], x[6], x[7]}};
}
template <bool NT>
__device__ __forceinline__ void store_raw8(uint16_t* p, const Raw8<BF16>& r) {
  if (NT) __builtin_nontemporal_store(r.v, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = r.v;
}
template <bool NT>
__device__ __forceinline__ void store_raw8(float* p, const Raw8<F32>& r) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
  if (NT) {
    __builtin_nontemporal_store(r.a, q);
    __builtin_nontemporal_store(r.b, q + 1);
  } else {
    q[0] = r.a;
    q[1] = r.b;
  }
}

template <typename ST, bool NT = false>
__device__ __forceinline__ void store8(typename ST::elem* p, const float (&x)[8]);

template <>
__device__ __forceinline__ void store8<BF16, false>(uint16_t* p, const float (&x)[8]) {
  u32x4 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
  *reinterpret_cast<u32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store8<BF16, true>(uint16_t* p, const float (&x)[8]) {
  u32x4 v = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
template <>
__device__ __forceinline__ void store8<F32, false>(float* p, const float (&x)[8]) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
  q[0] = f32x4{x[0], x[1], x[2], x[3]};
  q[1] = f32x4{x[4], x[5], x[6], x[7]};
}
template <>
__device__ __forceinline__ void store8<F32, true>(float* p, const float (&x)[8]) {
  f32x4* q = reinterpret_cast<f32x4*>(p);
  __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, q);
  __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, q + 1);
}

// Single state values (slow paths only).
template <typename ST> __device__ __forceinline__ float load_elem(const typename ST::elem* p, int64_t i);
template <> __device__ __forceinline__ float load_elem<F32>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<BF16>(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
template <typename ST> __device__ __forceinline__ void store_elem(typename ST::elem* p, int64_t i, float v);
template <> __device__ __forceinline__ void store_elem<F32>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_elem<BF16>(uint16_t* p, int64_t i, float v) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

__device__ __forceinline__ float sigmoidf_(float u) { return 1.0f / (1.0f + expf(-u)); }

}  // namespace mhc
