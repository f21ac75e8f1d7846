/*
 * Seeded synthetic input generator shared by the parity tests, the benchmark
 * and the oracle-side checks.  It holds none of the method's arithmetic: it
 * only turns (seed, tensor tag, element index) into a normal deviate and
 * stores it in the requested storage type.
 *
 * Counter-based construction, so any element can be produced on its own and
 * the result does not depend on how the work is split over threads:
 *   key      = splitmix64_mix(seed * 0x100000001B3 + tag)          (per tensor)
 *   bits(c)  = splitmix64_mix(key + (c + 1) * 0x9E3779B97F4A7C15)   (SplitMix64,
 *              Steele, Lea & Flood 2014; finaliser constants as published)
 *   u1       = ((bits(2i) >> 11) + 1) * 2^-53     in (0, 1]
 *   u2       =  (bits(2i+1) >> 11)    * 2^-53     in [0, 1)
 *   z_i      = sqrt(-2 ln u1) * cos(2 pi u2)      (Box & Muller 1958, one of the pair)
 *   value_i  = mean + std * z_i   (+ diag_add on the diagonal of n x n blocks)
 * fp32 storage rounds the double to nearest; bf16 storage rounds the fp32 value
 * to the nearest bf16 with ties to even.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static uint64_t tensor_key(uint64_t seed, uint64_t tag) {
  return mix64(seed * 0x100000001B3ULL + tag);
}

static double normal_at(uint64_t key, uint64_t i) {
  const uint64_t g = 0x9E3779B97F4A7C15ULL;
  uint64_t b1 = mix64(key + (2 * i + 1) * g);
  uint64_t b2 = mix64(key + (2 * i + 2) * g);
  double u1 = ((double)(b1 >> 11) + 1.0) * 0x1.0p-53;
  double u2 = (double)(b2 >> 11) * 0x1.0p-53;
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Fill out[0..count) with element indices [offset, offset+count) of tensor
 * (seed, tag).  dtype 0 = fp32, 1 = bf16 (uint16 bits), 2 = fp64.
 * diag_n > 0 adds diag_add to elements whose index within consecutive
 * diag_n*diag_n blocks lies on the block diagonal (used for b_res = 2I + noise).
 * threads > 1 splits the range over OpenMP threads (result is identical). */
void synth_normal(uint64_t seed, uint64_t tag, int64_t offset, int64_t count,
                  double mean, double std, int dtype, int diag_n, double diag_add,
                  void* out, int threads) {
  const uint64_t key = tensor_key(seed, tag);
#pragma omp parallel for schedule(static) num_threads(threads > 0 ? threads : 1) if (threads > 1)
  for (int64_t j = 0; j < count; ++j) {
    int64_t i = offset + j;
    double v = mean + std * normal_at(key, (uint64_t)i);
    if (diag_n > 0) {
      int64_t w = i % ((int64_t)diag_n * diag_n);
      if (w / diag_n == w % diag_n) v += diag_add;
    }
    if (dtype == 0) ((float*)out)[j] = (float)v;
    else if (dtype == 1) ((uint16_t*)out)[j] = f32_to_bf16_rne((float)v);
    else ((double*)out)[j] = v;
  }
}

int synth_version(void) { return 1; }
