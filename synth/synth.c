/*
 * Seeded synthetic inputs shared by the oracle tests and the GPU path.
 *
 * This file holds no arithmetic of the draft head: it only turns
 * (seed, tensor id, element index) into numbers.  Both sides of every
 * parity check receive the very same bits from here.
 *
 * Definition (counter based, so any element can be drawn on its own):
 *   mix(z)  = SplitMix64 output finaliser (Steele, Lea, Flood, "Fast
 *             splittable pseudorandom number generators", OOPSLA 2014)
 *   key     = mix(seed) ^ mix(tensor_id + 1)
 *   u64(i)  = mix(key + (i + 1) * 0x9E3779B97F4A7C15)
 *   U(i)    = (u64(i) >> 11) * 2^-53                      in [0, 1)
 *   normal element i (Box-Muller, cosine branch, one value per pair):
 *           sqrt(-2 ln(1 - U(2i))) * cos(2 pi U(2i+1)) * std
 *           rounded to fp32 (round to nearest even), and for bf16
 *           tensors rounded once more, fp32 -> bf16 to nearest even.
 *   uniform integer element i in [0, n): floor(u64(i) * n / 2^64).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline uint64_t key_of(uint64_t seed, uint64_t tensor_id) {
  return mix64(seed) ^ mix64(tensor_id + 1);
}

static inline double unit_of(uint64_t u) {
  return (double)(u >> 11) * (1.0 / 9007199254740992.0);
}

static inline float normal_at(uint64_t key, uint64_t i, double std) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = 1.0 - unit_of(draw(key, 2 * i));
  double u2 = unit_of(draw(key, 2 * i + 1));
  return (float)(sqrt(-2.0 * log(u1)) * cos(two_pi * u2) * std);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7FFFu + lsb;
  return (uint16_t)(x >> 16);
}

void synth_raw_u64(uint64_t seed, uint64_t tensor_id, uint64_t n, uint64_t *out) {
  uint64_t key = key_of(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = draw(key, (uint64_t)i);
}

void synth_normal_f32(uint64_t seed, uint64_t tensor_id, uint64_t n, double std, float *out) {
  uint64_t key = key_of(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = normal_at(key, (uint64_t)i, std);
}

void synth_normal_bf16(uint64_t seed, uint64_t tensor_id, uint64_t n, double std, uint16_t *out) {
  uint64_t key = key_of(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) out[i] = f32_to_bf16_rne(normal_at(key, (uint64_t)i, std));
}

void synth_uniform_int(uint64_t seed, uint64_t tensor_id, uint64_t n, uint64_t bound, int32_t *out) {
  uint64_t key = key_of(seed, tensor_id);
  for (uint64_t i = 0; i < n; ++i) {
    unsigned __int128 p = (unsigned __int128)draw(key, i) * bound;
    out[i] = (int32_t)(uint64_t)(p >> 64);
  }
}
