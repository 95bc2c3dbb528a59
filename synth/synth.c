/*
 * Seeded synthetic inputs shared by the GPU path and the CPU oracle.
 *
 * This file holds random-number generation only: no step of the decoder is
 * computed here.  Every value is a pure function of (seed, tensor name,
 * element index), so a tensor can be regenerated in pieces, in any order and
 * by any number of threads, with identical bits.
 *
 *   key(seed, name) = mix64(seed * PHI + fnv1a64(name))
 *   bits(key, i)    = mix64(key ^ mix64(i + PHI))          (64 bits)
 *   normal          = Box-Muller on the two 32-bit halves (cosine branch),
 *                     in double, scaled by std, rounded to float, then to
 *                     bf16 with round-to-nearest-even where asked.
 *   uniform id      = (high 32 bits * vocab) >> 32.
 *
 * mix64 is the SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHI 0x9E3779B97F4A7C15ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t fnv1a64(const char* s) {
  uint64_t h = 0xcbf29ce484222325ull;
  for (; *s; ++s) {
    h ^= (uint8_t)*s;
    h *= 0x100000001b3ull;
  }
  return h;
}

uint64_t synth_key(uint64_t seed, const char* name) {
  return mix64(seed * PHI + fnv1a64(name));
}

static inline uint64_t bits_at(uint64_t key, uint64_t i) { return mix64(key ^ mix64(i + PHI)); }

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t b = bits_at(key, i);
  double u1 = ((double)(uint32_t)(b >> 32) + 0.5) * (1.0 / 4294967296.0);
  double u2 = ((double)(uint32_t)b + 0.5) * (1.0 / 4294967296.0);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925286766559 * u2);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Elements [start, start + n) of the tensor stream `key`, as bf16 bits. */
void synth_normal_bf16(uint64_t key, uint64_t start, uint64_t n, double mean, double std,
                       uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    float v = (float)(mean + std * normal_at(key, start + (uint64_t)j));
    out[j] = f32_to_bf16_rne(v);
  }
}

void synth_normal_f32(uint64_t key, uint64_t start, uint64_t n, double mean, double std,
                      float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < (int64_t)n; ++j)
    out[j] = (float)(mean + std * normal_at(key, start + (uint64_t)j));
}

void synth_uniform_ids(uint64_t key, uint64_t start, uint64_t n, uint32_t vocab, int32_t* out) {
  for (uint64_t j = 0; j < n; ++j) {
    uint64_t hi = bits_at(key, start + j) >> 32;
    out[j] = (int32_t)((hi * (uint64_t)vocab) >> 32);
  }
}

/* Integers uniform in [lo, hi] (inclusive), e.g. prompt lengths. */
void synth_uniform_int(uint64_t key, uint64_t start, uint64_t n, int32_t lo, int32_t hi,
                       int32_t* out) {
  uint64_t span = (uint64_t)(hi - lo + 1);
  for (uint64_t j = 0; j < n; ++j) {
    uint64_t h = bits_at(key, start + j) >> 32;
    out[j] = lo + (int32_t)((h * span) >> 32);
  }
}
