/*
 * Seeded synthetic inputs for the decode step: weights, prompt tokens,
 * synthetic KV contents, page-table permutations and sequence lengths.
 *
 * This file holds no arithmetic of the decode method itself.  It only turns
 * (seed, tensor id, element index) into numbers, so that the CPU oracle and
 * the GPU path can be fed identical inputs without either one producing them
 * for the other.  numpy mirror: synth/__init__.py (bit-identical, tested).
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014) used in counter mode.  Element i of stream
 * (seed, tid) is the (i+1)-th SplitMix64 output of state key(seed, tid):
 *     word(i) = mix64(key + (i + 1) * GOLDEN)
 *     key     = mix64(mix64(seed + GOLDEN) ^ (tid * TID_MUL))
 *
 * Normal deviates: Irwin-Hall sum of the four 16-bit fields of word(i),
 *     s = u0 + u1 + u2 + u3 - 131070          (exact integer, |s| < 2^18)
 *     v = bf16_rne( f32(s) * f32(sigma / SD) ),  SD = sqrt((65536^2 - 1) / 3)
 * one fp32 multiply and one bf16 rounding, so every implementation that
 * follows these lines gets the same bits.
 *
 * Gains near one: v = bf16_rne( 1.0f + f32(s) * f32(sigma / SD) ).
 * Uniform integers in [0, n): Lemire multiply-shift on the high 32 bits.
 * Permutations: Fisher-Yates, swap partner for position i drawn from word(i).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYNTH_GOLDEN 0x9E3779B97F4A7C15ULL
#define SYNTH_TID_MUL 0xD1B54A32D192ED03ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t tid) {
  return mix64(mix64(seed + SYNTH_GOLDEN) ^ (tid * SYNTH_TID_MUL));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * SYNTH_GOLDEN);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0; /* NaN */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline int32_t irwin_hall(uint64_t w) {
  return (int32_t)(w & 0xFFFF) + (int32_t)((w >> 16) & 0xFFFF) +
         (int32_t)((w >> 32) & 0xFFFF) + (int32_t)((w >> 48) & 0xFFFF) - 131070;
}

float synth_normal_scale(double sigma) {
  const double sd = sqrt((65536.0 * 65536.0 - 1.0) / 3.0);
  return (float)(sigma / sd);
}

/* out[j] = bf16 bits of N(0, sigma^2) deviate at element start + j. */
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count,
                       double sigma, uint16_t* out) {
  const uint64_t key = synth_key(seed, tid);
  const float c = synth_normal_scale(sigma);
  int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static) if (n > 262144)
  for (int64_t j = 0; j < n; ++j) {
    float s = (float)irwin_hall(word_at(key, start + (uint64_t)j));
    out[j] = f32_to_bf16_rne(s * c);
  }
}

/* out[j] = bf16 bits of 1 + N(0, sigma^2) at element start + j. */
void synth_gain_bf16(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count,
                     double sigma, uint16_t* out) {
  const uint64_t key = synth_key(seed, tid);
  const float c = synth_normal_scale(sigma);
  int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static) if (n > 262144)
  for (int64_t j = 0; j < n; ++j) {
    float s = (float)irwin_hall(word_at(key, start + (uint64_t)j));
    float t = s * c;
    out[j] = f32_to_bf16_rne(1.0f + t);
  }
}

/* out[j] = uniform integer in [0, n) at element start + j (n < 2^32). */
void synth_uniform_u32(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count,
                       uint32_t n, uint32_t* out) {
  const uint64_t key = synth_key(seed, tid);
  int64_t m = (int64_t)count;
#pragma omp parallel for schedule(static) if (m > 262144)
  for (int64_t j = 0; j < m; ++j) {
    uint64_t w = word_at(key, start + (uint64_t)j);
    out[j] = (uint32_t)(((w >> 32) * (uint64_t)n) >> 32);
  }
}

/* Fisher-Yates permutation of 0..n-1 (n < 2^31). */
void synth_permutation(uint64_t seed, uint64_t tid, uint32_t n, int32_t* out) {
  const uint64_t key = synth_key(seed, tid);
  for (uint32_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (uint32_t i = n; i-- > 1;) {
    uint64_t w = word_at(key, i);
    uint32_t j = (uint32_t)(((w >> 32) * (uint64_t)(i + 1)) >> 32);
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}
