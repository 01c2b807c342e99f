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
 *
 * FP8 weights (8-bit floating point, OCP E4M3: 1 sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, subnormals, no infinities, largest finite 448):
 *     code = e4m3_rne( f32(s) * f32(32 / SD) )   (the same s; |value| < 111)
 * the nearest code, ties to the even one.  Row scales:
 *     scale = f32(sigma / 32) * f32(bf16_rne(1 + f32(s') * f32(0.02 / SD)))
 * with s' from the scale stream of the tensor, so code * scale is a weight of
 * about the same spread as the bf16 recipe's.
 *
 * FP4 weights (OCP E2M1: 1 sign, 2 exponent bits with bias 1, 1 mantissa bit,
 * magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two codes a byte, element 2j in the
 * low nibble of byte j:
 *     code = e2m1_rne( f32(s) * f32(1.5 / SD) )   (|value| < 5.2: no saturation)
 * and row scales f32(sigma / 1.5) * (the same gain near one).
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

/* The E4M3 code nearest to f, ties to the even code; |f| >= 464 saturates to
 * the largest finite code (448).  Subnormal codes hold m * 2^-9, m = 1..7. */
static inline uint8_t f32_to_e4m3_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
  u &= 0x7FFFFFFFu;
  float a;
  memcpy(&a, &u, 4);
  uint8_t code;
  if (!(a < 464.0f)) {
    code = 0x7E;
  } else if (a < 0.015625f) {
    code = (uint8_t)nearbyintf(a * 512.0f); /* 0 .. 8; 8 is the smallest normal code */
  } else {
    u += 0x7FFFFu + ((u >> 20) & 1u); /* round the mantissa to 3 bits, ties to even */
    const int e = (int)(u >> 23) - 127;
    const uint32_t c = ((uint32_t)(e + 7) << 3) | ((u >> 20) & 7u);
    code = (uint8_t)(c > 0x7Eu ? 0x7Eu : c);
  }
  return (uint8_t)(sign | code);
}

uint8_t synth_e4m3_rne(float f) { return f32_to_e4m3_rne(f); }

/* out[j] = E4M3 code of the normal deviate at element start + j, spread 32. */
void synth_fp8_codes(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, uint8_t* out) {
  const uint64_t key = synth_key(seed, tid);
  const float c = synth_normal_scale(32.0);
  int64_t n = (int64_t)count;
#pragma omp parallel for schedule(static) if (n > 262144)
  for (int64_t j = 0; j < n; ++j) {
    float s = (float)irwin_hall(word_at(key, start + (uint64_t)j));
    out[j] = f32_to_e4m3_rne(s * c);
  }
}

/* out[j] = row scale start + j: f32(sigma / 32) * (a gain near one, as bf16). */
void synth_fp8_scales(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, double sigma,
                      double gain_sigma, float* out) {
  const uint64_t key = synth_key(seed, tid);
  const float c = synth_normal_scale(gain_sigma);
  const float base = (float)(sigma / 32.0);
  for (uint64_t j = 0; j < count; ++j) {
    float s = (float)irwin_hall(word_at(key, start + j));
    uint16_t g = f32_to_bf16_rne(1.0f + s * c);
    uint32_t gu = (uint32_t)g << 16;
    float gf;
    memcpy(&gf, &gu, 4);
    out[j] = base * gf;
  }
}

/* The E2M1 code nearest to f, ties to the even code (mantissa bit 0); |f| > 6
 * saturates to 6. */
static inline uint8_t f32_to_e2m1_rne(float f) {
  const uint8_t sign = f < 0.0f || (f == 0.0f && signbit(f)) ? 8 : 0;
  const float a = fabsf(f);
  uint8_t m;
  if (a <= 0.25f) m = 0;          /* 0 (tie at 0.25 -> 0) */
  else if (a < 0.75f) m = 1;      /* 0.5 */
  else if (a <= 1.25f) m = 2;     /* 1 (ties at 0.75 and 1.25 -> 1) */
  else if (a < 1.75f) m = 3;      /* 1.5 */
  else if (a <= 2.5f) m = 4;      /* 2 (ties at 1.75 and 2.5 -> 2) */
  else if (a < 3.5f) m = 5;       /* 3 */
  else if (a <= 5.0f) m = 6;      /* 4 (ties at 3.5 and 5 -> 4) */
  else m = 7;                     /* 6 */
  return (uint8_t)(sign | m);
}

uint8_t synth_e2m1_rne(float f) { return f32_to_e2m1_rne(f); }

/* Packed FP4 codes of elements start .. start + count - 1 (start, count even):
 * out[j] holds elements start + 2j (low nibble) and start + 2j + 1 (high). */
void synth_fp4_codes(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, uint8_t* out) {
  const uint64_t key = synth_key(seed, tid);
  const float c = synth_normal_scale(1.5);
  int64_t n = (int64_t)(count / 2);
#pragma omp parallel for schedule(static) if (n > 131072)
  for (int64_t j = 0; j < n; ++j) {
    const uint64_t e = start + 2 * (uint64_t)j;
    const uint8_t lo = f32_to_e2m1_rne((float)irwin_hall(word_at(key, e)) * c);
    const uint8_t hi = f32_to_e2m1_rne((float)irwin_hall(word_at(key, e + 1)) * c);
    out[j] = (uint8_t)(lo | (hi << 4));
  }
}

/* FP4 row scales: f32(sigma / 1.5) * (a gain near one, as bf16). */
void synth_fp4_scales(uint64_t seed, uint64_t tid, uint64_t start, uint64_t count, double sigma,
                      double gain_sigma, float* out) {
  synth_fp8_scales(seed, tid, start, count, sigma * 32.0 / 1.5, gain_sigma, out);
}
