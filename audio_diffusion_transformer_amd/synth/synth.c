/*
 * Seeded, counter-based synthetic input generator.
 *
 * This file holds no arithmetic of the DiT forward: it only turns
 * (seed, stream, element index) into numbers.  Both the CPU oracle and the
 * GPU path consume the bytes it writes, so the two sides see identical inputs.
 *
 * Definition (published SplitMix64, Steele/Lea/Flood 2014):
 *   mix(z)   = z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *              z *= 0x94D049BB133111EB; z ^= z>>31
 *   key      = mix(seed + GAMMA) ^ mix(stream + 2*GAMMA)
 *   raw(i)   = mix(key + (i+1)*GAMMA)       (the i-th SplitMix64 output from key)
 *   U(i)     = ((raw(i) >> 11) + 0.5) * 2^-53          in (0, 1)
 *   N(2p)    = sqrt(-2 ln U(2p)) * cos(2 pi U(2p+1))    (Box-Muller)
 *   N(2p+1)  = sqrt(-2 ln U(2p)) * sin(2 pi U(2p+1))
 * Values are formed in double, then rounded to float (RNE); bf16 outputs are
 * the float rounded to bf16 (RNE, NaN kept quiet).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z ^= z >> 30; z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27; z *= 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return mix64(seed + GAMMA) ^ mix64(stream + 2 * GAMMA);
}

static inline double unit(uint64_t key, uint64_t i) {
  uint64_t r = mix64(key + (i + 1) * GAMMA);
  return ((double)(r >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t i) {
  uint64_t p = i >> 1;
  double u1 = unit(key, 2 * p), u2 = unit(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double a = 6.283185307179586476925286766559 * u2;
  return (i & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u; memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

void synth_uniform_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                       double* out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = unit(key, start + (uint64_t)j);
}

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                      double* out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = normal_at(key, start + (uint64_t)j);
}

/* mean + std * N(i), rounded to bf16 bits.  Works pair by pair so that each
 * Box-Muller pair is formed once; the values equal normal_at(key, i). */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                       double mean, double std, uint16_t* out) {
  uint64_t key = synth_key(seed, stream);
  int64_t first_pair = (int64_t)(start >> 1);
  int64_t last_pair = (int64_t)((start + (uint64_t)n + 1) >> 1);
#pragma omp parallel for schedule(static)
  for (int64_t p = first_pair; p < last_pair; ++p) {
    double u1 = unit(key, 2 * (uint64_t)p), u2 = unit(key, 2 * (uint64_t)p + 1);
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    double v[2] = {r * cos(a), r * sin(a)};
    for (int e = 0; e < 2; ++e) {
      int64_t j = 2 * p + e - (int64_t)start;
      if (j >= 0 && j < n) out[j] = f32_to_bf16_rne((float)(mean + std * v[e]));
    }
  }
}

/* lo + (hi - lo) * U(i), rounded to float. */
void synth_uniform_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n,
                       double lo, double hi, float* out) {
  uint64_t key = synth_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j)
    out[j] = (float)(lo + (hi - lo) * unit(key, start + (uint64_t)j));
}

/* float -> bf16 bits, RNE: used to store derived inputs (e.g. correlated fields). */
void synth_f32_to_bf16(const float* in, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = f32_to_bf16_rne(in[j]);
}
