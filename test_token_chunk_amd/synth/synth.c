/*
 * Seeded synthetic inputs shared by the HIP path and the oracle.
 *
 * This file holds no arithmetic of the TTT method: it only turns seeds into
 * arrays (model weights drawn from N(0, std), token ids drawn uniformly or
 * from a Zipf law).  The same arrays are handed to both sides.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used in its counter form: the i-th output
 * of the stream keyed by K is mix(K + (i + 1) * GOLDEN).  A stream key is the
 * stream id-th output of the generator seeded with the user seed, so every
 * tensor and every batch row has an independent, randomly addressable stream.
 *
 * Normals: Box-Muller in fp64 on consecutive uniform pairs.
 * bf16 rounding: round-to-nearest-even of the fp32 value (IEEE bit pattern).
 * Zipf(s) over ranks 1..V: inverse CDF on an fp64 table, id = rank - 1.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* i-th output (0-based) of SplitMix64 seeded with `key`. */
uint64_t synth_splitmix64_at(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GOLDEN); }

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return synth_splitmix64_at(seed, stream); }

/* uniform double in [0, 1) with 53 random bits */
static inline double u01(uint64_t x) { return (double)(x >> 11) * (1.0 / 9007199254740992.0); }

static inline float round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  u &= 0xFFFF0000u;
  float r;
  memcpy(&r, &u, 4);
  return r;
}

void synth_uniform(uint64_t seed, uint64_t stream, double* out, int64_t n) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = u01(synth_splitmix64_at(key, (uint64_t)i));
}

/* out[i] ~ N(0, std^2); if round_bf16_flag, each value is rounded (RNE) to bf16. */
void synth_normal(uint64_t seed, uint64_t stream, double std, int round_bf16_flag, float* out, int64_t n) {
  uint64_t key = synth_stream_key(seed, stream);
  int64_t pairs = (n + 1) / 2;
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < pairs; ++j) {
    double u1 = u01(synth_splitmix64_at(key, (uint64_t)(2 * j)));
    double u2 = u01(synth_splitmix64_at(key, (uint64_t)(2 * j + 1)));
    double r = sqrt(-2.0 * log(1.0 - u1));
    double z0 = r * cos(two_pi * u2) * std, z1 = r * sin(two_pi * u2) * std;
    float f0 = (float)z0, f1 = (float)z1;
    if (round_bf16_flag) { f0 = round_bf16(f0); f1 = round_bf16(f1); }
    out[2 * j] = f0;
    if (2 * j + 1 < n) out[2 * j + 1] = f1;
  }
}

void synth_tokens_uniform(uint64_t seed, uint64_t stream, int32_t vocab, int32_t* out, int64_t n) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    int64_t id = (int64_t)(u01(synth_splitmix64_at(key, (uint64_t)i)) * (double)vocab);
    if (id >= vocab) id = vocab - 1;
    out[i] = (int32_t)id;
  }
}

/* Zipf(s): P(rank r) proportional to r^-s for r = 1..vocab; id = r - 1. */
int synth_tokens_zipf(uint64_t seed, uint64_t stream, int32_t vocab, double s, int32_t* out, int64_t n) {
  double* cdf = (double*)malloc(sizeof(double) * (size_t)vocab);
  if (!cdf) return -1;
  double acc = 0.0;
  for (int32_t r = 0; r < vocab; ++r) { acc += pow((double)(r + 1), -s); cdf[r] = acc; }
  for (int32_t r = 0; r < vocab; ++r) cdf[r] /= acc;
  cdf[vocab - 1] = 1.0;
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double u = u01(synth_splitmix64_at(key, (uint64_t)i));
    int32_t lo = 0, hi = vocab - 1; /* smallest r with cdf[r] > u */
    while (lo < hi) {
      int32_t mid = lo + (hi - lo) / 2;
      if (cdf[mid] > u) hi = mid; else lo = mid + 1;
    }
    out[i] = lo;
  }
  free(cdf);
  return 0;
}
