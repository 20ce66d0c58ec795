/* Counter-based SplitMix64 words and Box-Muller normals (see synth/__init__.py).
 * Word i of (seed, stream) is mix64(key + (i + 1) * G), key = mix64(seed * P +
 * stream); normal element e uses words 2e and 2e + 1.  Threads split the index
 * range; every value depends only on its index. */
#include <math.h>
#include <stdint.h>

#define G 0x9E3779B97F4A7C15ull
#define P 0xD1B54A32D192ED03ull

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t key_of(uint64_t seed, uint64_t stream) { return mix64(seed * P + stream); }

void syn_words(uint64_t seed, uint64_t stream, int64_t start, int64_t count, uint64_t* out) {
  const uint64_t k = key_of(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = mix64(k + (uint64_t)(start + i + 1) * G);
}

void syn_normal(uint64_t seed, uint64_t stream, int64_t start, int64_t count, double sigma,
                double* out) {
  const uint64_t k = key_of(seed, stream);
  const double two_pi = 2.0 * M_PI;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    const uint64_t e = (uint64_t)(start + i);
    const uint64_t a = mix64(k + (2 * e + 1) * G);
    const uint64_t b = mix64(k + (2 * e + 2) * G);
    const double u1 = ((double)(a >> 11) + 0.5) * 0x1p-53;
    const double u2 = (double)(b >> 11) * 0x1p-53;
    const double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
    out[i] = z * sigma;
  }
}
