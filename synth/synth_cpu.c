/* synth_cpu.c -- host implementation of the seeded input definition in
 * synth/__init__.py (SplitMix64 counter hash, four-term Irwin-Hall integer,
 * one fp32 multiply, optional zero/outlier mix).  It produces fp32 values
 * only; conversion to a 16-bit storage type stays with numpy / torch.  Holds
 * none of the ZeRO step's arithmetic.  Built with gcc -O2 -fopenmp. */
#include <stdint.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;
static const uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
static const uint64_t kMix2 = 0x94D049BB133111EBull;
static const uint32_t kZeroCut = 42949672u;     /* floor(0.01 * 2^32) */
static const uint32_t kOutlierCut = 4294967u;   /* floor(0.001 * 2^32) */

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

/* out[i] = value at position (positions ? positions[i] : pos_base + i). */
void synth_values_f32(float* out, int64_t n, uint64_t key, uint64_t sel_key, int mix,
                      const int64_t* positions, int64_t pos_base, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t pos = (uint64_t)(positions ? positions[i] : pos_base + i);
    const uint64_t u = mix64(key + (pos + 1) * kGamma);
    const int64_t s = (int64_t)(u & 0xFFFF) + (int64_t)((u >> 16) & 0xFFFF) +
                      (int64_t)((u >> 32) & 0xFFFF) + (int64_t)(u >> 48) - 131070;
    float x = (float)s * scale;
    if (mix) {
      const uint64_t w = mix64(sel_key + (pos + 1) * kGamma);
      const uint32_t hi = (uint32_t)(w >> 32);
      if (hi < kZeroCut) x = 0.0f;
      else if (hi < kZeroCut + kOutlierCut) x = (w & 1) ? -100.0f : 100.0f;
    }
    out[i] = x;
  }
}
