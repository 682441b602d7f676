/* synth_cpu.c -- host implementation of the seeded input definition in
 * synth/__init__.py: SplitMix64 counter hash, Box-Muller normal draw in fp32
 * (own logarithm and cosine polynomials, fixed operation order), one fp32
 * multiply by sigma, optional zero/outlier mix.  It produces fp32 values
 * only; conversion to a 16-bit storage type stays with numpy / torch.  Holds
 * none of the ZeRO step's arithmetic.  Built with gcc -O2 -fopenmp
 * -ffp-contract=off (one rounding per operation, as the definition needs). */
#include <math.h>
#include <stdint.h>

static const uint64_t kGamma = 0x9E3779B97F4A7C15ull;
static const uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
static const uint64_t kMix2 = 0x94D049BB133111EBull;
static const uint32_t kZeroCut = 42949672u;     /* floor(0.01 * 2^32) */
static const uint32_t kOutlierCut = 4294967u;   /* floor(0.001 * 2^32) */

/* fp32 roundings of (-1)^j/(2j)!, (-1)^j/(2j+1)!, 1/(2j+1). */
static const float kCos[8] = {0x1.0p+0f, -0x1.0p-1f, 0x1.555556p-5f, -0x1.6c16c2p-10f, 0x1.a01a02p-16f,
                              -0x1.27e4fcp-22f, 0x1.1eed8ep-29f, -0x1.93974ap-37f};
static const float kSin[8] = {0x1.0p+0f, -0x1.555556p-3f, 0x1.111112p-7f, -0x1.a01a02p-13f, 0x1.71de3ap-19f,
                              -0x1.ae6456p-26f, 0x1.612462p-33f, -0x1.ae7f3ep-41f};
static const float kLog[7] = {0x1.0p+0f, 0x1.555556p-2f, 0x1.99999ap-3f, 0x1.24924ap-3f, 0x1.c71c72p-4f,
                              0x1.745d18p-4f, 0x1.3b13b2p-4f};
static const float kLn2 = 0x1.62e43p-1f;
static const float kSqrt2 = 0x1.6a09e6p+0f;
static const float kQStep = 0x1.921fb6p-22f;   /* fp32(pi) * 2^-23 */

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

static inline float horner(const float* c, int n, float x2) {
  float p = c[n - 1];
  for (int j = n - 2; j >= 0; --j) p = c[j] + x2 * p;
  return p;
}

/* Box-Muller unit normal of the hash u (operation order as in the
 * definition). */
static inline float unit_normal(uint64_t u) {
  const uint32_t a1 = (uint32_t)(u >> 40) + 1u;          /* 1 .. 2^24 */
  int e = 31 - __builtin_clz(a1);                          /* a1 = m' 2^e, m' in [1, 2) */
  float m = ldexpf((float)a1, -e);                         /* exact */
  e -= 24;                                                 /* u1 = a1 2^-24 = m 2^e */
  if (m >= kSqrt2) {
    m = m * 0.5f;
    e += 1;
  }
  const float s = (m - 1.0f) / (m + 1.0f);
  const float s2 = s * s;
  const float t = s * horner(kLog, 7, s2);
  const float ln_u1 = (float)e * kLn2 + (t + t);
  const float r = sqrtf(ln_u1 * -2.0f);
  const uint32_t k = (uint32_t)(u & 0xFFFFFFFFu) >> 8;
  const uint32_t h = k >> 22;
  const float x = (float)(k & 0x3FFFFFu) * kQStep;
  const float x2 = x * x;
  const float cx = horner(kCos, 8, x2);
  const float sx = x * horner(kSin, 8, x2);
  const float c = h == 0 ? cx : h == 1 ? -sx : h == 2 ? -cx : sx;
  return r * c;
}

/* out[i] = value at position (positions ? positions[i] : pos_base + i). */
void synth_values_f32(float* out, int64_t n, uint64_t key, uint64_t sel_key, int mix,
                      const int64_t* positions, int64_t pos_base, float scale) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t pos = (uint64_t)(positions ? positions[i] : pos_base + i);
    float x = unit_normal(mix64(key + (pos + 1) * kGamma)) * scale;
    if (mix) {
      const uint64_t w = mix64(sel_key + (pos + 1) * kGamma);
      const uint32_t hi = (uint32_t)(w >> 32);
      if (hi < kZeroCut) x = 0.0f;
      else if (hi < kZeroCut + kOutlierCut) x = (w & 1) ? -100.0f : 100.0f;
    }
    out[i] = x;
  }
}
