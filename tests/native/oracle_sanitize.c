/*
 * The CPU oracle's C functions under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point on edge inputs (zero counts,
 * one rank, 130 ranks, every 16-bit pattern through the decode, a strided
 * sweep of fp32 patterns through both encoders, NaN/Inf/denormal Adam
 * inputs).  Built with zero_oracle.c and run by tests/test_host_tables.py;
 * prints "oracle sanitize ok" and returns 0 when nothing trips.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double orc_f16_value(uint16_t h);
double orc_bf16_value(uint16_t h);
uint16_t orc_f32_to_f16(float x);
uint16_t orc_f32_to_bf16(float x);
void orc_cast_f32_to_16(const float* x, uint16_t* out, int64_t n, int dt);
void orc_cast_bits_range_to_16(uint32_t first, int64_t n, uint16_t* out, int dt);
void orc_adam_consts(double lr, double beta1, double beta2, double eps, double grad_scale, int64_t t,
                     float out[9]);
void orc_reduce(int32_t n_ranks, const void* const* slices, int dt, int64_t count, float grad_scale,
                float* out);
void orc_adam(int64_t count, const float* gr, float* w, float* m, float* v, const float c[9], uint16_t* p,
              int pdt);
void orc_adam_f64(int64_t count, const double* g, double* w, double* m, double* v, double lr, double beta1,
                  double beta2, double eps, int64_t t);
void orc_widen_to_f64(const void* src, int dt, int64_t count, double* out);
uint32_t orc_f32_bits(float x);
float orc_bits_f32(uint32_t b);

int main(void) {
  /* Decode every 16-bit pattern of both formats. */
  static uint16_t all16[65536];
  static double dec[65536];
  for (uint32_t h = 0; h < 65536; ++h) all16[h] = (uint16_t)h;
  for (int dt = 1; dt <= 2; ++dt) orc_widen_to_f64(all16, dt, 65536, dec);
  (void)orc_f16_value(0x7c01);
  (void)orc_bf16_value(0xff81);

  /* Encode a strided sweep of fp32 patterns (every 4099th) with both. */
  enum { N = 1 << 20 };
  uint16_t* out = (uint16_t*)malloc(N * sizeof *out);
  float* xs = (float*)malloc(N * sizeof *xs);
  for (uint32_t i = 0; i < N; ++i) xs[i] = orc_bits_f32(i * 4099u);
  orc_cast_f32_to_16(xs, out, N, 1);
  orc_cast_f32_to_16(xs, out, N, 2);
  orc_cast_bits_range_to_16(0x7f7fff00u, 512, out, 1);   /* across fp32 max into Inf/NaN */
  orc_cast_bits_range_to_16(0xff7fff00u, 512, out, 2);
  orc_cast_f32_to_16(xs, out, 0, 1);                     /* zero count */

  /* Reduce: 1 rank, 130 ranks, zero count. */
  enum { C = 1000, R = 130 };
  uint16_t* g = (uint16_t*)malloc((size_t)R * C * sizeof *g);
  for (int i = 0; i < R * C; ++i) g[i] = (uint16_t)(i * 2654435761u >> 16);
  const void* ptrs[R];
  for (int q = 0; q < R; ++q) ptrs[q] = g + (size_t)q * C;
  float* red = (float*)malloc(C * sizeof *red);
  orc_reduce(1, ptrs, 2, C, 1.0f, red);
  orc_reduce(R, ptrs, 1, C, 1.0f / 128, red);
  orc_reduce(R, ptrs, 2, 0, 1.0f, red);

  /* Adam on ordinary, zero, NaN, Inf and denormal inputs; both param types. */
  float c[9];
  orc_adam_consts(1e-4, 0.9, 0.999, 1e-8, 1.0, 1, c);
  orc_adam_consts(1e-4, 0.9, 0.999, 1e-8, 1.0, 1000000, c);
  float gr[8] = {1e-3f, 0.0f, -0.0f, NAN, INFINITY, -INFINITY, 1e-40f, -3.0f};
  float w[8], m[8], v[8];
  uint16_t p[8];
  for (int dt = 1; dt <= 2; ++dt) {
    for (int i = 0; i < 8; ++i) { w[i] = 0.01f * (float)i; m[i] = 0.0f; v[i] = 0.0f; }
    orc_adam(8, gr, w, m, v, c, p, dt);
    orc_adam(8, gr, w, m, v, c, NULL, dt);
    orc_adam(0, gr, w, m, v, c, p, dt);
  }
  orc_adam(C, red, (float*)calloc(C, 4), (float*)calloc(C, 4), (float*)calloc(C, 4), c,
           (uint16_t*)calloc(C, 2), 2);
  double g64[4] = {1e-3, 0.0, -1.0, 1e-300}, w64[4] = {0}, m64[4] = {0}, v64[4] = {0};
  orc_adam_f64(4, g64, w64, m64, v64, 1e-4, 0.9, 0.999, 1e-8, 3);
  (void)orc_f32_bits(w[0]);
  printf("oracle sanitize ok\n");
  return 0;
}
