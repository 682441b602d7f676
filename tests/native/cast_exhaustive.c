/* Exhaustive check of the oracle's fp32 -> fp16 / bf16 round-to-nearest-even
 * conversions over all 2^32 fp32 bit patterns, against references that share
 * nothing with the oracle's arithmetic formulation:
 *   fp16: the x86 F16C conversion instruction (vcvtps2ph, round to nearest even);
 *   bf16: integer rounding of the 16 dropped bits, half to even.
 * NaN inputs must map to a NaN of the same sign.
 * Usage: cast_exhaustive f16|bf16 ; exit status 0 when every pattern agrees. */
#include <immintrin.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t orc_f32_to_f16(float x);
uint16_t orc_f32_to_bf16(float x);

static uint16_t ref_f16(float x) { return (uint16_t)_cvtss_sh(x, _MM_FROUND_TO_NEAREST_INT); }

static uint16_t ref_bf16(uint32_t b) {
  uint32_t lsb = (b >> 16) & 1u;
  return (uint16_t)((b + 0x7fffu + lsb) >> 16);
}

static int is_nan16(uint16_t h, int bf) {
  return bf ? ((h & 0x7f80u) == 0x7f80u && (h & 0x7fu)) : ((h & 0x7c00u) == 0x7c00u && (h & 0x3ffu));
}

int main(int argc, char** argv) {
  int bf = argc > 1 && strcmp(argv[1], "bf16") == 0;
  if (!bf && !__builtin_cpu_supports("f16c")) { printf("SKIP no f16c\n"); return 2; }
  unsigned long long bad = 0;
  uint32_t first_bad = 0;
  #pragma omp parallel for schedule(static) reduction(+:bad)
  for (long long i = 0; i < (1LL << 32); ++i) {
    uint32_t b = (uint32_t)i;
    float x;
    memcpy(&x, &b, 4);
    uint16_t got = bf ? orc_f32_to_bf16(x) : orc_f32_to_f16(x);
    int ok;
    if (x != x) {
      ok = is_nan16(got, bf) && ((got >> 15) == (b >> 31));
    } else {
      uint16_t want = bf ? ref_bf16(b) : ref_f16(x);
      ok = got == want;
    }
    if (!ok) {
      if (bad == 0) first_bad = b;
      bad++;
    }
  }
  printf("%s mismatches=%llu first=0x%08x\n", bf ? "bf16" : "f16", bad, first_bad);
  return bad ? 1 : 0;
}
