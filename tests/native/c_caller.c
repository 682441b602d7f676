/*
 * A plain C caller of libzero.so: no Python and no PyTorch in the process, the
 * HIP runtime of /opt/rocm only.  It builds a plan, allocates device memory
 * with hipMalloc, runs the fused step (zero_adam_step with the N_d gradient
 * slices) for two steps and, separately, zero_shard_reduce followed by
 * zero_adam_step from the reduced gradient, and checks every result bit
 * against the CPU oracle's functions (liboracle.so: orc_reduce,
 * orc_adam_consts, orc_adam) on the same inputs.  Also checks an error path:
 * a bad rank returns ZERO_EINVAL with a message and launches nothing.
 *
 * Case: 100,003 parameters in three tensors, N_d = 4, bucket cap 60,000,
 * shard_align 8, owner rank 2, bf16 gradients, fp16 parameters, Stage 2
 * (parameters written into the full flat buffer at the owner's ranges).
 * Inputs come from a fixed xorshift generator; padding is zero.
 *
 * Prints "c_caller ok" and returns 0 on success; prints the first mismatch
 * and returns 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zero.h"

/* The oracle's C entry points (tests/ may use the oracle). */
void orc_reduce(int32_t n_ranks, const void* const* slices, int dt, int64_t count, float grad_scale,
                float* out);
void orc_adam_consts(double lr, double beta1, double beta2, double eps, double grad_scale, int64_t t,
                     float out[9]);
void orc_adam(int64_t count, const float* gr, float* w, float* m, float* v, const float c[9], uint16_t* p,
              int pdt);

#define CHECK_HIP(x)                                                             \
  do {                                                                           \
    hipError_t e_ = (x);                                                         \
    if (e_ != hipSuccess) {                                                      \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);      \
      return 1;                                                                  \
    }                                                                            \
  } while (0)
#define CHECK_Z(x)                                                               \
  do {                                                                           \
    zero_status s_ = (x);                                                        \
    if (s_ != ZERO_OK) {                                                         \
      printf("libzero error %d at line %d: %s\n", s_, __LINE__, zero_last_error()); \
      return 1;                                                                  \
    }                                                                            \
  } while (0)

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static uint32_t next_u32(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (uint32_t)(rng_state >> 16);
}
/* A bf16 pattern of magnitude about 1e-3 (exponent 2^-10 .. 2^-9), random sign. */
static uint16_t random_bf16(void) {
  uint32_t r = next_u32();
  return (uint16_t)(((r & 1u) << 15) | (117u << 7) | ((r >> 1) & 0x7fu));
}
/* An fp32 master weight of magnitude below about 0.03. */
static float random_w(void) {
  return ((float)(next_u32() & 0xffffff) / 16777216.0f - 0.5f) * 0.06f;
}

static int compare_u32(const char* what, const void* a, const void* b, int64_t n) {
  const uint32_t* x = (const uint32_t*)a;
  const uint32_t* y = (const uint32_t*)b;
  for (int64_t i = 0; i < n; ++i)
    if (x[i] != y[i]) {
      printf("%s differs at %lld: gpu 0x%08x oracle 0x%08x\n", what, (long long)i, x[i], y[i]);
      return 1;
    }
  return 0;
}

static int compare_u16(const char* what, const uint16_t* x, const uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (x[i] != y[i]) {
      printf("%s differs at %lld: gpu 0x%04x oracle 0x%04x\n", what, (long long)i, x[i], y[i]);
      return 1;
    }
  return 0;
}

int main(void) {
  const int64_t sizes[3] = {50001, 30000, 20002};
  const int64_t psi = sizes[0] + sizes[1] + sizes[2];
  const int32_t n_d = 4, owner = 2;
  const double lr = 1e-4, b1 = 0.9, b2 = 0.999, eps = 1e-8, gs = 1.0 / 4;

  zero_plan_t plan;
  CHECK_Z(zero_plan(psi, n_d, sizes, 3, 60000, 8, &plan));
  int64_t P, S;
  int32_t nb, nd;
  CHECK_Z(zero_plan_info(plan, &P, &S, &nb, &nd));

  /* Host inputs: n_d compact gradient slices (owner's partition), master. */
  uint16_t* g = (uint16_t*)calloc((size_t)(n_d * S), 2);
  float* w0 = (float*)calloc((size_t)S, 4);
  for (int32_t b = 0; b < nb; ++b) {
    int64_t flat_off, numel, padded, sn, soff;
    CHECK_Z(zero_plan_bucket(plan, b, &flat_off, &numel, &padded, &sn, &soff));
    for (int64_t i = 0; i < sn; ++i) {
      const int64_t pos = flat_off + owner * sn + i;   /* flat position of shard element */
      const int real = pos < flat_off + numel;
      for (int32_t q = 0; q < n_d; ++q) g[q * S + soff + i] = real ? random_bf16() : 0;
      w0[soff + i] = real ? random_w() : 0.0f;
    }
  }

  /* Device buffers. */
  void *dg, *dfull;
  float *dw, *dm, *dv, *dred;
  CHECK_HIP(hipMalloc(&dg, (size_t)(n_d * S) * 2));
  CHECK_HIP(hipMalloc((void**)&dw, (size_t)S * 4));
  CHECK_HIP(hipMalloc((void**)&dm, (size_t)S * 4));
  CHECK_HIP(hipMalloc((void**)&dv, (size_t)S * 4));
  CHECK_HIP(hipMalloc((void**)&dred, (size_t)S * 4));
  CHECK_HIP(hipMalloc(&dfull, (size_t)P * 2));
  CHECK_HIP(hipMemcpy(dg, g, (size_t)(n_d * S) * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dw, w0, (size_t)S * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(dm, 0, (size_t)S * 4));
  CHECK_HIP(hipMemset(dv, 0, (size_t)S * 4));
  CHECK_HIP(hipMemset(dfull, 0, (size_t)P * 2));

  const void* ptrs[4];
  for (int32_t q = 0; q < n_d; ++q) ptrs[q] = (const char*)dg + (size_t)(q * S) * 2;
  zero_grad_src src = {ZERO_BF16, n_d, ptrs, NULL};
  zero_adam_hyper hp = {lr, b1, b2, eps, gs};

  /* Oracle state. */
  float* w = (float*)malloc((size_t)S * 4);
  float* m = (float*)calloc((size_t)S, 4);
  float* v = (float*)calloc((size_t)S, 4);
  float* red = (float*)malloc((size_t)S * 4);
  uint16_t* p16 = (uint16_t*)malloc((size_t)S * 2);
  memcpy(w, w0, (size_t)S * 4);
  const void* hslices[4];
  for (int32_t q = 0; q < n_d; ++q) hslices[q] = g + q * S;

  /* Two fused steps. */
  for (int64_t t = 1; t <= 2; ++t) {
    CHECK_Z(zero_adam_step(plan, owner, &hp, t, &src, NULL, dw, dm, dv, dfull, ZERO_F16, 1, NULL));
    float c[9];
    orc_adam_consts(lr, b1, b2, eps, gs, t, c);
    orc_reduce(n_d, hslices, ZERO_BF16, S, (float)gs, red);
    orc_adam(S, red, w, m, v, c, p16, ZERO_F16);
  }
  /* Then the unfused pair for a third step. */
  CHECK_Z(zero_shard_reduce(plan, owner, &src, gs, dred, NULL));
  CHECK_Z(zero_adam_step(plan, owner, &hp, 3, NULL, dred, dw, dm, dv, dfull, ZERO_F16, 1, NULL));
  {
    float c[9];
    orc_adam_consts(lr, b1, b2, eps, gs, 3, c);
    orc_reduce(n_d, hslices, ZERO_BF16, S, (float)gs, red);
    orc_adam(S, red, w, m, v, c, p16, ZERO_F16);
  }
  CHECK_HIP(hipDeviceSynchronize());

  /* Error path: nothing launched, message set. */
  if (zero_adam_step(plan, n_d, &hp, 4, &src, NULL, dw, dm, dv, dfull, ZERO_F16, 1, NULL) != ZERO_EINVAL ||
      strstr(zero_last_error(), "rank") == NULL) {
    printf("bad rank not rejected\n");
    return 1;
  }

  /* Read back and compare. */
  float* gw = (float*)malloc((size_t)S * 4);
  float* gm = (float*)malloc((size_t)S * 4);
  float* gv = (float*)malloc((size_t)S * 4);
  float* gred = (float*)malloc((size_t)S * 4);
  uint16_t* gfull = (uint16_t*)malloc((size_t)P * 2);
  CHECK_HIP(hipMemcpy(gw, dw, (size_t)S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gm, dm, (size_t)S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gv, dv, (size_t)S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gred, dred, (size_t)S * 4, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gfull, dfull, (size_t)P * 2, hipMemcpyDeviceToHost));
  int bad = compare_u32("master", gw, w, S) || compare_u32("m", gm, m, S) || compare_u32("v", gv, v, S) ||
            compare_u32("reduced", gred, red, S);
  /* Parameters: the owner's ranges hold the rounded master, the rest stays 0. */
  for (int32_t b = 0; b < nb && !bad; ++b) {
    int64_t flat_off, numel, padded, sn, soff;
    CHECK_Z(zero_plan_bucket(plan, b, &flat_off, &numel, &padded, &sn, &soff));
    bad = compare_u16("params", gfull + flat_off + owner * sn, p16 + soff, sn);
    for (int64_t i = 0; i < padded && !bad; ++i) {
      const int owned = i >= owner * sn && i < (owner + 1) * sn;
      if (!owned && gfull[flat_off + i] != 0) {
        printf("non-owned parameter %lld written\n", (long long)(flat_off + i));
        bad = 1;
      }
    }
  }
  zero_plan_destroy(plan);
  hipFree(dg);
  hipFree(dw);
  hipFree(dm);
  hipFree(dv);
  hipFree(dred);
  hipFree(dfull);
  if (bad) return 1;
  printf("c_caller ok: psi=%lld n_d=%d owner=%d S=%lld buckets=%d, 3 steps bit-exact\n", (long long)psi, n_d,
         owner, (long long)S, nb);
  return 0;
}
