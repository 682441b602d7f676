// synth_fill.hip -- bulk GPU fills of the seeded synthetic inputs.
//
// The numbers at each position are defined in synth/__init__.py (SplitMix64
// counter hash, Box-Muller normal draw in fp32 with fixed polynomials and
// operation order, one fp32 multiply by sigma, then the round-to-nearest-even
// conversion of the storage type).  This file is a third implementation of
// that definition, for the GPU; it holds none of the ZeRO step's arithmetic.
// Built with -ffp-contract=off: one rounding per operation, and HIP's
// correctly rounded fp32 division and square root.  Tests check it bit for bit
// against the numpy one.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kMix2 = 0x94D049BB133111EBull;
constexpr uint32_t kZeroCut = 42949672u;     // floor(0.01 * 2^32)
constexpr uint32_t kOutlierCut = 4294967u;   // floor(0.001 * 2^32)

// fp32 roundings of (-1)^j/(2j)!, (-1)^j/(2j+1)!, 1/(2j+1).
__constant__ const float kCos[8] = {0x1.0p+0f, -0x1.0p-1f, 0x1.555556p-5f, -0x1.6c16c2p-10f, 0x1.a01a02p-16f,
                                    -0x1.27e4fcp-22f, 0x1.1eed8ep-29f, -0x1.93974ap-37f};
__constant__ const float kSin[8] = {0x1.0p+0f, -0x1.555556p-3f, 0x1.111112p-7f, -0x1.a01a02p-13f,
                                    0x1.71de3ap-19f, -0x1.ae6456p-26f, 0x1.612462p-33f, -0x1.ae7f3ep-41f};
__constant__ const float kLog[7] = {0x1.0p+0f, 0x1.555556p-2f, 0x1.99999ap-3f, 0x1.24924ap-3f, 0x1.c71c72p-4f,
                                    0x1.745d18p-4f, 0x1.3b13b2p-4f};
constexpr float kLn2 = 0x1.62e43p-1f;
constexpr float kSqrt2 = 0x1.6a09e6p+0f;
constexpr float kQStep = 0x1.921fb6p-22f;   // fp32(pi) * 2^-23

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

template <int N>
__device__ __forceinline__ float horner(const float* c, float x2) {
  float p = c[N - 1];
#pragma unroll
  for (int j = N - 2; j >= 0; --j) p = c[j] + x2 * p;
  return p;
}

// Box-Muller unit normal of the hash u (operation order as in the definition).
__device__ __forceinline__ float unit_normal(uint64_t u) {
  const uint32_t a1 = (uint32_t)(u >> 40) + 1u;      // 1 .. 2^24
  int e = 31 - __clz((int)a1);                       // a1 = m' 2^e, m' in [1, 2)
  float m = ldexpf((float)a1, -e);                   // exact
  e -= 24;                                           // u1 = a1 2^-24 = m 2^e
  if (m >= kSqrt2) {
    m = m * 0.5f;
    e += 1;
  }
  const float s = (m - 1.0f) / (m + 1.0f);
  const float s2 = s * s;
  const float t = s * horner<7>(kLog, s2);
  const float ln_u1 = (float)e * kLn2 + (t + t);
  const float r = __builtin_sqrtf(ln_u1 * -2.0f);
  const uint32_t k = (uint32_t)(u & 0xFFFFFFFFu) >> 8;
  const uint32_t h = k >> 22;
  const float x = (float)(k & 0x3FFFFFu) * kQStep;
  const float x2 = x * x;
  const float cx = horner<8>(kCos, x2);
  const float sx = x * horner<8>(kSin, x2);
  return r * (h == 0 ? cx : h == 1 ? -sx : h == 2 ? -cx : sx);
}

__device__ __forceinline__ float value_at(uint64_t key, uint64_t sel_key, int mix,
                                          uint64_t pos, float scale) {
  float x = unit_normal(mix64(key + (pos + 1) * kGamma)) * scale;
  if (mix) {
    uint64_t w = mix64(sel_key + (pos + 1) * kGamma);
    uint32_t hi = (uint32_t)(w >> 32);
    if (hi < kZeroCut) x = 0.0f;
    else if (hi < kZeroCut + kOutlierCut) x = (w & 1) ? -100.0f : 100.0f;
  }
  return x;
}

// NT: store with non-temporal stores (streaming, as a receive of incoming
// data would) instead of ordinary cached stores; the values are the same.
template <int DT, bool NT>
__global__ void __launch_bounds__(256) fill_kernel(void* __restrict__ out, int64_t n, uint64_t key,
                                                   uint64_t sel_key, int mix, int64_t pos_base,
                                                   float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float x = value_at(key, sel_key, mix, (uint64_t)(pos_base + i), scale);
    if constexpr (DT == 0) {
      if constexpr (NT) __builtin_nontemporal_store(x, (float*)out + i);
      else ((float*)out)[i] = x;
    } else {
      uint16_t h;
      if constexpr (DT == 1) h = __builtin_bit_cast(uint16_t, __float2half_rn(x));
      else h = __builtin_bit_cast(uint16_t, (__bf16)x);
      if constexpr (NT) __builtin_nontemporal_store(h, (uint16_t*)out + i);
      else ((uint16_t*)out)[i] = h;
    }
  }
}

template <bool NT>
void launch_fill(int dt, int64_t blocks, hipStream_t st, void* out, int64_t n, uint64_t key, uint64_t sel_key,
                 int mix, int64_t pos_base, float scale) {
  if (dt == 0)
    hipLaunchKernelGGL((fill_kernel<0, NT>), dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
  else if (dt == 1)
    hipLaunchKernelGGL((fill_kernel<1, NT>), dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
  else
    hipLaunchKernelGGL((fill_kernel<2, NT>), dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
}

}  // namespace

// out: device buffer of n elements of dtype dt (0 f32, 1 f16, 2 bf16); nt != 0
// stores with non-temporal stores.  Returns 0 on success, a HIP error code
// otherwise.
extern "C" int synth_fill(void* out, int dt, int64_t n, uint64_t key, uint64_t sel_key, int mix,
                          int64_t pos_base, float scale, int nt, void* stream) {
  if (n <= 0) return 0;
  if (!out || dt < 0 || dt > 2) return (int)hipErrorInvalidValue;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = (hipStream_t)stream;
  if (nt) launch_fill<true>(dt, blocks, st, out, n, key, sel_key, mix, pos_base, scale);
  else launch_fill<false>(dt, blocks, st, out, n, key, sel_key, mix, pos_base, scale);
  return (int)hipGetLastError();
}
