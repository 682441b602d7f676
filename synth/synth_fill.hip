// synth_fill.hip -- bulk GPU fills of the seeded synthetic inputs.
//
// The numbers at each position are defined in synth/__init__.py (SplitMix64
// counter hash, four-term Irwin-Hall integer, one fp32 multiply, then the
// round-to-nearest-even conversion of the storage type).  This file is a
// second implementation of that definition for the GPU; it holds none of the
// ZeRO step's arithmetic.  Tests check it bit for bit against the numpy one.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kMix1 = 0xBF58476D1CE4E5B9ull;
constexpr uint64_t kMix2 = 0x94D049BB133111EBull;
constexpr uint32_t kZeroCut = 42949672u;     // floor(0.01 * 2^32)
constexpr uint32_t kOutlierCut = 4294967u;   // floor(0.001 * 2^32)

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * kMix1;
  z = (z ^ (z >> 27)) * kMix2;
  return z ^ (z >> 31);
}

__device__ __forceinline__ float value_at(uint64_t key, uint64_t sel_key, int mix,
                                          uint64_t pos, float scale) {
  uint64_t u = mix64(key + (pos + 1) * kGamma);
  int64_t s = (int64_t)(u & 0xFFFF) + (int64_t)((u >> 16) & 0xFFFF) +
              (int64_t)((u >> 32) & 0xFFFF) + (int64_t)(u >> 48) - 131070;
  float x = (float)s * scale;
  if (mix) {
    uint64_t w = mix64(sel_key + (pos + 1) * kGamma);
    uint32_t hi = (uint32_t)(w >> 32);
    if (hi < kZeroCut) x = 0.0f;
    else if (hi < kZeroCut + kOutlierCut) x = (w & 1) ? -100.0f : 100.0f;
  }
  return x;
}

template <int DT>
__global__ void __launch_bounds__(256) fill_kernel(void* __restrict__ out, int64_t n, uint64_t key,
                                                   uint64_t sel_key, int mix, int64_t pos_base,
                                                   float scale) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    float x = value_at(key, sel_key, mix, (uint64_t)(pos_base + i), scale);
    if constexpr (DT == 0) {
      ((float*)out)[i] = x;
    } else if constexpr (DT == 1) {
      ((__half*)out)[i] = __float2half_rn(x);
    } else {
      __bf16 b = (__bf16)x;
      ((uint16_t*)out)[i] = __builtin_bit_cast(uint16_t, b);
    }
  }
}

}  // namespace

// out: device buffer of n elements of dtype dt (0 f32, 1 f16, 2 bf16).
// Returns 0 on success, a HIP error code otherwise.
extern "C" int synth_fill(void* out, int dt, int64_t n, uint64_t key, uint64_t sel_key, int mix,
                          int64_t pos_base, float scale, void* stream) {
  if (n <= 0) return 0;
  if (!out || dt < 0 || dt > 2) return (int)hipErrorInvalidValue;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t st = (hipStream_t)stream;
  if (dt == 0)
    hipLaunchKernelGGL(fill_kernel<0>, dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
  else if (dt == 1)
    hipLaunchKernelGGL(fill_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
  else
    hipLaunchKernelGGL(fill_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, st, out, n, key, sel_key, mix, pos_base, scale);
  return (int)hipGetLastError();
}
