// probes.hip -- HBM calibration probes for the benchmark: a plain read, a
// plain write and a plain copy of a large buffer, each in 16-byte
// non-temporal accesses, 8 per lane, so their bandwidth can be reported
// beside the step's.  No arithmetic of the ZeRO step; part of libsynth.so
// (bench and test support), not of libzero.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

constexpr int kThreads = 256;
constexpr int kUnits = 8;   // 16-byte units per lane

// Reads `units` 16-byte units; each workgroup stores one word (the xor of
// what its first lane read), so the loads cannot be dropped.
__global__ void __launch_bounds__(kThreads) probe_read(const u32x4* src, int64_t units, uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const int64_t u = base + (int64_t)i * kThreads;
    if (u < units) acc ^= __builtin_nontemporal_load((const gu32x4*)(src + u));
  }
  const uint32_t x = __builtin_amdgcn_readfirstlane(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

__global__ void __launch_bounds__(kThreads) probe_write(u32x4* dst, int64_t units, uint32_t value) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x;
  const u32x4 v = {value, value, value, value};
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const int64_t u = base + (int64_t)i * kThreads;
    if (u < units) __builtin_nontemporal_store(v, (gu32x4*)(dst + u));
  }
}

__global__ void __launch_bounds__(kThreads) probe_copy(u32x4* dst, const u32x4* src, int64_t units) {
  const int64_t base = (int64_t)blockIdx.x * kThreads * kUnits + threadIdx.x;
  u32x4 r[kUnits];
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const int64_t u = base + (int64_t)i * kThreads;
    if (u < units) r[i] = __builtin_nontemporal_load((const gu32x4*)(src + u));
  }
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const int64_t u = base + (int64_t)i * kThreads;
    if (u < units) __builtin_nontemporal_store(r[i], (gu32x4*)(dst + u));
  }
}

int64_t blocks_for(int64_t units) { return (units + kThreads * kUnits - 1) / (kThreads * kUnits); }

}  // namespace

// kind 0: read `bytes` at src (sink: one word per workgroup, see
// synth_probe_sink_words); 1: write `bytes` at dst; 2: copy `bytes` from src
// to dst.  bytes must be a multiple of 16 and pointers 16-byte aligned.
// Returns 0 or a HIP error code.
extern "C" int64_t synth_probe_sink_words(int64_t bytes) { return blocks_for(bytes / 16); }

extern "C" int synth_probe(int kind, void* dst, const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes <= 0) return 0;
  if ((bytes & 15) || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
  const int64_t units = bytes / 16;
  const int64_t blocks = blocks_for(units);
  if (blocks > INT32_MAX) return (int)hipErrorInvalidValue;
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0) {
    if (!src || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_read, dim3((unsigned)blocks), dim3(kThreads), 0, st, (const u32x4*)src, units, sink);
  } else if (kind == 1) {
    if (!dst) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_write, dim3((unsigned)blocks), dim3(kThreads), 0, st, (u32x4*)dst, units, 0x3c003c00u);
  } else if (kind == 2) {
    if (!dst || !src) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_copy, dim3((unsigned)blocks), dim3(kThreads), 0, st, (u32x4*)dst, (const u32x4*)src, units);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
