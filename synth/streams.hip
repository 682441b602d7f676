// streams.hip -- streams restricted to a subset of the compute units, for
// the Stage-3 prefetch loop of the benchmark and tests: layer compute on one
// set of CUs, the next layer's gather on the rest.  Plain HIP runtime calls,
// no kernels; part of libsynth.so (bench and test support), not of libzero.so.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

// Compute units of the current device.
extern "C" int synth_cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(out, hipDeviceAttributeMultiprocessorCount, dev);
  return (int)e;
}

// A stream whose kernels run only on the CUs whose bits are set in mask
// (n_words 32-bit words, bit i = CU i as the runtime numbers them), at the
// default priority.  Returns a HIP error code; *out receives the stream.
extern "C" int synth_stream_create_cu_masked(uint32_t n_words, const uint32_t* mask, void** out) {
  if (!mask || !out || n_words == 0) return (int)hipErrorInvalidValue;
  hipStream_t s = nullptr;
  const hipError_t e = hipExtStreamCreateWithCUMask(&s, n_words, mask);
  *out = (void*)s;
  return (int)e;
}

extern "C" int synth_stream_destroy(void* s) { return (int)hipStreamDestroy((hipStream_t)s); }

// An elastic stand-in for a layer's compute in the Stage-3 prefetch study:
// `blocks` workgroups of 256 threads, each thread reading one 16-bit weight
// of the gathered layer and running `iters` dependent fp32 multiply-adds on
// it, each workgroup storing one word.  Unlike a GEMM sized to the chip, its
// many short workgroups leave compute units free as they retire, so a kernel
// on another stream can take them.  `lds_bytes` of dynamic LDS per workgroup
// (at least 4, at most 64 KiB) bounds how many workgroups share a CU, and so
// the wave slots left to other kernels.  Bench support only.
namespace {
__global__ void __launch_bounds__(256) elastic_compute(const uint16_t* w, int64_t n, int32_t iters, float* out) {
  extern __shared__ float acc[];
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) % n;
  float x = (float)w[i] * 0x1.0p-16f;
  const float a = 0.999f, b = 1e-3f;
  for (int32_t k = 0; k < iters; ++k) x = __builtin_fmaf(x, a, b);
  if (threadIdx.x == 0) acc[0] = 0.0f;
  __syncthreads();
  atomicAdd(&acc[0], x);
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = acc[0];
}
}  // namespace

// out: `blocks` floats.  Returns a HIP error code.
extern "C" int synth_elastic_compute(const void* w, int64_t n, int32_t iters, int32_t blocks, int32_t lds_bytes,
                                     float* out, void* stream) {
  if (!w || n <= 0 || !out || blocks <= 0 || iters < 0 || lds_bytes < 4 || lds_bytes > 65536)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(elastic_compute, dim3((unsigned)blocks), dim3(256), (unsigned)lds_bytes, (hipStream_t)stream,
                     (const uint16_t*)w, n, iters, out);
  return (int)hipGetLastError();
}
