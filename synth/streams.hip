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
