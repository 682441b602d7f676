// probes.hip -- HBM calibration probes for the benchmark: a plain read, a
// plain write and a plain copy of a large buffer, each in 16-byte
// non-temporal accesses, so their bandwidth can be reported beside the
// step's.  No arithmetic of the ZeRO step; part of libsynth.so
// (bench and test support), not of libzero.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) u32x4 gu32x4;

// Workgroup shape per probe, the fastest of a sweep of 64-1024 threads and
// 2-16 units per lane on MI355X (read: 1024 x 8; write and copy: 256 x 4;
// copies with 8 units per lane ran 15% slower).
constexpr int kReadThreads = 1024, kReadUnits = 8;
constexpr int kWriteThreads = 256, kWriteUnits = 4;
constexpr int kCopyThreads = 256, kCopyUnits = 4;

// Every kernel below gives full workgroups (all U units of every lane in
// range; the branch is uniform) a path without per-unit bounds checks, in
// which wave w covers the workgroup's w-th 64 * U units as 1 KiB wave-wide
// spans: every address is one lane base plus an immediate offset, and all of
// a lane's loads are in flight together.  Only the last workgroup checks each
// unit.
__device__ __forceinline__ uint32_t wave_lane(int units_per_lane) {
  return (threadIdx.x >> 6) * (64 * units_per_lane) + (threadIdx.x & 63);
}

template <bool NT>
__device__ __forceinline__ u32x4 load16(const gu32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// Reads `units` 16-byte units (NT: non-temporal loads; else ordinary cached
// loads); each workgroup stores one word (the xor of what its first lane
// read), so the loads cannot be dropped.
template <int T, int U, bool NT>
__global__ void __launch_bounds__(T) probe_read(const u32x4* src, int64_t units, uint32_t* sink) {
  const int64_t first = (int64_t)blockIdx.x * T * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (first + T * U <= units) {
    const gu32x4* wv = (const gu32x4*)(src + first) + wave_lane(U);
    u32x4 r[U];
#pragma unroll
    for (int i = 0; i < U; ++i) r[i] = load16<NT>(wv + i * 64);
#pragma unroll
    for (int i = 0; i < U; ++i) acc ^= r[i];
  } else {
    for (int i = 0; i < U; ++i) {
      const int64_t u = first + threadIdx.x + (int64_t)i * T;
      if (u < units) acc ^= load16<NT>((const gu32x4*)(src + u));
    }
  }
  const uint32_t x = __builtin_amdgcn_readfirstlane(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (threadIdx.x == 0) sink[blockIdx.x] = x;
}

template <int T, int U>
__global__ void __launch_bounds__(T) probe_write(u32x4* dst, int64_t units, uint32_t value) {
  const int64_t first = (int64_t)blockIdx.x * T * U;
  const u32x4 v = {value, value, value, value};
  if (first + T * U <= units) {
    gu32x4* dw = (gu32x4*)(dst + first) + wave_lane(U);
#pragma unroll
    for (int i = 0; i < U; ++i) __builtin_nontemporal_store(v, dw + i * 64);
  } else {
    for (int i = 0; i < U; ++i) {
      const int64_t u = first + threadIdx.x + (int64_t)i * T;
      if (u < units) __builtin_nontemporal_store(v, (gu32x4*)(dst + u));
    }
  }
}

template <int T, int U>
__global__ void __launch_bounds__(T) probe_copy(u32x4* dst, const u32x4* src, int64_t units) {
  const int64_t first = (int64_t)blockIdx.x * T * U;
  if (first + T * U <= units) {
    const gu32x4* sw = (const gu32x4*)(src + first) + wave_lane(U);
    gu32x4* dw = (gu32x4*)(dst + first) + wave_lane(U);
    u32x4 r[U];
#pragma unroll
    for (int i = 0; i < U; ++i) r[i] = __builtin_nontemporal_load(sw + i * 64);
#pragma unroll
    for (int i = 0; i < U; ++i) __builtin_nontemporal_store(r[i], dw + i * 64);
  } else {
    for (int i = 0; i < U; ++i) {
      const int64_t u = first + threadIdx.x + (int64_t)i * T;
      if (u < units) __builtin_nontemporal_store(__builtin_nontemporal_load((const gu32x4*)(src + u)),
                                                 (gu32x4*)(dst + u));
    }
  }
}

// A copy on a capped grid: each workgroup walks chunks of T * U units
// blockIdx.x, blockIdx.x + gridDim.x, ... (full chunks, wave layout as above);
// workgroup 0 then copies the ragged tail unit by unit.  With few workgroups
// it holds a few CUs and draws a fraction of HBM bandwidth, as a rate-limited
// background transfer would.
template <int T, int U>
__global__ void __launch_bounds__(T) probe_copy_capped(u32x4* dst, const u32x4* src, int64_t units) {
  const int64_t chunk = (int64_t)T * U;
  const int64_t full = units / chunk;
  const uint32_t wl = wave_lane(U);
  for (int64_t c = blockIdx.x; c < full; c += gridDim.x) {
    const gu32x4* sw = (const gu32x4*)(src + c * chunk) + wl;
    gu32x4* dw = (gu32x4*)(dst + c * chunk) + wl;
    u32x4 r[U];
#pragma unroll
    for (int i = 0; i < U; ++i) r[i] = __builtin_nontemporal_load(sw + i * 64);
#pragma unroll
    for (int i = 0; i < U; ++i) __builtin_nontemporal_store(r[i], dw + i * 64);
  }
  if (blockIdx.x == 0)
    for (int64_t u = full * chunk + threadIdx.x; u < units; u += T)
      __builtin_nontemporal_store(__builtin_nontemporal_load((const gu32x4*)(src + u)), (gu32x4*)(dst + u));
}

int64_t blocks_for(int64_t units, int per_block) { return (units + per_block - 1) / per_block; }

}  // namespace

// kind 0: read `bytes` at src (sink: one word per workgroup, see
// synth_probe_sink_words); 1: write `bytes` at dst; 2: copy `bytes` from src
// to dst; 3: as 0 with ordinary cached loads instead of non-temporal ones.  bytes must be a multiple of 16 and pointers 16-byte aligned.
// Returns 0 or a HIP error code.
extern "C" int64_t synth_probe_sink_words(int64_t bytes) { return blocks_for(bytes / 16, kReadThreads * kReadUnits); }

extern "C" int synth_probe(int kind, void* dst, const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes <= 0) return 0;
  if ((bytes & 15) || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15)) return (int)hipErrorInvalidValue;
  const int64_t units = bytes / 16;
  hipStream_t st = (hipStream_t)stream;
  if (kind == 0 || kind == 3) {
    const int64_t blocks = blocks_for(units, kReadThreads * kReadUnits);
    if (!src || !sink || blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    if (kind == 0)
      hipLaunchKernelGGL((probe_read<kReadThreads, kReadUnits, true>), dim3((unsigned)blocks), dim3(kReadThreads), 0,
                         st, (const u32x4*)src, units, sink);
    else
      hipLaunchKernelGGL((probe_read<kReadThreads, kReadUnits, false>), dim3((unsigned)blocks), dim3(kReadThreads), 0,
                         st, (const u32x4*)src, units, sink);
  } else if (kind == 1) {
    const int64_t blocks = blocks_for(units, kWriteThreads * kWriteUnits);
    if (!dst || blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((probe_write<kWriteThreads, kWriteUnits>), dim3((unsigned)blocks), dim3(kWriteThreads), 0, st,
                       (u32x4*)dst, units, 0x3c003c00u);
  } else if (kind == 2) {
    const int64_t blocks = blocks_for(units, kCopyThreads * kCopyUnits);
    if (!dst || !src || blocks > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL((probe_copy<kCopyThreads, kCopyUnits>), dim3((unsigned)blocks), dim3(kCopyThreads), 0, st,
                       (u32x4*)dst, (const u32x4*)src, units);
  } else {
    return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// Copy `bytes` from src to dst on at most `max_blocks` workgroups of the copy
// shape (fewer when the copy has fewer chunks).  Same alignment rules as
// synth_probe.  Returns 0 or a HIP error code.
extern "C" int synth_probe_copy_capped(void* dst, const void* src, int64_t bytes, int32_t max_blocks, void* stream) {
  if (bytes <= 0) return 0;
  if (!dst || !src || max_blocks <= 0 || (bytes & 15) || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15))
    return (int)hipErrorInvalidValue;
  const int64_t units = bytes / 16;
  int64_t blocks = units / (kCopyThreads * kCopyUnits);
  if (blocks > max_blocks) blocks = max_blocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((probe_copy_capped<kCopyThreads, kCopyUnits>), dim3((unsigned)blocks), dim3(kCopyThreads), 0,
                     (hipStream_t)stream, (u32x4*)dst, (const u32x4*)src, units);
  return (int)hipGetLastError();
}
