// zero_internal.h -- structures shared by the host launcher and the gfx950
// kernels of libzero.so.  Everything a kernel needs travels in its kernel
// arguments (no device-side tables, no allocation): per-launch tables are
// capped so the argument block stays under 4 KiB, and larger plans are
// covered by several launches.
#pragma once

#include <stdint.h>

#include "zero.h"

namespace zk {

constexpr int kMaxRanks = ZERO_MAX_RANKS;   // gradient pointers per launch
constexpr int kMaxSeg = 64;                  // shard segments per step launch
constexpr int kMaxCopy = 112;                // copy entries per copy launch
constexpr int64_t kSegMaxElems = int64_t(1) << 28;  // keeps per-lane byte offsets in 32 bits

constexpr int kThreads = 256;               // copy and element kernels: 4 wave64s
constexpr int kStepThreads = 512;           // vector step kernel: 8 wave64s (8 wave tiles)
constexpr int kStepVec = 8;                 // elements per lane in the vector step kernel
constexpr int kCopyUnits = 8;               // 16-byte units per lane in the copy kernel

// Write windows (vector step kernel, fused and reduce-only modes): a wave that
// has its results ready waits until the device's constant-rate real-time
// counter (the rate hipDeviceAttributeWallClockRate reports; 100 MHz on
// MI355X) enters the first win_open ticks of a win_period-tick period, then
// stores.  Stores of the whole device are thereby gathered into short bursts
// instead of trickling between the gradient reads.
constexpr uint32_t kMaxWindowPeriod = 100000;    // ticks (1 ms at 100 MHz)
constexpr uint32_t kWindowSpinMax = 1u << 16;    // bound on a wave's wait-loop iterations

// One contiguous piece of the owner's shard (a bucket's slice, or part of it).
struct StepSeg {
  int64_t shard_off;    // element offset in the shard-local arrays (state, compact grads)
  int64_t full_off;     // element offset in a full gradient buffer (Stage 1)
  int64_t dst_off;      // element offset in the parameter destination
  int32_t len;          // elements, <= kSegMaxElems
  int32_t block_start;  // first workgroup of this piece in the launch
};

enum StepMode : int {
  kFused = 0,        // reduce ranks in registers, then Adam, cast, store
  kFromReduced = 1,  // Adam reading an fp32 reduced gradient
  kReduceOnly = 2    // fold ranks, write fp32
};

enum StepFlags : int {
  kFlagInitFromOut = 1,   // reduce: continue the fold from the fp32 output
  kFlagApplyScale = 2     // reduce: multiply by grad_scale at the end
};

struct StepArgs {
  const void* grad[kMaxRanks];
  uint32_t full_mask[kMaxRanks / 32];
  const float* reduced;   // kFromReduced input
  float* out;             // kReduceOnly output
  float* master;
  float* m;
  float* v;
  void* dst;
  float c[9];             // b1, 1-b1, b2, 1-b2, 1-b1^t, 1-b2^t, lr, eps, grad_scale
  int32_t n_ranks;
  int32_t n_seg;
  int32_t flags;
  uint32_t win_period;    // write window period in real-time-counter ticks; 0 = store at once
  uint32_t win_open;      // ticks at the start of each period during which waves store
  int32_t pad_;
  StepSeg seg[kMaxSeg];
};

// One copy: n elements from src (nullptr = zeros) to dst + dst_off.
struct CopyEnt {
  const void* src;
  int64_t dst_off;
  int64_t n;
  int32_t block_start;
  int32_t pad_;
};

struct CopyArgs {
  void* dst;
  int32_t n_ent;
  int32_t pad_;
  CopyEnt ent[kMaxCopy];
};

// Ranges of the fused step's own fp32 state read ahead of it with ordinary
// (cached) loads; nothing is written.  See warm_kernel in zero_kernels.hip.
constexpr int kWarmRanges = 3;
constexpr int kWarmThreads = 1024;   // workgroup
constexpr int kWarmUnits = 8;        // 16-byte loads per lane
struct WarmArgs {
  const void* base[kWarmRanges];      // 16-byte aligned
  int64_t units[kWarmRanges];         // 16-byte units of each range
  int32_t block_start[kWarmRanges];   // first workgroup of each range
  int32_t n;                          // ranges in use
};

static_assert(sizeof(StepArgs) <= 4096, "step kernel arguments must fit 4 KiB");
static_assert(sizeof(CopyArgs) <= 4096, "copy kernel arguments must fit 4 KiB");

// Kernel launchers (zero_kernels.hip).  Return a hipError_t as int.
int launch_step(const StepArgs& a, int mode, int gdt, int pdt, int ndc, bool vec, int n_blocks,
                void* stream);
int launch_copy(const CopyArgs& a, int esz, int n_blocks, void* stream);
int launch_warm(const WarmArgs& a, int n_blocks, void* stream);
const char* hip_error_string(int err);
// Workgroups of the chosen step kernel that the current device holds at once
// (blocks per CU at the kernel's register use x CUs); 0 if unknown.
int resident_blocks(int mode, int gdt, int pdt, int ndc, bool vec);
// Ticks per second of the current device's real-time counter; 0 if unknown.
double wall_clock_hz();
// Peak HBM bytes per second of the current device from its memory clock and
// bus width (clock x 4 transfers x width); 0 if unknown.
double hbm_peak_bps();

}  // namespace zk
