// zero_api.cpp -- host side of libzero.so: the plan, argument checks, launch
// tables and the extern "C" entry points declared in include/zero.h.
//
// The plan follows the ZeRO pages' ownership convention (mind-map page,
// "shrink the problem: four GPUs": rank i keeps the i-th contiguous block)
// applied per bucket (concept page, design trade-off 1: collectives run over
// buckets).  Nothing here allocates device memory; every kernel receives its
// tables in its kernel arguments, split over several launches when a plan has
// more pieces than one argument block holds.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "zero.h"
#include "zero_internal.h"

#define ZERO_VERSION_NUMBER 200  // 0.2.0

struct zero_plan_s {
  int64_t psi = 0;
  int32_t n_d = 1;
  int64_t bucket_cap = 0;
  int32_t align = 1;
  int64_t psi_pad = 0;
  int64_t shard_total = 0;
  struct Bucket {
    int64_t flat_off, numel, padded, shard_numel, shard_off;
  };
  std::vector<Bucket> buckets;
  std::vector<int64_t> t_numel;
  std::vector<int64_t> t_off;
  std::vector<int32_t> t_bucket;
};

namespace {

thread_local std::string g_err;

zero_status fail(zero_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

zero_status ok() { return ZERO_OK; }

int esize(int dt) { return dt == ZERO_F32 ? 4 : 2; }
bool is16(int dt) { return dt == ZERO_F16 || dt == ZERO_BF16; }
bool valid_dt(int dt) { return dt == ZERO_F32 || dt == ZERO_F16 || dt == ZERO_BF16; }

struct Range {
  uint64_t lo, hi;  // [lo, hi) bytes
  const char* what;
};

Range range_of(const void* p, int64_t elems, int es, const char* what) {
  const uint64_t lo = (uint64_t)(uintptr_t)p;
  return Range{lo, lo + (uint64_t)elems * (uint64_t)es, what};
}

bool overlap(const Range& a, const Range& b) {
  if (a.hi == a.lo || b.hi == b.lo) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void* p, int bytes) { return ((uintptr_t)p % (uintptr_t)bytes) == 0; }

zero_status hip_fail(int err) {
  return fail(ZERO_EHIP, "HIP launch failed: %s (%d)", zk::hip_error_string(err), err);
}

// The nine fp32 constants of step t, rounded once from fp64.
void adam_consts(const zero_adam_hyper& h, int64_t t, float c[9]) {
  c[0] = (float)h.beta1;
  c[1] = (float)(1.0 - h.beta1);
  c[2] = (float)h.beta2;
  c[3] = (float)(1.0 - h.beta2);
  c[4] = (float)(1.0 - std::pow(h.beta1, (double)t));
  c[5] = (float)(1.0 - std::pow(h.beta2, (double)t));
  c[6] = (float)h.lr;
  c[7] = (float)h.eps;
  c[8] = (float)h.grad_scale;
}

// One piece of the owner's shard, before it is packed into a launch.
struct Piece {
  int64_t shard_off, full_off, dst_off, len;
};

std::vector<Piece> owner_pieces(const zero_plan_s& p, int32_t rank, bool dst_full) {
  std::vector<Piece> out;
  for (const auto& b : p.buckets) {
    const int64_t own = b.flat_off + (int64_t)rank * b.shard_numel;
    for (int64_t k = 0; k < b.shard_numel; k += zk::kSegMaxElems) {
      const int64_t len = std::min<int64_t>(zk::kSegMaxElems, b.shard_numel - k);
      out.push_back(Piece{b.shard_off + k, own + k, (dst_full ? own : b.shard_off) + k, len});
    }
  }
  return out;
}

// Pieces for the vector kernel and for the element kernel.  The vector kernel
// needs every offset it addresses -- the shard offset (state, compact
// gradients, reduced gradient), the destination offset and, where a rank
// reads a full buffer, the full offset -- to be a multiple of 4 elements; its
// length is free.  A piece whose offsets agree modulo 4 gives its first
// (< 4) elements to the element kernel and the rest to the vector kernel;
// one whose offsets disagree modulo 4 goes to the element kernel whole.
void split_pieces(const std::vector<Piece>& ps, bool uses_full, bool uses_dst, std::vector<Piece>& vec,
                  std::vector<Piece>& elem) {
  for (const auto& q : ps) {
    const int64_t r = q.shard_off & 3;
    const bool agree = (!uses_dst || (q.dst_off & 3) == r) && (!uses_full || (q.full_off & 3) == r);
    if (!agree) {
      elem.push_back(q);
      continue;
    }
    const int64_t head = std::min<int64_t>((4 - r) & 3, q.len);
    if (head > 0) elem.push_back(Piece{q.shard_off, q.full_off, q.dst_off, head});
    if (q.len > head) vec.push_back(Piece{q.shard_off + head, q.full_off + head, q.dst_off + head, q.len - head});
  }
}

int ndc_for(int n) { return (n == 4 || n == 8 || n == 16 || n == 64) ? n : 0; }

// Write-window setting: period in the high 32 bits, open ticks in the low 32;
// kWindowAuto = automatic.  One word, so a reader never sees a torn pair.
// The process-wide default, and per-stream settings that override it.
constexpr uint64_t kWindowAuto = ~0ull;
std::atomic<uint64_t> g_window{kWindowAuto};
std::mutex g_stream_window_mu;
std::vector<std::pair<void*, uint64_t>> g_stream_window;   // guarded by g_stream_window_mu
std::atomic<int> g_stream_window_count{0};                 // entries, read without the lock

uint64_t window_setting(void* stream) {
  if (g_stream_window_count.load(std::memory_order_acquire) > 0) {
    std::lock_guard<std::mutex> lk(g_stream_window_mu);
    for (const auto& e : g_stream_window)
      if (e.first == stream) return e.second;
  }
  return g_window.load(std::memory_order_relaxed);
}

// Encodes a (period, open) request; false if out of range.
bool encode_window(int64_t period_ticks, int64_t open_ticks, uint64_t& w) {
  if (period_ticks == -1) {
    w = kWindowAuto;
    return true;
  }
  if (period_ticks < 0 || period_ticks > (int64_t)zk::kMaxWindowPeriod) return false;
  if (period_ticks > 0 && (open_ticks < 1 || open_ticks > period_ticks)) return false;
  w = period_ticks == 0 ? 0 : ((uint64_t)period_ticks << 32) | (uint64_t)open_ticks;
  return true;
}

// Automatic choice.  A wave waits at most one period, so the period must stay
// well below the lifetime of a workgroup, or every generation of resident
// workgroups ends up taking a whole number of periods.  Sweeps on MI355X of
// the fused step (7.5B at N_d = 64, 13B at N_d = 16, a Stage-3 layer) and of
// the reduction found the best period near 0.62 of the time one generation of
// resident workgroups takes to stream its bytes at ~6.5 TB/s, and the best
// opening near the written share of the bytes (at least 1/16 of the period).
// The kernel compiled for 16 ranks (a quarter of its bytes written) does best
// at 0.74: 1.4-2.2% faster than at 0.62 on four shapes (13B, and 100M-400M
// shards in bf16 and fp16), with the gain gone by 0.82 and a loss from 0.86.
// Reduce-only launches (3-11% written) do best at 0.45: 0.2-4.6% faster than
// at 0.62 on the 7.5B shard and N_d = 32, 128 and 200, in two same-process
// comparisons; on the 16-rank kernel shorter periods lose (1.6% at 0.45), so
// it keeps 0.62 there.
// Launches with few ranks per written element or few elements gain nothing.
// A launch of few generations does better with a shorter period: its waits at
// the end are not hidden by later generations.  Up to 6 generations take at
// most half the period (a Stage-3 layer is three), and the full period is
// reached at 12.  The kernel for rank counts that are not compiled in (other
// than 4, 8, 16, 64) does better with an opening of 1.5 times the written
// share once that share passes 12% (N_d below ~44): 2-5% at N_d = 24 and 32,
// where the written share alone left its waves waiting.  The last two rules
// come from a same-process comparison over 14 shapes (N_d 16-128, shards of
// 20M-812M elements); neither changes the window of the workloads above.  The
// streaming rate is a fixed share of the HBM peak the device reports (memory
// clock x 4 transfers x bus width: 8.19 TB/s on MI355X, 5.3 TB/s on MI300X),
// and periods are converted to ticks with the rate the device reports for its
// real-time counter.
constexpr int kAutoMinRanks = 16;
constexpr double kAutoShortGenerations = 6.0;
constexpr double kAutoFullGenerations = 12.0;
constexpr int64_t kAutoMinElems = int64_t(1) << 23;
constexpr double kAutoStreamShare = 6.5e12 / 8.192e12;   // 6.5 TB/s on MI355X
constexpr double kAutoPeriodShare = 0.62;                 // of one generation's streaming time
constexpr double kAutoPeriodShare16 = 0.74;               //   for the 16-rank kernel's fused step
constexpr double kAutoPeriodShareReduce = 0.45;           //   for other reduce-only launches
constexpr double kAutoWideOpeningShare = 0.12;            // generic kernel: written share above which
constexpr double kAutoWideOpening = 1.5;                  //   the opening is this multiple of it

void auto_window(int mode, int gdt, int pdt, int ndc, int n_ranks, int64_t elems, int64_t blocks,
                 zk::StepArgs& a) {
  if (n_ranks < kAutoMinRanks || elems < kAutoMinElems) return;
  const int resident = zk::resident_blocks(mode, gdt, pdt, ndc, true);
  if (resident <= 0 || blocks < 2 * (int64_t)resident) return;
  const double hz = zk::wall_clock_hz();
  const double peak = zk::hbm_peak_bps();
  if (!(hz > 0) || !(peak > 0)) return;
  const double read = 2.0 * n_ranks + (mode == zk::kFused ? 12.0 : (a.flags & zk::kFlagInitFromOut) ? 4.0 : 0.0);
  const double written = mode == zk::kFused ? 14.0 : 4.0;
  const double gen_bytes = (double)resident * zk::kStepThreads * zk::kStepVec * (read + written);
  const bool fused = mode == zk::kFused;
  const double share = ndc == 16 ? (fused ? kAutoPeriodShare16 : kAutoPeriodShare)
                                 : (fused ? kAutoPeriodShare : kAutoPeriodShareReduce);
  double period = gen_bytes / (kAutoStreamShare * peak) * share * hz;
  const double gens = (double)blocks / resident;
  period *= gens < kAutoShortGenerations
                ? std::min(0.5, gens / kAutoShortGenerations)
                : std::min(1.0, 0.5 + 0.5 * (gens - kAutoShortGenerations) /
                                          (kAutoFullGenerations - kAutoShortGenerations));
  const double min_period = 2e-6 * hz;   // 2 us
  period = std::min<double>(std::max(period, min_period), (double)zk::kMaxWindowPeriod);
  const double w_share = written / (read + written);
  const double o_share = ndc == 0 && w_share > kAutoWideOpeningShare ? kAutoWideOpening * w_share : w_share;
  const double open = period * std::min(0.5, std::max(o_share, 1.0 / 16.0));
  a.win_period = (uint32_t)period;
  a.win_open = std::max<uint32_t>(1, std::min<uint32_t>((uint32_t)open, a.win_period));
}

void pick_window(int mode, int gdt, int pdt, int ndc, int n_ranks, int64_t elems, int64_t blocks, bool vec,
                 void* stream, zk::StepArgs& a) {
  a.win_period = 0;
  a.win_open = 0;
  if (!vec || mode == zk::kFromReduced) return;
  const uint64_t w = window_setting(stream);
  if (w != kWindowAuto) {
    a.win_period = (uint32_t)(w >> 32);
    a.win_open = (uint32_t)w;
    return;
  }
  auto_window(mode, gdt, pdt, ndc, n_ranks, elems, blocks, a);
}

// Launch the step kernel over all pieces, in chunks of kMaxSeg.
zero_status run_step(zk::StepArgs& a, const std::vector<Piece>& ps, int mode, int gdt, int pdt,
                     bool vec, void* stream) {
  const int per_block = vec ? zk::kStepThreads * zk::kStepVec : zk::kThreads;
  size_t i = 0;
  while (i < ps.size()) {
    int nseg = 0;
    int64_t blocks = 0;
    int64_t elems = 0;
    for (; i < ps.size() && nseg < zk::kMaxSeg; ++i) {
      const Piece& q = ps[i];
      const int64_t nb = (q.len + per_block - 1) / per_block;
      if (blocks + nb > INT32_MAX) break;
      zk::StepSeg& s = a.seg[nseg++];
      s.shard_off = q.shard_off;
      s.full_off = q.full_off;
      s.dst_off = q.dst_off;
      s.len = (int32_t)q.len;
      s.block_start = (int32_t)blocks;
      blocks += nb;
      elems += q.len;
    }
    a.n_seg = nseg;
    if (blocks == 0) continue;
    pick_window(mode, gdt, pdt, ndc_for(a.n_ranks), a.n_ranks, elems, blocks, vec, stream, a);
    const int err = zk::launch_step(a, mode, gdt, pdt, ndc_for(a.n_ranks), vec, (int)blocks, stream);
    if (err != 0) return hip_fail(err);
  }
  return ok();
}

// The step over the owner's pieces: the vector kernel where the buffers
// allow it (fp32 bases 16-byte aligned, 16-bit bases 8-byte aligned; offsets
// as split_pieces requires), the element kernel for the rest.  The two sets
// of pieces are disjoint.
zero_status run_step_all(zk::StepArgs& a, const std::vector<Piece>& ps, int mode, int gdt, int pdt,
                         bool vec_ok, bool uses_full, void* stream) {
  if (!vec_ok) return run_step(a, ps, mode, gdt, pdt, false, stream);
  std::vector<Piece> vec, elem;
  split_pieces(ps, uses_full, mode != zk::kReduceOnly, vec, elem);
  if (zero_status st = run_step(a, vec, mode, gdt, pdt, true, stream)) return st;
  return run_step(a, elem, mode, gdt, pdt, false, stream);
}

// Fill the rank table of a step launch with ranks [q0, q0 + n).
void set_ranks(zk::StepArgs& a, const zero_grad_src& src, int q0, int n) {
  memset(a.grad, 0, sizeof a.grad);
  memset(a.full_mask, 0, sizeof a.full_mask);
  for (int i = 0; i < n; ++i) {
    a.grad[i] = src.ptrs[q0 + i];
    if (src.is_full && src.is_full[q0 + i]) a.full_mask[i >> 5] |= 1u << (i & 31);
  }
  a.n_ranks = n;
}

// Common checks of a gradient source; collects the read ranges.
zero_status check_src(const zero_plan_s& p, const zero_grad_src* src, std::vector<Range>& reads,
                      bool& vec_ok) {
  if (!src) return fail(ZERO_EINVAL, "gradient source is NULL");
  if (src->n != p.n_d) return fail(ZERO_EINVAL, "gradient source has %d ranks, plan has n_d=%d", src->n, p.n_d);
  if (!src->ptrs) return fail(ZERO_EINVAL, "gradient pointer array is NULL");
  if (!is16(src->dtype)) return fail(ZERO_EUNSUPPORTED, "gradient dtype %d is not 16-bit", src->dtype);
  for (int q = 0; q < src->n; ++q) {
    const void* g = src->ptrs[q];
    const bool full = src->is_full && src->is_full[q];
    const int64_t n = full ? p.psi_pad : p.shard_total;
    if (!g && n > 0) return fail(ZERO_EINVAL, "gradient pointer of rank %d is NULL", q);
    if (!aligned(g, 2)) return fail(ZERO_EINVAL, "gradient of rank %d is not 2-byte aligned", q);
    if (!aligned(g, 8)) vec_ok = false;   // the vector kernel loads 4 elements (8 bytes) per rank
    reads.push_back(range_of(g, n, 2, "gradient"));
  }
  return ok();
}

zero_status check_plan(zero_plan_t p) {
  if (!p) return fail(ZERO_EINVAL, "plan is NULL");
  return ok();
}

// Warm-up read before a large fused step or reduction (warm_kernel), when
// enabled with zero_set_warm_read: as much as MI355X's Infinity Cache holds
// (256 MiB) of the step's own fp32 state (master first, then m and v), or of
// the reduction's fp32 output.  Only for launches that read at least 1 GiB of
// gradients.  Measured on MI355X: right after gradients written with ordinary
// stores the step is ~11% faster (7.5B, N_d = 64; 7.5% for a Stage-3 layer,
// 3% for 13B) and the reduction ~11%; when the gradients are already clean
// (written non-temporally, or launches back to back) it costs the step 1-2%
// and the reduction, which does not read those lines again, 2%.  Small
// launches (GPT-2's 0.25 GB) lose either way and never warm up.
constexpr int64_t kWarmBytes = int64_t(256) << 20;
constexpr int64_t kWarmMinGradBytes = int64_t(1) << 30;
std::atomic<int> g_warm{0};

zero_status warm_state(float* const* st, int n_st, int64_t S, int32_t n_d, void* stream) {
  if (!g_warm.load(std::memory_order_relaxed)) return ok();
  if (2 * (int64_t)n_d * S < kWarmMinGradBytes) return ok();
  for (int i = 0; i < n_st; ++i)
    if (!aligned(st[i], 16)) return ok();
  zk::WarmArgs w;
  memset(&w, 0, sizeof w);
  const int64_t per_block = (int64_t)zk::kWarmThreads * zk::kWarmUnits;
  int64_t left = kWarmBytes, blocks = 0;
  for (int i = 0; i < std::min(n_st, zk::kWarmRanges) && left >= 16; ++i) {
    const int64_t units = std::min<int64_t>(left, S * 4) / 16;
    if (units <= 0) continue;
    w.base[w.n] = st[i];
    w.units[w.n] = units;
    w.block_start[w.n] = (int32_t)blocks;
    blocks += (units + per_block - 1) / per_block;
    left -= units * 16;
    ++w.n;
  }
  if (w.n == 0) return ok();
  const int err = zk::launch_warm(w, (int)blocks, stream);
  return err ? hip_fail(err) : ok();
}

// Copy entries -> launches of kMaxCopy entries.
zero_status run_copies(std::vector<zk::CopyEnt>& ents, void* dst, int es, void* stream) {
  zk::CopyArgs a;
  memset(&a, 0, sizeof a);
  a.dst = dst;
  const int64_t units_per_block = (int64_t)zk::kThreads * zk::kCopyUnits;
  size_t i = 0;
  while (i < ents.size()) {
    int n = 0;
    int64_t blocks = 0;
    for (; i < ents.size() && n < zk::kMaxCopy; ++i) {
      const zk::CopyEnt& e = ents[i];
      if (e.n == 0) continue;
      const uint64_t d0 = (uint64_t)(uintptr_t)dst + (uint64_t)e.dst_off * es;
      const uint64_t d1 = d0 + (uint64_t)e.n * es;
      const int64_t units = (int64_t)(((d1 + 15) >> 4) - (d0 >> 4));
      const int64_t nb = (units + units_per_block - 1) / units_per_block;
      if (nb > INT32_MAX) return fail(ZERO_EINVAL, "copy of %lld elements exceeds one launch", (long long)e.n);
      if (blocks + nb > INT32_MAX) break;
      a.ent[n] = e;
      a.ent[n].block_start = (int32_t)blocks;
      ++n;
      blocks += nb;
    }
    a.n_ent = n;
    if (n == 0) continue;
    const int err = zk::launch_copy(a, es, (int)blocks, stream);
    if (err != 0) return hip_fail(err);
  }
  return ok();
}

}  // namespace

extern "C" {

int32_t zero_version(void) { return ZERO_VERSION_NUMBER; }

zero_status zero_set_write_window(int64_t period_ticks, int64_t open_ticks) {
  uint64_t w = 0;
  if (!encode_window(period_ticks, open_ticks, w))
    return fail(ZERO_EINVAL, "window (%lld, %lld): period_ticks must be -1 or in [0, %u], open_ticks in [1, period_ticks]",
                (long long)period_ticks, (long long)open_ticks, zk::kMaxWindowPeriod);
  g_window.store(w);
  return ok();
}

zero_status zero_set_stream_write_window(void* stream, int64_t period_ticks, int64_t open_ticks) {
  try {
    std::lock_guard<std::mutex> lk(g_stream_window_mu);
    auto it = std::find_if(g_stream_window.begin(), g_stream_window.end(),
                           [&](const std::pair<void*, uint64_t>& e) { return e.first == stream; });
    if (period_ticks == -2) {   // back to the process-wide setting
      if (it != g_stream_window.end()) g_stream_window.erase(it);
    } else {
      uint64_t w = 0;
      if (!encode_window(period_ticks, open_ticks, w))
        return fail(ZERO_EINVAL,
                    "window (%lld, %lld): period_ticks must be -2, -1 or in [0, %u], open_ticks in [1, period_ticks]",
                    (long long)period_ticks, (long long)open_ticks, zk::kMaxWindowPeriod);
      if (it != g_stream_window.end()) it->second = w;
      else g_stream_window.emplace_back(stream, w);
    }
    g_stream_window_count.store((int)g_stream_window.size(), std::memory_order_release);
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_set_stream_write_window");
  }
}

zero_status zero_set_warm_read(int32_t enable) {
  if (enable != 0 && enable != 1) return fail(ZERO_EINVAL, "enable must be 0 or 1 (got %d)", enable);
  g_warm.store(enable);
  return ok();
}

const char* zero_last_error(void) { return g_err.c_str(); }

zero_status zero_plan(int64_t psi, int32_t n_d, const int64_t* tensor_numel, int32_t n_tensors,
                      int64_t bucket_cap, int32_t shard_align, zero_plan_t* out) {
  try {
    if (!out) return fail(ZERO_EINVAL, "out is NULL");
    *out = nullptr;
    if (n_d < 1) return fail(ZERO_EINVAL, "n_d must be >= 1 (got %d)", n_d);
    if (shard_align < 1) return fail(ZERO_EINVAL, "shard_align must be >= 1 (got %d)", shard_align);
    if (bucket_cap < 0) return fail(ZERO_EINVAL, "bucket_cap must be >= 0");
    if (n_tensors < 0) return fail(ZERO_EINVAL, "n_tensors must be >= 0");
    if (n_tensors > 0 && !tensor_numel) return fail(ZERO_EINVAL, "tensor_numel is NULL");
    if (psi < 0) return fail(ZERO_EINVAL, "psi must be >= 0");
    int64_t sum = 0;
    for (int32_t t = 0; t < n_tensors; ++t) {
      if (tensor_numel[t] < 0) return fail(ZERO_EINVAL, "tensor %d has negative size", t);
      if (tensor_numel[t] > INT64_MAX / 4 - sum) return fail(ZERO_EINVAL, "tensor sizes overflow");
      sum += tensor_numel[t];
    }
    if (sum != psi)
      return fail(ZERO_EINVAL, "tensor sizes sum to %lld, psi is %lld", (long long)sum, (long long)psi);
    const int64_t unit = (int64_t)n_d * shard_align;

    zero_plan_s* p = new zero_plan_s();
    p->psi = psi;
    p->n_d = n_d;
    p->bucket_cap = bucket_cap;
    p->align = shard_align;
    p->t_numel.assign(tensor_numel, tensor_numel + n_tensors);
    p->t_off.resize(n_tensors);
    p->t_bucket.resize(n_tensors);

    // Greedy list-order bucketing: close the open bucket when the next tensor
    // would take it past the cap.
    int64_t flat = 0, shard = 0, open_numel = 0;
    bool open = false;
    // The padded layout must stay addressable in bytes for fp32 buffers:
    // psi_pad * 4 <= INT64_MAX.  Each bucket adds less than `unit` padding,
    // so the check runs before every addition.
    constexpr int64_t kMaxPadded = INT64_MAX / 4;
    bool too_big = false;
    auto close_bucket = [&]() {
      const int64_t rem = open_numel % unit;
      const int64_t pad = rem ? unit - rem : 0;
      if (open_numel > kMaxPadded - flat || pad > kMaxPadded - flat - open_numel) {
        too_big = true;
        return;
      }
      const int64_t padded = open_numel + pad;
      const int64_t sn = padded / n_d;
      p->buckets.push_back({flat, open_numel, padded, sn, shard});
      flat += padded;
      shard += sn;
      open = false;
      open_numel = 0;
    };
    for (int32_t t = 0; t < n_tensors && !too_big; ++t) {
      const int64_t n = tensor_numel[t];
      if (open && bucket_cap > 0 && open_numel + n > bucket_cap) close_bucket();
      if (too_big) break;
      p->t_bucket[t] = (int32_t)p->buckets.size();
      p->t_off[t] = flat + open_numel;
      open_numel += n;
      open = true;
    }
    if (open && !too_big) close_bucket();
    if (too_big) {
      delete p;
      return fail(ZERO_EINVAL, "padded layout exceeds %lld elements (n_d * shard_align = %lld per bucket)",
                  (long long)kMaxPadded, (long long)unit);
    }
    p->psi_pad = flat;
    p->shard_total = shard;
    *out = p;
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_plan");
  }
}

void zero_plan_destroy(zero_plan_t plan) { delete plan; }

zero_status zero_plan_info(zero_plan_t p, int64_t* psi_pad, int64_t* shard_total, int32_t* n_buckets,
                           int32_t* n_d) {
  if (check_plan(p)) return ZERO_EINVAL;
  if (psi_pad) *psi_pad = p->psi_pad;
  if (shard_total) *shard_total = p->shard_total;
  if (n_buckets) *n_buckets = (int32_t)p->buckets.size();
  if (n_d) *n_d = p->n_d;
  return ok();
}

zero_status zero_plan_bucket(zero_plan_t p, int32_t b, int64_t* flat_off, int64_t* numel,
                             int64_t* padded, int64_t* shard_numel, int64_t* shard_off) {
  if (check_plan(p)) return ZERO_EINVAL;
  if (b < 0 || b >= (int32_t)p->buckets.size()) return fail(ZERO_EINVAL, "bucket %d out of range", b);
  const auto& k = p->buckets[b];
  if (flat_off) *flat_off = k.flat_off;
  if (numel) *numel = k.numel;
  if (padded) *padded = k.padded;
  if (shard_numel) *shard_numel = k.shard_numel;
  if (shard_off) *shard_off = k.shard_off;
  return ok();
}

zero_status zero_plan_tensor(zero_plan_t p, int32_t t, int32_t* bucket, int64_t* flat_off) {
  if (check_plan(p)) return ZERO_EINVAL;
  if (t < 0 || t >= (int32_t)p->t_numel.size()) return fail(ZERO_EINVAL, "tensor %d out of range", t);
  if (bucket) *bucket = p->t_bucket[t];
  if (flat_off) *flat_off = p->t_off[t];
  return ok();
}

size_t zero_flatten_workspace_bytes(zero_plan_t) { return 0; }

zero_status zero_flatten(zero_plan_t p, const void* const* tensors, zero_dtype dt, void* flat,
                         void* workspace, size_t ws_bytes, void* stream) {
  try {
    (void)workspace;
    (void)ws_bytes;   // zero_flatten_workspace_bytes() is 0 for every plan
    if (check_plan(p)) return ZERO_EINVAL;
    if (!valid_dt(dt)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dt);
    const int es = esize(dt);
    const int32_t nt = (int32_t)p->t_numel.size();
    if (nt > 0 && !tensors) return fail(ZERO_EINVAL, "tensor pointer array is NULL");
    if (!flat && p->psi_pad > 0) return fail(ZERO_EINVAL, "flat is NULL");
    if (!aligned(flat, es)) return fail(ZERO_EINVAL, "flat is not element aligned");
    const Range out = range_of(flat, p->psi_pad, es, "flat");
    std::vector<zk::CopyEnt> ents;
    ents.reserve(nt + p->buckets.size());
    for (int32_t t = 0; t < nt; ++t) {
      const int64_t n = p->t_numel[t];
      if (n == 0) continue;
      if (!tensors[t]) return fail(ZERO_EINVAL, "tensor %d is NULL", t);
      if (!aligned(tensors[t], es)) return fail(ZERO_EINVAL, "tensor %d is not element aligned", t);
      if (overlap(out, range_of(tensors[t], n, es, "tensor")))
        return fail(ZERO_EINVAL, "flat overlaps tensor %d", t);
      ents.push_back(zk::CopyEnt{tensors[t], p->t_off[t], n, 0, 0});
    }
    for (const auto& b : p->buckets)   // zero padding at each bucket's end
      if (b.padded > b.numel) ents.push_back(zk::CopyEnt{nullptr, b.flat_off + b.numel, b.padded - b.numel, 0, 0});
    return run_copies(ents, flat, es, stream);
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_flatten");
  }
}

zero_status zero_gather_pack(zero_plan_t p, const void* const* shards, zero_dtype dt, void* full,
                             void* stream) {
  try {
    if (check_plan(p)) return ZERO_EINVAL;
    if (!valid_dt(dt)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dt);
    const int es = esize(dt);
    if (!shards) return fail(ZERO_EINVAL, "shard pointer array is NULL");
    if (!full && p->psi_pad > 0) return fail(ZERO_EINVAL, "full is NULL");
    if (!aligned(full, es)) return fail(ZERO_EINVAL, "full is not element aligned");
    const Range out = range_of(full, p->psi_pad, es, "full");
    for (int32_t q = 0; q < p->n_d; ++q) {
      if (!shards[q] && p->shard_total > 0) return fail(ZERO_EINVAL, "shard %d is NULL", q);
      if (!aligned(shards[q], es)) return fail(ZERO_EINVAL, "shard %d is not element aligned", q);
      if (overlap(out, range_of(shards[q], p->shard_total, es, "shard")))
        return fail(ZERO_EINVAL, "full overlaps shard %d", q);
    }
    std::vector<zk::CopyEnt> ents;
    ents.reserve((size_t)p->n_d * p->buckets.size());
    for (const auto& b : p->buckets)
      for (int32_t q = 0; q < p->n_d; ++q)
        ents.push_back(zk::CopyEnt{(const char*)shards[q] + b.shard_off * es,
                                   b.flat_off + (int64_t)q * b.shard_numel, b.shard_numel, 0, 0});
    return run_copies(ents, full, es, stream);
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_gather_pack");
  }
}

zero_status zero_reshard(zero_plan_t sp, zero_plan_t dp, int32_t dst_rank, const void* const* src_shards,
                         zero_dtype dt, void* dst_shard, void* stream) {
  try {
    if (!sp || !dp) return fail(ZERO_EINVAL, "plan is NULL");
    if (!valid_dt(dt)) return fail(ZERO_EINVAL, "unknown dtype %d", (int)dt);
    if (sp->t_numel != dp->t_numel)
      return fail(ZERO_EINVAL, "plans describe different tensor lists");
    if (dst_rank < 0 || dst_rank >= dp->n_d)
      return fail(ZERO_EINVAL, "dst_rank %d outside [0, %d)", dst_rank, dp->n_d);
    const int es = esize(dt);
    if (!src_shards) return fail(ZERO_EINVAL, "source shard pointer array is NULL");
    if (!dst_shard && dp->shard_total > 0) return fail(ZERO_EINVAL, "dst_shard is NULL");
    if (!aligned(dst_shard, es)) return fail(ZERO_EINVAL, "dst_shard is not element aligned");
    const Range out = range_of(dst_shard, dp->shard_total, es, "dst_shard");
    for (int32_t q = 0; q < sp->n_d; ++q) {
      if (!src_shards[q] && sp->shard_total > 0) return fail(ZERO_EINVAL, "source shard %d is NULL", q);
      if (!aligned(src_shards[q], es)) return fail(ZERO_EINVAL, "source shard %d is not element aligned", q);
      if (overlap(out, range_of(src_shards[q], sp->shard_total, es, "source shard")))
        return fail(ZERO_EINVAL, "dst_shard overlaps source shard %d", q);
    }
    // Walk the destination rank's owned ranges bucket by bucket: real
    // elements come from whichever source rank owns the same tensor element,
    // padding is written as zero.
    std::vector<zk::CopyEnt> ents;
    const int32_t nt = (int32_t)dp->t_numel.size();
    int32_t t = 0;
    for (size_t b = 0; b < dp->buckets.size(); ++b) {
      const auto& B = dp->buckets[b];
      const int64_t lo = B.flat_off + (int64_t)dst_rank * B.shard_numel;
      const int64_t hi = lo + B.shard_numel;
      while (t < nt && dp->t_bucket[t] < (int32_t)b) ++t;
      for (int32_t u = t; u < nt && dp->t_bucket[u] == (int32_t)b; ++u) {
        const int64_t x0 = std::max(lo, dp->t_off[u]);
        const int64_t x1 = std::min(hi, dp->t_off[u] + dp->t_numel[u]);
        if (x0 >= x1) continue;
        const auto& SB = sp->buckets[sp->t_bucket[u]];
        for (int64_t i = x0 - dp->t_off[u]; i < x1 - dp->t_off[u];) {
          const int64_t rel = sp->t_off[u] + i - SB.flat_off;   // position inside the source bucket
          const int64_t q = rel / SB.shard_numel;
          const int64_t within = rel - q * SB.shard_numel;
          const int64_t n = std::min(x1 - dp->t_off[u] - i, SB.shard_numel - within);
          ents.push_back(zk::CopyEnt{(const char*)src_shards[q] + (SB.shard_off + within) * es,
                                     B.shard_off + (dp->t_off[u] + i - lo), n, 0, 0});
          i += n;
        }
      }
      const int64_t pad_lo = std::max(lo, B.flat_off + B.numel);
      if (pad_lo < hi) ents.push_back(zk::CopyEnt{nullptr, B.shard_off + (pad_lo - lo), hi - pad_lo, 0, 0});
    }
    return run_copies(ents, dst_shard, es, stream);
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_reshard");
  }
}

zero_status zero_shard_reduce(zero_plan_t p, int32_t rank, const zero_grad_src* src,
                              double grad_scale, float* out, void* stream) {
  try {
    if (check_plan(p)) return ZERO_EINVAL;
    if (rank < 0 || rank >= p->n_d) return fail(ZERO_EINVAL, "rank %d outside [0, %d)", rank, p->n_d);
    std::vector<Range> reads;
    bool vec_ok = true;   // base alignment the vector kernel needs
    if (zero_status st = check_src(*p, src, reads, vec_ok)) return st;
    if (!out && p->shard_total > 0) return fail(ZERO_EINVAL, "out is NULL");
    if (!aligned(out, 4)) return fail(ZERO_EINVAL, "out is not 4-byte aligned");
    if (!aligned(out, 16)) vec_ok = false;
    const Range w = range_of(out, p->shard_total, 4, "out");
    for (const auto& r : reads)
      if (overlap(w, r)) return fail(ZERO_EINVAL, "out overlaps a gradient buffer");

    const std::vector<Piece> ps = owner_pieces(*p, rank, false);
    const bool uses_full = src->is_full && std::any_of(src->is_full, src->is_full + src->n, [](uint8_t f) { return f != 0; });
    zk::StepArgs a;
    memset(&a, 0, sizeof a);
    a.out = out;
    a.c[8] = (float)grad_scale;
    if (zero_status st = warm_state(&out, 1, p->shard_total, p->n_d, stream)) return st;
    // Ranks beyond one launch's table: later launches continue from out.
    for (int q0 = 0; q0 < p->n_d; q0 += zk::kMaxRanks) {
      const int n = std::min(zk::kMaxRanks, p->n_d - q0);
      set_ranks(a, *src, q0, n);
      a.flags = (q0 > 0 ? zk::kFlagInitFromOut : 0) | (q0 + n == p->n_d ? zk::kFlagApplyScale : 0);
      if (zero_status st = run_step_all(a, ps, zk::kReduceOnly, src->dtype, ZERO_F16, vec_ok, uses_full, stream))
        return st;
    }
    return ok();
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_shard_reduce");
  }
}

zero_status zero_adam_step(zero_plan_t p, int32_t rank, const zero_adam_hyper* hp, int64_t t,
                           const zero_grad_src* slices, const float* reduced, float* master,
                           float* m, float* v, void* param_dst, zero_dtype param_dt,
                           int32_t dst_is_full, void* stream) {
  try {
    if (check_plan(p)) return ZERO_EINVAL;
    if (rank < 0 || rank >= p->n_d) return fail(ZERO_EINVAL, "rank %d outside [0, %d)", rank, p->n_d);
    if (!hp) return fail(ZERO_EINVAL, "hyper-parameters are NULL");
    if (t < 1) return fail(ZERO_EINVAL, "step t must be >= 1 (got %lld)", (long long)t);
    if (!is16(param_dt)) return fail(ZERO_EUNSUPPORTED, "parameter dtype %d is not 16-bit", (int)param_dt);
    const int64_t S = p->shard_total;
    const int64_t dst_elems = dst_is_full ? p->psi_pad : S;
    std::vector<Range> reads;
    bool vec_ok = true;   // base alignment the vector kernel needs
    if (slices) {
      if (p->n_d > zk::kMaxRanks)
        return fail(ZERO_EUNSUPPORTED, "fused step reads at most %d ranks; use zero_shard_reduce and pass reduced",
                    zk::kMaxRanks);
      if (zero_status st = check_src(*p, slices, reads, vec_ok)) return st;
    } else {
      if (!reduced && S > 0) return fail(ZERO_EINVAL, "both slices and reduced are NULL");
      if (!aligned(reduced, 4)) return fail(ZERO_EINVAL, "reduced is not 4-byte aligned");
      if (!aligned(reduced, 16)) vec_ok = false;
      reads.push_back(range_of(reduced, S, 4, "reduced"));
    }
    float* const st_ptr[3] = {master, m, v};
    const char* st_name[3] = {"master", "m", "v"};
    std::vector<Range> writes;
    for (int i = 0; i < 3; ++i) {
      if (!st_ptr[i] && S > 0) return fail(ZERO_EINVAL, "%s is NULL", st_name[i]);
      if (!aligned(st_ptr[i], 4)) return fail(ZERO_EINVAL, "%s is not 4-byte aligned", st_name[i]);
      if (!aligned(st_ptr[i], 16)) vec_ok = false;
      writes.push_back(range_of(st_ptr[i], S, 4, st_name[i]));
    }
    if (!param_dst && dst_elems > 0) return fail(ZERO_EINVAL, "param_dst is NULL");
    if (!aligned(param_dst, 2)) return fail(ZERO_EINVAL, "param_dst is not 2-byte aligned");
    if (!aligned(param_dst, 8)) vec_ok = false;   // 4 elements (8 bytes) per store
    writes.push_back(range_of(param_dst, dst_elems, 2, "param_dst"));
    for (size_t i = 0; i < writes.size(); ++i) {
      for (size_t j = i + 1; j < writes.size(); ++j)
        if (overlap(writes[i], writes[j]))
          return fail(ZERO_EINVAL, "%s overlaps %s", writes[i].what, writes[j].what);
      for (const auto& r : reads)
        if (overlap(writes[i], r)) return fail(ZERO_EINVAL, "%s overlaps %s", writes[i].what, r.what);
    }

    const std::vector<Piece> ps = owner_pieces(*p, rank, dst_is_full != 0);
    const bool uses_full = slices && slices->is_full &&
                           std::any_of(slices->is_full, slices->is_full + slices->n, [](uint8_t f) { return f != 0; });
    zk::StepArgs a;
    memset(&a, 0, sizeof a);
    adam_consts(*hp, t, a.c);
    a.master = master;
    a.m = m;
    a.v = v;
    a.dst = param_dst;
    if (slices) {
      set_ranks(a, *slices, 0, p->n_d);
      if (zero_status st = warm_state(st_ptr, 3, S, p->n_d, stream)) return st;
      return run_step_all(a, ps, zk::kFused, slices->dtype, param_dt, vec_ok, uses_full, stream);
    }
    a.reduced = reduced;
    a.n_ranks = 0;
    return run_step_all(a, ps, zk::kFromReduced, ZERO_BF16, param_dt, vec_ok, false, stream);
  } catch (const std::bad_alloc&) {
    return fail(ZERO_ENOMEM, "host allocation failed");
  } catch (...) {
    return fail(ZERO_EINVAL, "unexpected failure in zero_adam_step");
  }
}

}  // extern "C"
