// Host-side launch tables of libzero, checked on the CPU.
//
// zero_api.cpp is compiled together with this file, which stands in for the
// two kernel launchers: instead of launching, they replay the kernels' own
// workgroup -> entry/segment indexing over the recorded argument blocks and
// mark every element each launch would touch.  For random plans the test
// checks that every destination element is written exactly once, that every
// source element read lies inside its buffer, and that the step's segments
// tile the owner's shard at the plan's offsets.  Built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer; no GPU is involved.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <map>
#include <utility>
#include <random>
#include <vector>

#include "zero.h"
#include "zero_internal.h"

namespace {

// Fake device address spaces: each buffer gets its own 1 TiB-aligned base so
// an address identifies (buffer, byte offset).
constexpr uint64_t kSpan = 1ull << 40;
uint64_t fake_base(int id) { return (uint64_t)(id + 1) * kSpan; }

struct Buffer {
  int64_t bytes = 0;         // shift + elements * es
  int64_t shift = 0;         // bytes before element 0
  std::vector<uint8_t> writes;   // per element, saturating at 255
  int es = 2;
};
std::map<int, Buffer> g_buf;   // id -> buffer
int g_fail = 0;

#define EXPECT(c, ...)                     \
  do {                                     \
    if (!(c)) {                            \
      if (g_fail < 20) {                   \
        fprintf(stderr, "FAIL: " __VA_ARGS__); \
        fprintf(stderr, "\n");             \
      }                                    \
      ++g_fail;                            \
    }                                      \
  } while (0)

// A buffer of elems elements of es bytes whose element 0 sits shift bytes
// past a 1 TiB boundary (shift breaks 16-byte alignment on purpose).
void* make(int id, int64_t elems, int es, int64_t shift = 0) {
  Buffer& b = g_buf[id];
  b.shift = shift;
  b.bytes = shift + elems * es;
  b.es = es;
  b.writes.assign(elems, 0);
  return (void*)(uintptr_t)(fake_base(id) + shift);
}

int buf_of(uint64_t addr) { return (int)(addr / kSpan) - 1; }

void touch_read(uint64_t addr, int64_t bytes) {
  const int id = buf_of(addr);
  auto it = g_buf.find(id);
  EXPECT(it != g_buf.end(), "read from unknown buffer %d", id);
  if (it == g_buf.end()) return;
  const int64_t off = (int64_t)(addr - fake_base(id));
  EXPECT(off >= it->second.shift && off + bytes <= it->second.bytes, "read out of bounds: buffer %d off %lld len %lld size %lld",
         id, (long long)off, (long long)bytes, (long long)it->second.bytes);
}

void touch_write(uint64_t addr, int64_t elems, int es) {
  const int id = buf_of(addr);
  auto it = g_buf.find(id);
  EXPECT(it != g_buf.end(), "write to unknown buffer %d", id);
  if (it == g_buf.end()) return;
  const int64_t off = (int64_t)(addr - fake_base(id)) - it->second.shift;
  EXPECT(off % es == 0, "misaligned write");
  const int64_t e0 = off / es;
  EXPECT(e0 >= 0 && e0 + elems <= (int64_t)it->second.writes.size(), "write out of bounds: buffer %d", id);
  if (e0 < 0 || e0 + elems > (int64_t)it->second.writes.size()) return;
  uint8_t* w = it->second.writes.data() + e0;
  for (int64_t i = 0; i < elems; ++i) w[i] += w[i] != 255;
}

void expect_all_written_once(int id, const char* what) {
  const auto& w = g_buf[id].writes;  // counts saturate at 255
  for (size_t i = 0; i < w.size(); ++i)
    if (w[i] != 1) {
      EXPECT(false, "%s element %zu written %d times", what, i, (int)w[i]);
      return;
    }
}

struct StepRec {
  zk::StepArgs a;
  int mode, gdt, pdt, ndc, blocks;
  bool vec;
};
std::vector<StepRec> g_steps;

}  // namespace

// ---- stand-ins for the launchers: replay the kernels' indexing ----------
// When set, the next launch "fails" with this HIP error code.
int g_inject_error = 0;

namespace zk {

int launch_copy(const CopyArgs& a, int esz, int n_blocks, void*) {
  if (g_inject_error) {
    const int e = g_inject_error;
    g_inject_error = 0;
    return e;
  }
  // Entry of each block: last entry whose block_start <= block.
  for (int e = 0; e < a.n_ent; ++e) {
    const CopyEnt& en = a.ent[e];
    const int b_end = e + 1 < a.n_ent ? a.ent[e + 1].block_start : n_blocks;
    EXPECT(b_end > en.block_start, "entry with no blocks");
    const uint64_t d0 = (uint64_t)(uintptr_t)a.dst + (uint64_t)en.dst_off * esz;
    const uint64_t d1 = d0 + (uint64_t)en.n * esz;
    const uint64_t u_first = d0 >> 4, u_end = (d1 + 15) >> 4;
    const uint64_t covered = (uint64_t)(b_end - en.block_start) * kThreads * kCopyUnits;
    EXPECT(u_first + covered >= u_end, "copy entry units not covered by its blocks");
    EXPECT(covered < (u_end - u_first) + (uint64_t)kThreads * kCopyUnits, "copy entry has a block too many");
    touch_write(d0, en.n, esz);
    if (en.src) touch_read((uint64_t)(uintptr_t)en.src, en.n * esz);
  }
  EXPECT(a.n_ent <= kMaxCopy, "too many copy entries");
  return 0;
}

// Warm-up reads: recorded, and checked for a consistent workgroup layout.
struct WarmRec {
  WarmArgs a;
  int blocks;
};
std::vector<WarmRec> g_warms;
int launch_warm(const WarmArgs& a, int n_blocks, void*) {
  if (g_inject_error) {
    const int e = g_inject_error;
    g_inject_error = 0;
    return e;
  }
  EXPECT(a.n >= 1 && a.n <= kWarmRanges, "warm-up with %d ranges", a.n);
  int64_t b = 0;
  for (int i = 0; i < a.n; ++i) {
    EXPECT(a.block_start[i] == b, "warm-up range %d starts at workgroup %d, not %lld", i, a.block_start[i], (long long)b);
    EXPECT(a.units[i] > 0 && ((uintptr_t)a.base[i] & 15) == 0, "warm-up range %d empty or misaligned", i);
    b += (a.units[i] + kWarmThreads * kWarmUnits - 1) / (kWarmThreads * kWarmUnits);
  }
  EXPECT(b == n_blocks, "warm-up launches %d workgroups for %lld", n_blocks, (long long)b);
  g_warms.push_back(WarmRec{a, n_blocks});
  return 0;
}

int launch_step(const StepArgs& a, int mode, int gdt, int pdt, int ndc, bool vec, int n_blocks, void*) {
  if (g_inject_error) {
    const int e = g_inject_error;
    g_inject_error = 0;
    return e;
  }
  g_steps.push_back(StepRec{a, mode, gdt, pdt, ndc, n_blocks, vec});
  return 0;
}

const char* hip_error_string(int) { return "stand-in launch error"; }

// Stand-in occupancy: 4 workgroups per CU for the fused kernel, 3 for the
// reduce kernel (arbitrary; the launcher must use whatever it is told), 256 CUs.
int resident_blocks(int mode, int, int, int, bool) { return mode == kFused ? 1024 : 768; }

// Stand-in real-time counter rate (MI355X reports 100 MHz); tests change it.
double g_wall_clock_hz = 1e8;
double wall_clock_hz() { return g_wall_clock_hz; }
// Stand-in HBM peak (MI355X: 2 GHz x 4 x 8192 bits); tests change it.
double g_hbm_peak_bps = 8.192e12;
double hbm_peak_bps() { return g_hbm_peak_bps; }

}  // namespace zk

namespace {

struct Rnd {
  std::mt19937_64 g;
  explicit Rnd(uint64_t s) : g(s) {}
  int64_t pick(std::initializer_list<int64_t> v) { return *(v.begin() + g() % v.size()); }
  int64_t range(int64_t lo, int64_t hi) { return lo + (int64_t)(g() % (uint64_t)(hi - lo)); }
};

struct PlanQ {
  int64_t psi_pad, S;
  int32_t nb, n_d;
  std::vector<int64_t> off, numel, padded, sn, soff;
};

PlanQ query(zero_plan_t p) {
  PlanQ q;
  zero_plan_info(p, &q.psi_pad, &q.S, &q.nb, &q.n_d);
  for (int b = 0; b < q.nb; ++b) {
    int64_t o, n, pd, s, so;
    zero_plan_bucket(p, b, &o, &n, &pd, &s, &so);
    q.off.push_back(o); q.numel.push_back(n); q.padded.push_back(pd); q.sn.push_back(s); q.soff.push_back(so);
  }
  return q;
}

// Replays recorded step launches; returns per-shard-element coverage counts
// and checks every segment against the plan.
// The write window the launcher must have chosen: none for Adam from the
// reduced gradient and for the element kernel; otherwise the forced setting,
// or, automatically, none for launches under 2^23 elements (the large
// automatic cases are checked by value in main).
int64_t g_forced_period = -1, g_forced_open = 0;

void check_window(const StepRec& r) {
  int64_t elems = 0;
  for (int s = 0; s < r.a.n_seg; ++s) elems += r.a.seg[s].len;
  uint32_t p = 0, o = 0;
  if (r.vec && r.mode != zk::kFromReduced) {
    if (g_forced_period >= 0) {
      p = (uint32_t)g_forced_period;
      o = g_forced_period ? (uint32_t)g_forced_open : 0;
    } else if (elems >= (int64_t(1) << 23)) {
      return;
    }
  }
  EXPECT(r.a.win_period == p && r.a.win_open == o, "write window (%u, %u), want (%u, %u)", r.a.win_period,
         r.a.win_open, p, o);
}

std::vector<uint8_t> replay_steps(const PlanQ& q, int rank, bool dst_full, uint64_t dst, int dst_es) {
  std::vector<uint8_t> hits(q.S, 0);
  for (const StepRec& r : g_steps) {
    check_window(r);
    const int per_block = r.vec ? zk::kStepThreads * zk::kStepVec : zk::kThreads;
    EXPECT(r.a.n_seg >= 1 && r.a.n_seg <= zk::kMaxSeg, "segment count");
    EXPECT(r.a.n_ranks >= 0 && r.a.n_ranks <= zk::kMaxRanks, "rank count");
    for (int s = 0; s < r.a.n_seg; ++s) {
      const zk::StepSeg& g = r.a.seg[s];
      const int b_end = s + 1 < r.a.n_seg ? r.a.seg[s + 1].block_start : r.blocks;
      EXPECT((int64_t)(b_end - g.block_start) * per_block >= g.len, "segment not covered by its blocks");
      EXPECT((int64_t)(b_end - g.block_start - 1) * per_block < g.len, "segment has a block too many");
      EXPECT(g.len >= 1 && g.len <= zk::kSegMaxElems, "segment length %d", g.len);
      if (r.vec) {
        bool any_full = false;
        for (int k = 0; k < r.a.n_ranks; ++k) any_full |= ((r.a.full_mask[k >> 5] >> (k & 31)) & 1u) != 0;
        const bool uses_dst = r.mode != zk::kReduceOnly;
        EXPECT((g.shard_off & 3) == 0 && (!uses_dst || (g.dst_off & 3) == 0) && (!any_full || (g.full_off & 3) == 0),
               "vector segment offsets not multiples of 4 elements");
      }
      int b = -1;
      for (int k = 0; k < q.nb; ++k)
        if (g.shard_off >= q.soff[k] && g.shard_off + g.len <= q.soff[k] + q.sn[k]) b = k;
      EXPECT(b >= 0, "segment not inside one bucket");
      if (b < 0) continue;
      const int64_t own = q.off[b] + (int64_t)rank * q.sn[b] + (g.shard_off - q.soff[b]);
      EXPECT(g.full_off == own, "full_off %lld != owner range %lld", (long long)g.full_off, (long long)own);
      EXPECT(g.dst_off == (dst_full ? own : g.shard_off), "dst_off wrong");
      for (int64_t i = 0; i < g.len; ++i) hits[g.shard_off + i] += hits[g.shard_off + i] != 255;
      touch_write(dst + (uint64_t)g.dst_off * dst_es, g.len, dst_es);
      for (int k = 0; k < r.a.n_ranks; ++k) {
        const bool full = (r.a.full_mask[k >> 5] >> (k & 31)) & 1u;
        touch_read((uint64_t)(uintptr_t)r.a.grad[k] + (full ? g.full_off : g.shard_off) * 2, g.len * 2);
      }
      if (r.mode == zk::kFromReduced) touch_read((uint64_t)(uintptr_t)r.a.reduced + g.shard_off * 4, g.len * 4);
      if (r.mode != zk::kReduceOnly)
        for (const float* x : {r.a.master, r.a.m, r.a.v}) touch_read((uint64_t)(uintptr_t)x + g.shard_off * 4, g.len * 4);
    }
  }
  return hits;
}

void expect_hits(const std::vector<uint8_t>& hits, int want, const char* what) {
  for (size_t j = 0; j < hits.size(); ++j)
    if (hits[j] != want) {
      EXPECT(false, "%s: shard element %zu covered %d times, want %d", what, j, (int)hits[j], want);
      return;
    }
}

void check_step(zero_plan_t p, int rank, bool dst_full, bool use_full_grads, int64_t shift) {
  const PlanQ q = query(p);
  g_buf.clear();
  g_steps.clear();
  const bool fused = q.n_d <= ZERO_MAX_RANKS;
  std::vector<const void*> ptrs(q.n_d);
  std::vector<uint8_t> isf(q.n_d);
  for (int r = 0; r < q.n_d; ++r) {
    isf[r] = use_full_grads && (r % 2 == 0);
    ptrs[r] = make(100 + r, isf[r] ? q.psi_pad : q.S, 2);
  }
  float* w = (float*)make(1, q.S, 4, shift);
  float* m = (float*)make(2, q.S, 4);
  float* v = (float*)make(3, q.S, 4);
  void* dst = make(4, dst_full ? q.psi_pad : q.S, 2);
  const float* red = fused ? nullptr : (const float*)make(5, q.S, 4);
  zero_grad_src src = {ZERO_BF16, q.n_d, ptrs.data(), isf.data()};
  zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 0.5};
  const zero_status st = zero_adam_step(p, rank, &hp, 3, fused ? &src : nullptr, red, w, m, v, dst, ZERO_F16,
                                        dst_full ? 1 : 0, nullptr);
  EXPECT(st == ZERO_OK, "zero_adam_step failed: %s", zero_last_error());
  for (const StepRec& r : g_steps) {
    EXPECT(r.mode == (fused ? zk::kFused : zk::kFromReduced), "step mode");
    if (shift) EXPECT(!r.vec, "vector kernel chosen for a misaligned buffer");
    if (fused) {
      EXPECT(r.a.n_ranks == q.n_d, "fused launch has %d ranks", r.a.n_ranks);
      for (int k = 0; k < q.n_d; ++k) {
        EXPECT(r.a.grad[k] == ptrs[k], "rank %d pointer", k);
        EXPECT((bool)((r.a.full_mask[k >> 5] >> (k & 31)) & 1u) == (bool)isf[k], "rank %d full flag", k);
      }
    }
  }
  expect_hits(replay_steps(q, rank, dst_full, (uint64_t)(uintptr_t)dst, 2), 1, "adam step");
  if (dst_full) {
    // Only the owner's ranges of the full buffer are written, each once.
    const auto& wr = g_buf[4].writes;
    for (int k = 0; k < q.nb; ++k)
      for (int64_t i = 0; i < q.padded[k]; ++i) {
        const int64_t pos = q.off[k] + i;
        const bool owned = i >= (int64_t)rank * q.sn[k] && i < (int64_t)(rank + 1) * q.sn[k];
        if (wr[pos] != (owned ? 1 : 0)) {
          EXPECT(false, "full buffer element %lld written %d times (owned %d)", (long long)pos, (int)wr[pos], owned);
          k = q.nb;
          break;
        }
      }
  } else {
    expect_all_written_once(4, "shard destination");
  }
}

// zero_shard_reduce: one pass per group of up to 128 ranks, each covering the
// shard once; the first pass starts the fold, later ones continue it from the
// output, and only the last applies the scale.
void check_reduce(zero_plan_t p, int rank, int64_t shift) {
  const PlanQ q = query(p);
  g_buf.clear();
  g_steps.clear();
  std::vector<const void*> ptrs(q.n_d);
  for (int r = 0; r < q.n_d; ++r) ptrs[r] = make(100 + r, q.S, 2, r == 1 ? shift : 0);
  float* out = (float*)make(1, q.S, 4);
  zero_grad_src src = {ZERO_F16, q.n_d, ptrs.data(), nullptr};
  EXPECT(zero_shard_reduce(p, rank, &src, 0.25, out, nullptr) == ZERO_OK, "reduce failed: %s", zero_last_error());
  const int groups = (q.n_d + zk::kMaxRanks - 1) / zk::kMaxRanks;
  int ranks_seen = 0, last_group = -1;
  for (const StepRec& r : g_steps) {
    EXPECT(r.mode == zk::kReduceOnly, "reduce mode");
    if (shift % 8 && q.n_d > 1) EXPECT(!r.vec, "vector kernel chosen for a gradient not 8-byte aligned");
    const int g0 = (int)(std::find(ptrs.begin(), ptrs.end(), r.a.grad[0]) - ptrs.begin());
    EXPECT(g0 % zk::kMaxRanks == 0, "group starts at rank %d", g0);
    const int grp = g0 / zk::kMaxRanks;
    if (grp != last_group) ranks_seen += r.a.n_ranks, last_group = grp;
    EXPECT(r.a.n_ranks == std::min(zk::kMaxRanks, q.n_d - g0), "group size");
    for (int k = 0; k < r.a.n_ranks; ++k) EXPECT(r.a.grad[k] == ptrs[g0 + k], "group rank pointer");
    EXPECT(((r.a.flags & zk::kFlagInitFromOut) != 0) == (grp > 0), "init-from-out flag");
    EXPECT(((r.a.flags & zk::kFlagApplyScale) != 0) == (grp == groups - 1), "scale flag");
    EXPECT(r.a.c[8] == 0.25f, "scale constant");
  }
  EXPECT(q.S == 0 || ranks_seen == q.n_d, "ranks folded %d of %d", ranks_seen, q.n_d);
  expect_hits(replay_steps(q, rank, false, (uint64_t)(uintptr_t)out, 4), groups, "reduce");
}

void check_copies(zero_plan_t p, const std::vector<int64_t>& sizes, Rnd& rnd) {
  const PlanQ q = query(p);
  const int es = rnd.pick({2, 4}) == 2 ? 2 : 4;
  const zero_dtype dt = es == 2 ? ZERO_BF16 : ZERO_F32;
  // flatten: tensors (possibly misaligned by whole elements) -> flat
  g_buf.clear();
  std::vector<const void*> tens(sizes.size());
  for (size_t t = 0; t < sizes.size(); ++t) {
    char* base = (char*)make(200 + (int)t, sizes[t] + 8, es);
    tens[t] = sizes[t] ? base + es * rnd.range(0, 8) : nullptr;
  }
  void* flat = make(1, q.psi_pad, es);
  EXPECT(zero_flatten(p, tens.data(), dt, flat, nullptr, 0, nullptr) == ZERO_OK, "flatten failed: %s", zero_last_error());
  expect_all_written_once(1, "flat");
  // gather_pack: shards -> full
  g_buf.clear();
  std::vector<const void*> sh(q.n_d);
  for (int r = 0; r < q.n_d; ++r) sh[r] = make(300 + r, q.S, es);
  void* full = make(2, q.psi_pad, es);
  EXPECT(zero_gather_pack(p, sh.data(), dt, full, nullptr) == ZERO_OK, "gather failed: %s", zero_last_error());
  expect_all_written_once(2, "full");
}

void check_reshard(const std::vector<int64_t>& sizes, int64_t psi, Rnd& rnd) {
  zero_plan_t a, b;
  const int na = (int)rnd.pick({1, 2, 3, 4, 8, 16, 64}), nb = (int)rnd.pick({1, 2, 3, 5, 16});
  zero_plan(psi, na, sizes.data(), (int32_t)sizes.size(), rnd.pick({0, 7, 64, 1000}), (int32_t)rnd.pick({1, 8, 64}), &a);
  zero_plan(psi, nb, sizes.data(), (int32_t)sizes.size(), rnd.pick({0, 9, 500}), (int32_t)rnd.pick({1, 4, 64}), &b);
  const PlanQ qa = query(a), qb = query(b);
  for (int r = 0; r < nb; ++r) {
    g_buf.clear();
    std::vector<const void*> sh(na);
    for (int k = 0; k < na; ++k) sh[k] = make(400 + k, qa.S, 4);
    void* out = make(1, qb.S, 4);
    EXPECT(zero_reshard(a, b, r, sh.data(), ZERO_F32, out, nullptr) == ZERO_OK, "reshard failed: %s",
           zero_last_error());
    expect_all_written_once(1, "reshard destination");
  }
  zero_plan_destroy(a);
  zero_plan_destroy(b);
}

}  // namespace

int main() {
  Rnd rnd(12345);
  int cases = 0;
  for (int it = 0; it < 300; ++it) {
    const int nt = (int)rnd.range(0, 12);
    std::vector<int64_t> sizes(nt);
    int64_t psi = 0;
    for (auto& s : sizes) {
      s = rnd.pick({0, 1, 3, 8, 17, 64, 100, 1000, 4099});
      psi += s;
    }
    const int n_d = (int)rnd.pick({1, 2, 3, 4, 5, 8, 16, 64, 130});
    zero_plan_t p;
    if (zero_plan(psi, n_d, sizes.data(), nt, rnd.pick({0, 1, 50, 1000, 100000}), (int32_t)rnd.pick({1, 8, 64}),
                  &p) != ZERO_OK) {
      EXPECT(false, "plan failed: %s", zero_last_error());
      continue;
    }
    const PlanQ q = query(p);
    const int rank = (int)rnd.range(0, n_d);
    check_step(p, rank, rnd.g() & 1, rnd.g() & 1, (rnd.g() % 4 == 0) ? 4 : 0);
    check_reduce(p, rank, rnd.pick({0, 0, 2, 8}));
    check_copies(p, sizes, rnd);
    if (nt) check_reshard(sizes, psi, rnd);
    zero_plan_destroy(p);
    ++cases;
    (void)q;
  }
  // A failed launch surfaces as ZERO_EHIP with the runtime's message, from
  // the step, the reduction and the copies alike.
  {
    std::vector<int64_t> sizes = {5000, 3000};
    zero_plan_t p;
    zero_plan(8000, 4, sizes.data(), 2, 0, 8, &p);
    const PlanQ q = query(p);
    std::vector<const void*> ptrs(4);
    for (int r = 0; r < 4; ++r) ptrs[r] = (const void*)(uintptr_t)fake_base(100 + r);
    zero_grad_src src = {ZERO_BF16, 4, ptrs.data(), nullptr};
    zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 0.25};
    g_inject_error = 700;
    EXPECT(zero_adam_step(p, 1, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                          (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                          (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_EHIP,
           "step launch error not reported");
    EXPECT(strstr(zero_last_error(), "stand-in launch error") && strstr(zero_last_error(), "700"),
           "step launch error text: %s", zero_last_error());
    g_inject_error = 701;
    EXPECT(zero_shard_reduce(p, 0, &src, 0.25, (float*)(uintptr_t)fake_base(5), nullptr) == ZERO_EHIP,
           "reduce launch error not reported");
    std::vector<const void*> sh(4);
    for (int r = 0; r < 4; ++r) sh[r] = (const void*)(uintptr_t)fake_base(300 + r);
    g_inject_error = 702;
    EXPECT(zero_gather_pack(p, sh.data(), ZERO_BF16, (void*)(uintptr_t)fake_base(6), nullptr) == ZERO_EHIP,
           "copy launch error not reported");
    EXPECT(strstr(zero_last_error(), "702") != nullptr, "copy launch error text: %s", zero_last_error());
    EXPECT(g_inject_error == 0, "error not consumed");
    (void)q;
    zero_plan_destroy(p);
  }
  // Write-window setting: range checks, forced values reach every fused and
  // reduce launch, and -1 restores the automatic choice.
  EXPECT(zero_set_write_window(-2, 0) == ZERO_EINVAL, "period -2 accepted");
  EXPECT(zero_set_stream_write_window(nullptr, -3, 0) == ZERO_EINVAL, "stream period -3 accepted");
  EXPECT(zero_set_stream_write_window(nullptr, 100, 101) == ZERO_EINVAL, "stream open > period accepted");
  EXPECT(zero_set_write_window(100001, 1) == ZERO_EINVAL, "period above 1 ms accepted");
  EXPECT(zero_set_write_window(100, 0) == ZERO_EINVAL, "open 0 accepted");
  EXPECT(zero_set_write_window(100, 101) == ZERO_EINVAL, "open > period accepted");
  for (const auto& pw : {std::pair<int64_t, int64_t>{400, 100}, {0, 0}, {100000, 100000}, {-1, 0}}) {
    EXPECT(zero_set_write_window(pw.first, pw.second) == ZERO_OK, "window setting refused");
    g_forced_period = pw.first;
    g_forced_open = pw.second;
    std::vector<int64_t> sizes = {4096, 800, 64 * 40};
    zero_plan_t p;
    zero_plan(sizes[0] + sizes[1] + sizes[2], 40, sizes.data(), 3, 0, 8, &p);
    check_step(p, 5, true, false, 0);
    check_step(p, 6, false, true, 4);
    check_reduce(p, 7, 0);
    zero_plan_destroy(p);
  }
  // The automatic window of a large launch: 64 ranks, 2^26 + 4096 elements
  // per shard, 16 generations of resident workgroups (only the tables are
  // built; no memory behind the pointers).
  {
    std::vector<int64_t> sizes = {((int64_t)1 << 26) * 64 + 4096 * 64};
    zero_plan_t p;
    zero_plan(sizes[0], 64, sizes.data(), 1, 0, 64, &p);
    g_steps.clear();
    const PlanQ q = query(p);
    std::vector<const void*> ptrs(64);
    for (int r = 0; r < 64; ++r) ptrs[r] = (const void*)(uintptr_t)fake_base(100 + r);
    zero_grad_src src = {ZERO_BF16, 64, ptrs.data(), nullptr};
    zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 1.0 / 64};
    EXPECT(zero_adam_step(p, 3, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                          (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                          (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
           "large step failed: %s", zero_last_error());
    // 1024 resident workgroups x 4096 elements x 154 bytes at 6.5 TB/s, times
    // 0.62, in 10 ns ticks: 6161; open for the written 14/154 of it: 560.
    EXPECT(g_steps.size() == 1 && g_steps[0].a.win_period == 6161 && g_steps[0].a.win_open == 560,
           "automatic window of a large fused launch: (%u, %u)", g_steps.empty() ? 0u : g_steps[0].a.win_period,
           g_steps.empty() ? 0u : g_steps[0].a.win_open);
    EXPECT(zero_adam_step(p, 3, &hp, 1, nullptr, (const float*)(uintptr_t)fake_base(5),
                          (float*)(uintptr_t)fake_base(1), (float*)(uintptr_t)fake_base(2),
                          (float*)(uintptr_t)fake_base(3), (void*)(uintptr_t)fake_base(4), ZERO_F16, 1,
                          nullptr) == ZERO_OK, "large from-reduced step failed: %s", zero_last_error());
    EXPECT(g_steps.size() == 2 && g_steps[1].a.win_period == 0, "window on Adam from the reduced gradient");
    // The reduction: 768 resident x 4096 x 132 bytes at the reduce-only share
    // of 0.45 -> 2874 ticks, open 1/16.
    zero_grad_src src16 = {ZERO_BF16, 64, ptrs.data(), nullptr};
    EXPECT(zero_shard_reduce(p, 3, &src16, 1.0 / 64, (float*)(uintptr_t)fake_base(5), nullptr) == ZERO_OK,
           "large reduce failed: %s", zero_last_error());
    EXPECT(g_steps.size() == 3 && g_steps[2].a.win_period == 2874 && g_steps[2].a.win_open == 179,
           "automatic window of a large reduce launch: (%u, %u)", g_steps.size() < 3 ? 0u : g_steps[2].a.win_period,
           g_steps.size() < 3 ? 0u : g_steps[2].a.win_open);
    // Three generations of resident workgroups (3 x 1024 x 4096 elements):
    // half the period, 3080 ticks, open 280.
    {
      std::vector<int64_t> s3 = {(int64_t)3 * 1024 * 4096 * 64};
      zero_plan_t p3;
      zero_plan(s3[0], 64, s3.data(), 1, 0, 64, &p3);
      g_steps.clear();
      EXPECT(zero_adam_step(p3, 1, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                            (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                            (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
             "3-generation step failed: %s", zero_last_error());
      EXPECT(g_steps.size() == 1 && g_steps[0].a.win_period == 3080 && g_steps[0].a.win_open == 280,
             "automatic window of a 3-generation launch: (%u, %u)", g_steps.empty() ? 0u : g_steps[0].a.win_period,
             g_steps.empty() ? 0u : g_steps[0].a.win_open);
      zero_plan_destroy(p3);
    }
    // Between 6 and 12 generations the period ramps from half to full: 8
    // generations take 2/3 of it, 4107 ticks, open 373.  Other rank counts at
    // 16 generations: the kernel for N_d = 32 (not compiled in) writes 14/90 of
    // its bytes, above 12%, so it opens for 1.5 times that share; N_d = 48
    // writes 14/122, below, and N_d = 16 (compiled in) keeps its written share
    // and takes 0.74 of a generation for its period instead of 0.62.
    {
      struct Case {
        int32_t n_d;
        int64_t shard;
        uint32_t period, open;
        const char* what;
      };
      const Case cases[] = {{64, (int64_t)8 * 1024 * 4096, 4107, 373, "8-generation launch"},
                            {32, (int64_t)16 * 1024 * 4096, 3600, 840, "N_d = 32 launch"},
                            {48, (int64_t)16 * 1024 * 4096, 4880, 560, "N_d = 48 launch"},
                            {16, (int64_t)16 * 1024 * 4096, 2769, 668, "N_d = 16 launch"}};
      for (const Case& c : cases) {
        std::vector<int64_t> sz = {c.shard * c.n_d};
        zero_plan_t pc;
        zero_plan(sz[0], c.n_d, sz.data(), 1, 0, 64, &pc);
        zero_grad_src srcc = {ZERO_BF16, c.n_d, ptrs.data(), nullptr};
        g_steps.clear();
        EXPECT(zero_adam_step(pc, 1, &hp, 1, &srcc, nullptr, (float*)(uintptr_t)fake_base(1),
                              (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                              (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
               "%s failed: %s", c.what, zero_last_error());
        EXPECT(g_steps.size() == 1 && g_steps[0].a.win_period == c.period && g_steps[0].a.win_open == c.open,
               "automatic window of a %s: (%u, %u)", c.what, g_steps.empty() ? 0u : g_steps[0].a.win_period,
               g_steps.empty() ? 0u : g_steps[0].a.win_open);
        zero_plan_destroy(pc);
      }
    }
    // Few ranks: no automatic window.
    std::vector<int64_t> s8 = {((int64_t)1 << 25) * 8};
    zero_plan_t p8;
    zero_plan(s8[0], 8, s8.data(), 1, 0, 64, &p8);
    zero_grad_src src8 = {ZERO_BF16, 8, ptrs.data(), nullptr};
    g_steps.clear();
    EXPECT(zero_adam_step(p8, 0, &hp, 1, &src8, nullptr, (float*)(uintptr_t)fake_base(1),
                          (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                          (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
           "n_d=8 step failed: %s", zero_last_error());
    EXPECT(g_steps.size() == 1 && g_steps[0].a.win_period == 0, "automatic window with 8 ranks");
    zero_plan_destroy(p8);
    (void)q;
    zero_plan_destroy(p);
  }
  // Warm-up read (zero_set_warm_read): off by default; when on, only when the
  // launch reads >= 1 GiB of gradients and the buffers are 16-byte aligned;
  // 256 MiB of the fused step's state (master first) or of the reduction's
  // output; never before Adam from the reduced gradient.
  {
    zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 1.0 / 64};
    std::vector<const void*> ptrs(64);
    for (int r = 0; r < 64; ++r) ptrs[r] = (const void*)(uintptr_t)fake_base(100 + r);
    auto warms_for = [&](int32_t n_d, int64_t shard, uint64_t state_shift) {
      std::vector<int64_t> sz = {shard * n_d};
      zero_plan_t pw;
      zero_plan(sz[0], n_d, sz.data(), 1, 0, 64, &pw);
      zero_grad_src sw = {ZERO_BF16, n_d, ptrs.data(), nullptr};
      zk::g_warms.clear();
      g_steps.clear();
      EXPECT(zero_adam_step(pw, 0, &hp, 1, &sw, nullptr, (float*)(uintptr_t)(fake_base(1) + state_shift),
                            (float*)(uintptr_t)(fake_base(2) + state_shift),
                            (float*)(uintptr_t)(fake_base(3) + state_shift), (void*)(uintptr_t)fake_base(4),
                            ZERO_F16, 1, nullptr) == ZERO_OK,
             "warm-up case step failed: %s", zero_last_error());
      zero_plan_destroy(pw);
      return zk::g_warms;
    };
    // Off by default; 0 and 1 only.
    EXPECT(warms_for(64, (int64_t)1 << 26, 0).empty(), "warm-up read on by default");
    EXPECT(zero_set_warm_read(2) == ZERO_EINVAL && zero_set_warm_read(-1) == ZERO_EINVAL, "warm-up setting 2 or -1 accepted");
    EXPECT(zero_set_warm_read(1) == ZERO_OK, "warm-up setting refused");
    // 7.5B-like: 64 ranks x 2^26 elements (8.6 GB of gradients): 256 MiB of master only.
    auto w1 = warms_for(64, (int64_t)1 << 26, 0);
    EXPECT(w1.size() == 1 && w1[0].a.n == 1 && w1[0].a.base[0] == (const void*)(uintptr_t)fake_base(1) &&
               w1[0].a.units[0] == ((int64_t)256 << 20) / 16 && w1[0].blocks == 2048,
           "warm-up of a large launch: %zu launches", w1.size());
    // A Stage-3 layer (64 x 12,584,576; 1.6 GB of gradients): all of master, m and v (151 MB).
    auto w2 = warms_for(64, 12584576, 0);
    EXPECT(w2.size() == 1 && w2[0].a.n == 3 && w2[0].a.units[0] == (int64_t)12584576 * 4 / 16 &&
               w2[0].a.units[2] == (int64_t)12584576 * 4 / 16 &&
               w2[0].a.base[2] == (const void*)(uintptr_t)fake_base(3),
           "warm-up of a Stage-3 layer: %zu launches", w2.size());
    // Small launches (8 ranks x 15.5M elements: 0.25 GB) and misaligned state: none.
    EXPECT(warms_for(8, 15456576, 0).empty(), "warm-up of a small launch");
    EXPECT(warms_for(64, (int64_t)1 << 26, 4).empty(), "warm-up with state not 16-byte aligned");
    // The warm-up's launch error is reported, and no step is launched after it.
    g_inject_error = 703;
    {
      std::vector<int64_t> sz = {((int64_t)1 << 26) * 64};
      zero_plan_t pw;
      zero_plan(sz[0], 64, sz.data(), 1, 0, 64, &pw);
      zero_grad_src sw = {ZERO_BF16, 64, ptrs.data(), nullptr};
      g_steps.clear();
      EXPECT(zero_adam_step(pw, 0, &hp, 1, &sw, nullptr, (float*)(uintptr_t)fake_base(1),
                            (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                            (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_EHIP &&
                 g_steps.empty(),
             "warm-up launch error not reported");
      // The reduction warms up 256 MiB of its own output; Adam from the
      // reduced gradient (whose input the library wrote non-temporally) does not.
      zk::g_warms.clear();
      EXPECT(zero_shard_reduce(pw, 0, &sw, 1.0 / 64, (float*)(uintptr_t)fake_base(5), nullptr) == ZERO_OK,
             "reduce failed: %s", zero_last_error());
      EXPECT(zk::g_warms.size() == 1 && zk::g_warms[0].a.n == 1 &&
                 zk::g_warms[0].a.base[0] == (const void*)(uintptr_t)fake_base(5) &&
                 zk::g_warms[0].a.units[0] == ((int64_t)256 << 20) / 16,
             "warm-up before the reduction: %zu launches", zk::g_warms.size());
      zk::g_warms.clear();
      EXPECT(zero_adam_step(pw, 0, &hp, 1, nullptr, (const float*)(uintptr_t)fake_base(5),
                            (float*)(uintptr_t)fake_base(1), (float*)(uintptr_t)fake_base(2),
                            (float*)(uintptr_t)fake_base(3), (void*)(uintptr_t)fake_base(4), ZERO_F16, 1,
                            nullptr) == ZERO_OK, "from-reduced step failed: %s", zero_last_error());
      EXPECT(zk::g_warms.empty(), "warm-up before Adam from the reduced gradient");
      zero_plan_destroy(pw);
    }
    EXPECT(zero_set_warm_read(0) == ZERO_OK, "warm-up setting refused");
    EXPECT(warms_for(64, (int64_t)1 << 26, 0).empty(), "warm-up read after turning it off");
  }
  // Scope of the setting: a stream's own setting wins on that stream only;
  // -2 returns the stream to the process-wide default.
  {
    std::vector<int64_t> sizes = {((int64_t)1 << 26) * 64};
    zero_plan_t p;
    zero_plan(sizes[0], 64, sizes.data(), 1, 0, 64, &p);
    std::vector<const void*> ptrs(64);
    for (int r = 0; r < 64; ++r) ptrs[r] = (const void*)(uintptr_t)fake_base(100 + r);
    zero_grad_src src = {ZERO_BF16, 64, ptrs.data(), nullptr};
    zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 1.0 / 64};
    void* sa = (void*)(uintptr_t)0x1000;
    void* sb = (void*)(uintptr_t)0x2000;
    auto window_on = [&](void* stream) {
      g_steps.clear();
      EXPECT(zero_adam_step(p, 0, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                            (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                            (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, stream) == ZERO_OK,
             "scoped step failed: %s", zero_last_error());
      return g_steps.empty() ? std::pair<uint32_t, uint32_t>{~0u, ~0u}
                             : std::pair<uint32_t, uint32_t>{g_steps[0].a.win_period, g_steps[0].a.win_open};
    };
    const auto automatic = window_on(sa);
    EXPECT(automatic.first > 0, "no automatic window on a large launch");
    EXPECT(zero_set_stream_write_window(sa, 0, 0) == ZERO_OK, "stream setting refused");
    EXPECT(zero_set_stream_write_window(nullptr, 3000, 300) == ZERO_OK, "null-stream setting refused");
    EXPECT(window_on(sa) == std::make_pair(0u, 0u), "stream A: own setting (off) not used");
    EXPECT(window_on(sb) == automatic, "stream B: changed by stream A's setting");
    EXPECT(window_on(nullptr) == std::make_pair(3000u, 300u), "default stream: own setting not used");
    EXPECT(zero_set_write_window(0, 0) == ZERO_OK, "default setting refused");
    EXPECT(window_on(sb) == std::make_pair(0u, 0u), "stream B: process default not followed");
    EXPECT(zero_set_stream_write_window(sa, 5000, 500) == ZERO_OK, "stream update refused");
    EXPECT(window_on(sa) == std::make_pair(5000u, 500u), "stream A: updated setting not used");
    EXPECT(zero_set_stream_write_window(sa, -2, 0) == ZERO_OK, "stream reset refused");
    EXPECT(zero_set_stream_write_window(nullptr, -2, 0) == ZERO_OK, "null-stream reset refused");
    EXPECT(window_on(sa) == std::make_pair(0u, 0u), "stream A: not back on the default");
    EXPECT(zero_set_write_window(-1, 0) == ZERO_OK, "automatic default refused");
    EXPECT(window_on(sa) == automatic && window_on(nullptr) == automatic, "not back to automatic");
    // The automatic period follows the counter rate the device reports: the
    // same launch at 50, 100 and 200 MHz takes 3080, 6161 and 12322 ticks
    // (1024 resident x 4096 elements x 154 B at 6.5 TB/s, times 0.62); no rate,
    // no window.
    const double rates[3] = {5e7, 1e8, 2e8};
    const uint32_t want_p[3] = {3080, 6161, 12322}, want_o[3] = {280, 560, 1120};
    for (int i = 0; i < 3; ++i) {
      zk::g_wall_clock_hz = rates[i];
      EXPECT(window_on(sb) == std::make_pair(want_p[i], want_o[i]), "automatic window at %.0f Hz: (%u, %u)",
             rates[i], window_on(sb).first, window_on(sb).second);
    }
    zk::g_wall_clock_hz = 0;
    EXPECT(window_on(sb) == std::make_pair(0u, 0u), "automatic window without a counter rate");
    zk::g_wall_clock_hz = 1e8;
    zero_plan_destroy(p);
  }
  // The plain Psi / N_d layout (align 1) of the 7.5B workload: every owner's
  // shard of 117,187,500 elements starts at a multiple of 4, so each runs
  // entirely in the vector kernel (tables only, no memory behind them).
  {
    std::vector<int64_t> sizes = {7500000000LL};
    zero_plan_t p;
    zero_plan(sizes[0], 64, sizes.data(), 1, 0, 1, &p);
    int64_t S = 0;
    zero_plan_info(p, nullptr, &S, nullptr, nullptr);
    EXPECT(S == 117187500, "align-1 shard %lld", (long long)S);
    // The 64 slices as rows of one [64, S] bf16 tensor: every other row starts
    // 8 bytes past a 16-byte boundary, which the vector kernel accepts.
    std::vector<const void*> ptrs(64);
    for (int r = 0; r < 64; ++r) ptrs[r] = (const void*)(uintptr_t)(fake_base(100) + (uint64_t)r * S * 2);
    EXPECT(((uintptr_t)ptrs[1] & 15) == 8, "row 1 of the slice tensor should be 8 bytes off");
    zero_grad_src src = {ZERO_BF16, 64, ptrs.data(), nullptr};
    zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 1.0 / 64};
    for (int owner : {0, 1, 63}) {
      g_steps.clear();
      EXPECT(zero_adam_step(p, owner, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                            (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                            (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
             "align-1 step failed: %s", zero_last_error());
      int64_t vec_elems = 0;
      bool all_vec = true;
      for (const auto& r : g_steps) {
        all_vec &= r.vec;
        for (int k = 0; k < r.a.n_seg; ++k) vec_elems += r.vec ? r.a.seg[k].len : 0;
      }
      EXPECT(all_vec && vec_elems == S, "align-1 owner %d: %lld of %lld elements in the vector kernel", owner,
             (long long)vec_elems, (long long)S);
    }
    // The same with the reduction, whose output is fp32 and 16-byte aligned.
    g_steps.clear();
    EXPECT(zero_shard_reduce(p, 5, &src, 1.0 / 64, (float*)(uintptr_t)fake_base(5), nullptr) == ZERO_OK,
           "align-1 reduce failed: %s", zero_last_error());
    EXPECT(g_steps.size() == 1 && g_steps[0].vec, "align-1 reduce not in the vector kernel");
    // A 16-bit destination only 8-byte aligned is fine too; an fp32 state
    // array 8 bytes off is not.
    g_steps.clear();
    EXPECT(zero_adam_step(p, 0, &hp, 1, &src, nullptr, (float*)(uintptr_t)fake_base(1),
                          (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                          (void*)(uintptr_t)(fake_base(4) + 8), ZERO_F16, 1, nullptr) == ZERO_OK,
           "8-byte destination: %s", zero_last_error());
    EXPECT(!g_steps.empty() && g_steps[0].vec, "8-byte aligned destination refused by the vector kernel");
    g_steps.clear();
    EXPECT(zero_adam_step(p, 0, &hp, 1, &src, nullptr, (float*)(uintptr_t)(fake_base(1) + 8),
                          (float*)(uintptr_t)fake_base(2), (float*)(uintptr_t)fake_base(3),
                          (void*)(uintptr_t)fake_base(4), ZERO_F16, 1, nullptr) == ZERO_OK,
           "8-byte master: %s", zero_last_error());
    EXPECT(!g_steps.empty() && !g_steps[0].vec, "fp32 state 8 bytes off given to the vector kernel");
    zero_plan_destroy(p);
  }
  // A plan whose padded layout would overflow int64 byte offsets is refused.
  {
    std::vector<int64_t> sizes = {1, 1, 1, 1, 1};
    zero_plan_t p = nullptr;
    EXPECT(zero_plan(5, 1 << 30, sizes.data(), 5, 1, 1 << 30, &p) == ZERO_EINVAL && p == nullptr,
           "overflowing padded layout accepted");
    EXPECT(strstr(zero_last_error(), "padded layout") != nullptr, "overflow error text: %s", zero_last_error());
    EXPECT(zero_plan(5, 1 << 20, sizes.data(), 5, 1, 1 << 10, &p) == ZERO_OK && p != nullptr,
           "large but valid padded layout refused: %s", zero_last_error());
    zero_plan_destroy(p);
  }
  // More buckets than one launch's segment table.
  {
    std::vector<int64_t> sizes(300);
    for (size_t i = 0; i < sizes.size(); ++i) sizes[i] = 8 + (int64_t)(i % 7) * 24;
    int64_t psi = 0;
    for (auto s : sizes) psi += s;
    zero_plan_t p;
    zero_plan(psi, 3, sizes.data(), (int32_t)sizes.size(), 1, 8, &p);
    check_step(p, 2, true, true, 0);
    check_reduce(p, 1, 0);
    check_copies(p, sizes, rnd);
    zero_plan_destroy(p);
  }
  // A bucket whose shard is longer than 2^28 elements: split into pieces.
  {
    std::vector<int64_t> sizes = {((int64_t)1 << 28) + 40, 5, 1000};
    zero_plan_t p;
    zero_plan(sizes[0] + sizes[1] + sizes[2], 1, sizes.data(), 3, 0, 64, &p);
    check_step(p, 0, true, false, 0);
    check_reduce(p, 0, 0);
    zero_plan_destroy(p);
  }
  printf("%d random plans checked, %d failures\n", cases, g_fail);
  return g_fail ? 1 : 0;
}
