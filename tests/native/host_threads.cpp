// libzero's host code called from many threads at once, under
// ThreadSanitizer.  zero_api.cpp is compiled with stand-in launchers that
// only count launches (atomically); eight threads build plans, query them and
// run every entry point, while another thread keeps changing the write-window
// setting, and each checks its own thread-local error text after a planted
// bad call.  The header promises that a plan is immutable (concurrent calls
// sharing one are safe), that zero_last_error is per thread, and that the
// window setting may change from any thread: TSan reports any data race.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "zero.h"
#include "zero_internal.h"

namespace {
std::atomic<long> g_step_launches{0}, g_copy_launches{0};
std::atomic<int> g_fail{0};
}  // namespace

namespace zk {
int launch_step(const StepArgs& a, int, int, int, int, bool, int n_blocks, void*) {
  if (a.n_seg < 1 || n_blocks < 1) g_fail++;
  g_step_launches++;
  return 0;
}
int launch_copy(const CopyArgs& a, int, int n_blocks, void*) {
  if (a.n_ent < 1 || n_blocks < 1) g_fail++;
  g_copy_launches++;
  return 0;
}
int launch_warm(const WarmArgs& a, int n_blocks, void*) {
  if (a.n < 1 || n_blocks < 1) g_fail++;
  return 0;
}
const char* hip_error_string(int) { return "stand-in"; }
int resident_blocks(int, int, int, int, bool) { return 1024; }
double wall_clock_hz() { return 1e8; }
double hbm_peak_bps() { return 8.192e12; }
}  // namespace zk

namespace {

constexpr uint64_t kSpan = 1ull << 40;
void* addr(int id, int64_t off = 0) { return (void*)(uintptr_t)((uint64_t)(id + 1) * kSpan + (uint64_t)off); }

void expect(bool c, const char* what) {
  if (!c) {
    fprintf(stderr, "FAIL: %s\n", what);
    g_fail++;
  }
}

void worker(int tid, zero_plan_t shared) {
  for (int it = 0; it < 200; ++it) {
    // A plan of the thread's own, and the shared one.
    const int64_t sizes[4] = {1000 + tid, 64, 4096 * (it % 3 + 1), 7};
    const int64_t psi = sizes[0] + sizes[1] + sizes[2] + sizes[3];
    zero_plan_t own = nullptr;
    expect(zero_plan(psi, 4 + tid % 3, sizes, 4, 2048, 8, &own) == ZERO_OK, "plan");
    for (zero_plan_t p : {own, shared}) {
      int64_t P, S;
      int32_t nb, nd;
      expect(zero_plan_info(p, &P, &S, &nb, &nd) == ZERO_OK, "info");
      std::vector<const void*> ptrs(nd);
      for (int q = 0; q < nd; ++q) ptrs[q] = addr(100 + q);
      zero_grad_src src = {ZERO_BF16, nd, ptrs.data(), nullptr};
      zero_adam_hyper hp = {1e-4, 0.9, 0.999, 1e-8, 1.0 / nd};
      expect(zero_adam_step(p, it % nd, &hp, it + 1, &src, nullptr, (float*)addr(1), (float*)addr(2),
                            (float*)addr(3), addr(4), ZERO_F16, 1, (void*)(uintptr_t)(0x100 * (1 + tid % 4))) == ZERO_OK,
             "step");
      expect(zero_shard_reduce(p, 0, &src, 0.25, (float*)addr(5), (void*)(uintptr_t)(0x100 * (1 + it % 4))) == ZERO_OK,
             "reduce");
      std::vector<const void*> shards(nd);
      for (int q = 0; q < nd; ++q) shards[q] = addr(200 + q);
      expect(zero_gather_pack(p, shards.data(), ZERO_BF16, addr(6), nullptr) == ZERO_OK, "gather");
      int32_t b;
      int64_t off;
      expect(zero_plan_tensor(p, 0, &b, &off) == ZERO_OK, "tensor");
    }
    const void* tens[4] = {addr(300), addr(301), addr(302), addr(303)};
    expect(zero_flatten(own, tens, ZERO_F32, addr(7), nullptr, 0, nullptr) == ZERO_OK, "flatten");
    // A planted bad call: this thread's error text names its own mistake.
    const std::string want = "rank " + std::to_string(-1 - tid);
    expect(zero_shard_reduce(own, -1 - tid, nullptr, 1.0, nullptr, nullptr) == ZERO_EINVAL, "bad rank");
    expect(strstr(zero_last_error(), want.c_str()) != nullptr, "per-thread error text");
    zero_plan_destroy(own);
  }
}

}  // namespace

int main() {
  const int64_t sizes[3] = {50000, 3, 70000};
  zero_plan_t shared = nullptr;
  if (zero_plan(120003, 8, sizes, 3, 60000, 64, &shared) != ZERO_OK) return 1;
  std::atomic<bool> stop{false};
  std::thread knob([&] {
    for (int i = 0; !stop.load(); ++i) {
      if (i % 3 == 0) zero_set_write_window(-1, 0);
      else if (i % 3 == 1) zero_set_write_window(0, 0);
      else zero_set_write_window(1000 + i % 500, 100);
      // Per-stream settings on the streams the workers launch on.
      void* s = (void*)(uintptr_t)(0x100 * (1 + i % 4));
      if (i % 5 == 0) zero_set_stream_write_window(s, -2, 0);
      else zero_set_stream_write_window(s, i % 2 ? 0 : 2000, 200);
      zero_set_warm_read(i % 3 == 0);
    }
  });
  std::vector<std::thread> ts;
  for (int t = 0; t < 8; ++t) ts.emplace_back(worker, t, shared);
  for (auto& t : ts) t.join();
  stop = true;
  knob.join();
  zero_plan_destroy(shared);
  printf("%ld step launches, %ld copy launches, %d failures\n", g_step_launches.load(), g_copy_launches.load(),
         g_fail.load());
  return g_fail.load() ? 1 : 0;
}
