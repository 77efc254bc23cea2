// Host check of the work-claim protocol (claim_next in plan.h, the same
// function the kernels call): threads stand in for workgroups. Workgroup ids
// 0 .. n + claim_extra(n) - 1 are handed out in order by a dispatch counter,
// as the hardware hands out a grid; each workgroup makes one claim starting
// with queue (id mod 8), through std::atomic counters. Threads are pinned to
// "XCDs" (ids congruent to their XCD mod 8) and some run slower than others,
// so queues empty at different times and stealing happens. Half the counter
// loads return a stale value (zero), which the protocol must tolerate. Checks:
// every item claimed exactly once, the rest of the workgroups got -1.
// Prints "ok <cases> <steals>" or a failure description, exit status 1 on
// failure; with the argument "control" it runs a planted double claim and
// prints "caught". Built with g++ -fsanitize=thread by
// tests/test_claim_protocol.py.
#include <atomic>
#include <cstdio>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "plan.h"

using bdattn::claim_extra;
using bdattn::claim_next;
using bdattn::kClaimQueues;

namespace {

struct Result {
  bool ok = true;
  long steals = 0;
};

// One grid of n items run by `threads` host threads. `broken`: a planted
// mistake for the control run (every other fetch_add on queue 0 returns the
// counter without adding 1, so an item goes out twice).
Result run_grid(int32_t n, int threads, unsigned seed, bool broken = false) {
  const int32_t grid = n + claim_extra(n);
  std::vector<std::atomic<int32_t>> ctr(kClaimQueues);
  for (auto& c : ctr) c.store(0);
  std::vector<std::atomic<int32_t>> taken(n > 0 ? n : 1);
  for (auto& t : taken) t.store(0);
  // one dispatch counter per XCD: XCD x runs workgroups x, x + 8, ...
  std::vector<std::atomic<int32_t>> next(kClaimQueues);
  for (int x = 0; x < kClaimQueues; ++x) next[x].store(x);
  std::atomic<int32_t> empty{0}, stolen{0};
  auto worker = [&](int tid) {
    const int xcd = tid % kClaimQueues;
    std::mt19937 rng(seed * 7919u + unsigned(tid));
    const int slow = xcd % 3;  // XCDs 0, 3, 6 fastest; 2, 5 slowest
    for (;;) {
      const int32_t wg = next[xcd].fetch_add(kClaimQueues);
      if (wg >= grid) break;
      const int32_t item = claim_next(
          wg % kClaimQueues, n,
          [&](int y) { return (rng() & 1) ? ctr[y].load(std::memory_order_relaxed) : 0; },
          [&](int y) {
            if (broken && y == 0 && (rng() & 1)) return ctr[y].load(std::memory_order_relaxed);
            return ctr[y].fetch_add(1, std::memory_order_relaxed);
          });
      if (item < 0) {
        empty.fetch_add(1);
        continue;
      }
      if (item % kClaimQueues != wg % kClaimQueues) stolen.fetch_add(1);
      if (item >= n) {
        taken[0].store(1 << 20);  // out of range: reported below
        continue;
      }
      taken[item].fetch_add(1);
      for (int w = 0; w < slow * 20; ++w) std::this_thread::yield();  // the item's work
    }
  };
  std::vector<std::thread> ts;
  for (int t = 0; t < threads; ++t) ts.emplace_back(worker, t);
  for (auto& t : ts) t.join();
  Result r;
  r.steals = stolen.load();
  for (int32_t i = 0; i < n; ++i) {
    if (taken[i].load() != 1) {
      std::printf("n=%d threads=%d: item %d claimed %d times\n", n, threads, i, taken[i].load());
      r.ok = false;
      return r;
    }
  }
  if (empty.load() != grid - n) {
    std::printf("n=%d: %d empty claims, expected %d\n", n, empty.load(), grid - n);
    r.ok = false;
  }
  return r;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc > 1 && std::string(argv[1]) == "control") {  // the check must catch a planted mistake
    const Result r = run_grid(1000, 8, 1, true);
    std::printf(r.ok ? "missed\n" : "caught\n");
    return r.ok ? 1 : 0;
  }
  const int32_t sizes[] = {0, 1, 3, 7, 8, 9, 15, 64, 100, 257, 1000, 4096, 20000};
  int cases = 0;
  long steals = 0;
  unsigned seed = 1;
  for (int32_t n : sizes) {
    for (int threads : {8, 16, 24}) {
      for (int rep = 0; rep < 3; ++rep) {
        const Result r = run_grid(n, threads, seed++);
        if (!r.ok) return 1;
        steals += r.steals;
        ++cases;
      }
    }
  }
  // a negative (clobbered) counter yields no item
  const int32_t none = claim_next(0, 16, [](int) { return -5; }, [](int) { return -5; });
  if (none != -1) {
    std::printf("a negative counter gave item %d\n", none);
    return 1;
  }
  std::printf("ok %d %ld\n", cases, steals);
  return 0;
}
