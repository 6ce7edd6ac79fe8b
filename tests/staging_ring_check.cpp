// Host-only check of the staging ring's reuse rule (long_context_swa_amd/csrc/staging_ring.h).
// A simulated device executes the uploads' copies in order, `lag` uploads behind the host; a shadow
// array records, per byte, the upload whose copy still has to read it.  Handing out a byte whose
// copy has neither executed nor been waited for is the failure being checked for.  The same
// scenarios run against a test-local copy of a front-only reuse rule (a plausible mistake), which
// must be caught, so the check has the power to see the failure.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <random>
#include <vector>

#include "staging_ring.h"

struct FrontOnly {  // reuse rule that waits only while the OLDEST live region overlaps
  explicit FrontOnly(size_t cap) : cap(cap) {}
  size_t reserve(size_t n, std::vector<uint64_t> &wait) {
    if (head + n > cap) head = 0;
    size_t b = head, e = head + n;
    while (!live.empty() && live.front().b < e && b < live.front().e) {
      wait.push_back(live.front().t);
      live.pop_front();
    }
    head = e;
    return b;
  }
  void publish(size_t b, size_t n, uint64_t t) { live.push_back({b, b + n, t}); }
  template <class D, class X> void retire(D done, X) {
    while (!live.empty() && done(live.front().t)) live.pop_front();
  }
  struct R { size_t b, e; uint64_t t; };
  size_t cap, head = 0;
  std::deque<R> live;
};

template <class Ring>
long run(unsigned seed, size_t cap, long n_up, long lag) {
  std::mt19937_64 rng(seed);
  Ring ring(cap);
  std::vector<long> owner(cap, -1);
  long done_floor = -1, violations = 0;
  std::vector<uint64_t> wait;
  for (long i = 0; i < n_up; ++i) {
    const long gpu_done = std::max(i - lag, done_floor);
    ring.retire([&](uint64_t t) { return (long)t <= gpu_done; }, [](uint64_t) {});
    size_t n = 256 * (1 + rng() % 16);
    if (rng() % 100 < 3) n = 256 * (60 + rng() % 60);  // occasional large upload
    wait.clear();
    const size_t b = ring.reserve(n, wait);
    long waited = -1;
    for (auto t : wait) waited = std::max(waited, (long)t);
    const long completed = std::max(gpu_done, waited);  // in-order copies: waiting on t finishes all <= t
    for (size_t x = b; x < b + n; ++x) {
      if (owner[x] > completed) { ++violations; break; }
    }
    for (size_t x = b; x < b + n; ++x) owner[x] = i;
    ring.publish(b, n, (uint64_t)i);
    done_floor = std::max(done_floor, waited);
  }
  return violations;
}

int main() {
  long bad_new = 0, bad_old = 0;
  for (unsigned seed = 1; seed <= 3; ++seed)
    for (long lag : {0L, 10L, 200L, 2000L, 100000L}) {
      bad_new += run<swa::RingSpace>(seed, 1 << 20, 8000, lag);
      bad_old += run<FrontOnly>(seed, 1 << 20, 8000, lag);
    }
  std::printf("ring_space_violations=%ld front_only_violations=%ld\n", bad_new, bad_old);
  return (bad_new == 0 && bad_old > 0) ? 0 : 1;
}
