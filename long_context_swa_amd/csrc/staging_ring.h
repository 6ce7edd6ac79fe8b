// Space management of the pinned host ring through which libswa stages small tables (page-table
// rows, decode work lists, commit metadata) for stream-ordered copies to the device.  Pure C++: the
// HIP side (events, copies) lives in pool.cpp; this header is also compiled by a host-only test.
//
// A region of the ring stays "live" from the moment its bytes are handed out until the copy that
// reads it is known to have executed.  Before a range is handed out again, EVERY live region that
// overlaps it is returned to the caller to wait for -- not only the oldest one: when a lap wraps
// before reaching the end of the previous lap, the oldest live region can sit beyond the new range
// while younger regions from the last lap still overlap it.
#pragma once

#include <cstddef>
#include <cstdint>
#include <deque>
#include <vector>

namespace swa {

class RingSpace {
 public:
  explicit RingSpace(size_t cap = 0) : cap_(cap) {}
  size_t capacity() const { return cap_; }
  size_t live_regions() const { return live_.size(); }

  // Place the next `n` bytes (0 < n <= capacity) at the head, wrapping to 0 if they do not fit.
  // Tokens of all live regions overlapping [offset, offset + n) are removed from the live set and
  // appended to `wait`; the caller must wait for each before writing the range.
  size_t reserve(size_t n, std::vector<uint64_t> &wait) {
    if (head_ + n > cap_) head_ = 0;
    const size_t b = head_, e = head_ + n;
    for (auto it = live_.begin(); it != live_.end();) {
      if (it->begin < e && b < it->end) {
        wait.push_back(it->token);
        it = live_.erase(it);
      } else {
        ++it;
      }
    }
    head_ = e;
    return b;
  }

  // The copy reading [offset, offset + n) is in flight until `token` completes.
  void publish(size_t offset, size_t n, uint64_t token) { live_.push_back({offset, offset + n, token}); }

  // Drop completed regions from the oldest end: `done(token)` reports completion (copies on one
  // stream complete in order); `dropped(token)` is called for each region removed.
  template <class Done, class Dropped>
  void retire(Done done, Dropped dropped) {
    while (!live_.empty() && done(live_.front().token)) {
      dropped(live_.front().token);
      live_.pop_front();
    }
  }

  // Remove every live region (after the caller waited for all of them).
  template <class Dropped>
  void clear(Dropped dropped) {
    for (auto &r : live_) dropped(r.token);
    live_.clear();
  }

 private:
  struct Region {
    size_t begin, end;
    uint64_t token;
  };
  size_t cap_, head_ = 0;
  std::deque<Region> live_;
};

}  // namespace swa
