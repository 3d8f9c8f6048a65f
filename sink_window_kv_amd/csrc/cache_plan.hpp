// Host-side bookkeeping of the frame-sink + local-ring KV cache.
//
// Pure C++ (no HIP): which frames are resident, in which store slot, with
// which time position.  Follows the LongLive paper review, section 3
// "Frame Sink" (the first frames' KV is pinned for the whole stream) and
// "Short-Window Attention" (a window of the most recent latent frames).
//
// Store slots: sink frame f -> slot f (0 <= f < n_sink); any later frame f
// -> slot n_sink + (f - n_sink) mod n_local, overwriting (evicting) the frame
// n_local earlier.  Logical order: sinks, then local frames oldest -> newest.
#pragma once

#include <cstdint>
#include <vector>

namespace sa {

constexpr int kMaxFrames = 64;

struct ResidentFrame {
  int64_t frame;  // frame number since creation / reset
  int64_t t;      // time position
  int32_t segment;  // 0 sink, 1 ring
  int32_t slot;     // index inside the segment
  int32_t store_slot;  // index into the [n_sink + n_local] store
};

class CachePlan {
 public:
  CachePlan() = default;
  CachePlan(int n_sink, int n_local) : n_sink_(n_sink), n_local_(n_local) {
    t_.assign(static_cast<size_t>(n_sink + n_local), 0);
  }

  int n_sink() const { return n_sink_; }
  int n_local() const { return n_local_; }
  int64_t n_appended() const { return n_appended_; }
  bool has_frames() const { return n_appended_ > 0; }
  int64_t newest_t() const { return newest_t_; }

  void reset() {
    n_appended_ = 0;
    newest_t_ = 0;
    for (auto& x : t_) x = 0;
  }

  int store_slot_of(int64_t frame) const {
    if (frame < n_sink_) return static_cast<int>(frame);
    return n_sink_ + static_cast<int>((frame - n_sink_) % n_local_);
  }

  // 0 if the chunk may be appended; otherwise a code: 1 = bad count,
  // 2 = chunk does not fit the ring, 3 = time does not increase.
  int check_append(int n_frames, int64_t t0) const {
    if (n_frames < 1 || n_frames > kMaxFrames) return 1;
    int64_t first = n_appended_;
    int64_t non_sink = 0;
    for (int i = 0; i < n_frames; ++i)
      if (first + i >= n_sink_) ++non_sink;
    if (non_sink > n_local_) return 2;
    if (n_appended_ > 0 && t0 <= newest_t_) return 3;
    if (t0 > INT64_MAX - n_frames) return 3;
    return 0;
  }

  // Store slots and times the chunk's frames go to (call check_append first).
  std::vector<ResidentFrame> plan_append(int n_frames, int64_t t0) const {
    std::vector<ResidentFrame> out;
    for (int i = 0; i < n_frames; ++i) {
      int64_t f = n_appended_ + i;
      ResidentFrame r;
      r.frame = f;
      r.t = t0 + i;
      r.segment = f < n_sink_ ? 0 : 1;
      r.store_slot = store_slot_of(f);
      r.slot = r.segment == 0 ? r.store_slot : r.store_slot - n_sink_;
      out.push_back(r);
    }
    return out;
  }

  void commit_append(int n_frames, int64_t t0) {
    for (int i = 0; i < n_frames; ++i) t_[store_slot_of(n_appended_ + i)] = t0 + i;
    n_appended_ += n_frames;
    newest_t_ = t0 + n_frames - 1;
  }

  // Resident frames in logical order.
  std::vector<ResidentFrame> resident() const {
    std::vector<ResidentFrame> out;
    int64_t n = n_appended_;
    int64_t n_s = n < n_sink_ ? n : n_sink_;
    for (int64_t f = 0; f < n_s; ++f) {
      int s = store_slot_of(f);
      out.push_back({f, t_[s], 0, s, s});
    }
    int64_t lo = n - n_local_;
    if (lo < n_sink_) lo = n_sink_;
    for (int64_t f = lo; f < n; ++f) {
      int s = store_slot_of(f);
      out.push_back({f, t_[s], 1, s - n_sink_, s});
    }
    return out;
  }

 private:
  int n_sink_ = 0;
  int n_local_ = 1;
  int64_t n_appended_ = 0;
  int64_t newest_t_ = 0;
  std::vector<int64_t> t_;  // time of the frame in each store slot
};

}  // namespace sa
