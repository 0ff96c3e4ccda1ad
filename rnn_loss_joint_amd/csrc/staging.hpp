// Ring of pinned host staging slots for the forward's host -> device copy of
// the tile plan, without host waits in steady state.
//
// Each upload takes a slot whose previous copy has completed (checked with a
// non-blocking event query), or, if every slot of sufficient size is still
// in flight, adds a slot (a pinned host allocation; device memory is never
// allocated). Only when kMaxSlots slots exist and none fits does an upload
// wait on the host, for the slot recorded earliest; those waits are counted.
// Slots are never freed while the process runs (freeing pinned memory can
// synchronize the device).
//
// The backend supplies the runtime calls, so the ring logic is plain C++:
//   void* alloc(size_t bytes);           pinned host allocation (null: failure)
//   E     make_event();                  an event (null: failure)
//   bool  done(E);                       non-blocking: has the event completed?
//   bool  wait(E);                       blocking wait (false: failure)
//   bool  copy(void* dst, const void* src, size_t n, S stream);  async H2D copy
//   bool  record(E, S stream);
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <cstring>
#include <mutex>
#include <vector>

namespace rnnt {

template <class Backend>
class StagingRing {
 public:
  using E = typename Backend::Event;
  using S = typename Backend::Stream;
  static constexpr int kMaxSlots = 16;
  static constexpr size_t kMinSlot = 64 * 1024;

  explicit StagingRing(Backend be = Backend()) : be_(be) { slots_.reserve(kMaxSlots); }

  // Copies src[0, n) to dst on `stream` through a pinned slot. Returns false
  // (and sets *what) if a runtime call fails.
  bool upload(void* dst, const void* src, size_t n, S stream, const char** what) {
    std::lock_guard<std::mutex> lk(mu_);
    Slot* s = nullptr;
    // a free slot that is large enough, the smallest such
    for (Slot& c : slots_)
      if (c.cap >= n && (!c.used || be_.done(c.ev)) && (!s || c.cap < s->cap)) s = &c;
    if (!s && (int)slots_.size() < kMaxSlots) {
      size_t cap = kMinSlot;
      while (cap < n) cap *= 2;
      Slot c{};
      c.host = be_.alloc(cap);
      if (!c.host) return fail(what, "pinned staging allocation failed");
      c.ev = be_.make_event();
      if (!c.ev) return fail(what, "staging event creation failed");
      c.cap = cap;
      slots_.push_back(c);
      s = &slots_.back();
    }
    if (!s) {
      // every slot is in use or too small: wait for the oldest large enough
      // one; if none is large enough, wait for the oldest and grow it
      Slot* oldest = nullptr;
      for (Slot& c : slots_)
        if (c.cap >= n && (!oldest || c.seq < oldest->seq)) oldest = &c;
      if (!oldest) {
        for (Slot& c : slots_)
          if (!oldest || c.seq < oldest->seq) oldest = &c;
      }
      ++host_waits_;
      if (oldest->used && !be_.wait(oldest->ev)) return fail(what, "staging event wait failed");
      if (oldest->cap < n) {
        size_t cap = oldest->cap;
        while (cap < n) cap *= 2;
        void* h = be_.alloc(cap);  // the old, smaller slot is kept allocated (see above)
        if (!h) return fail(what, "pinned staging allocation failed");
        retired_.push_back(oldest->host);
        oldest->host = h;
        oldest->cap = cap;
      }
      s = oldest;
    }
    std::memcpy(s->host, src, n);
    if (!be_.copy(dst, s->host, n, stream)) return fail(what, "staging copy failed");
    if (!be_.record(s->ev, stream)) return fail(what, "staging event record failed");
    s->used = true;
    s->seq = ++seq_;
    return true;
  }

  int64_t host_waits() const { return host_waits_; }
  int slots() const { return (int)slots_.size(); }

 private:
  struct Slot {
    void* host;
    size_t cap;
    E ev;
    bool used;
    uint64_t seq;
  };
  static bool fail(const char** what, const char* msg) {
    if (what) *what = msg;
    return false;
  }
  Backend be_;
  std::mutex mu_;
  std::vector<Slot> slots_;
  std::vector<void*> retired_;
  uint64_t seq_ = 0;
  int64_t host_waits_ = 0;
};

}  // namespace rnnt
