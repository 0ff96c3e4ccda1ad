// Host test of the forward's plan-upload ring (staging.hpp) with a simulated
// runtime: events complete only when the test says so, copies are recorded.
// Checks that back-to-back uploads on a busy stream never wait on the host
// while slots can be added, that completed slots are reused, and that a wait
// happens (and is counted) only once the ring is full.
#include <cstdio>
#include <cstring>
#include <vector>

#include "staging.hpp"

namespace {

struct Sim {
  std::vector<bool> complete;  // per event id
  std::vector<std::vector<char>> pinned;
  std::vector<std::vector<char>> copies;  // what each copy read, in order
  int waits = 0;
};

struct FakeBackend {
  using Event = int;  // 0 = none; ids from 1
  using Stream = int;
  Sim* sim;
  void* alloc(size_t n) {
    sim->pinned.emplace_back(n);
    return sim->pinned.back().data();
  }
  int make_event() {
    sim->complete.push_back(false);
    return (int)sim->complete.size();
  }
  bool done(int e) { return sim->complete[e - 1]; }
  bool wait(int e) {
    ++sim->waits;
    sim->complete[e - 1] = true;
    return true;
  }
  bool copy(void*, const void* src, size_t n, int) {
    const char* c = static_cast<const char*>(src);
    sim->copies.emplace_back(c, c + n);
    return true;
  }
  bool record(int e, int) {
    sim->complete[e - 1] = false;  // pending until the stream reaches it
    return true;
  }
};

int failures = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAIL %s\n", what);
    ++failures;
  }
}

}  // namespace

int main() {
  Sim sim;
  sim.pinned.reserve(64);  // keep slot memory in place while the vector grows
  rnnt::StagingRing<FakeBackend> ring(FakeBackend{&sim});
  const char* what = nullptr;
  std::vector<char> a(1000, 'a'), b(3000, 'b');
  // two forwards back to back on a stream that has not reached either copy
  check(ring.upload(nullptr, a.data(), a.size(), 0, &what), "upload 1");
  check(ring.upload(nullptr, b.data(), b.size(), 0, &what), "upload 2");
  check(ring.host_waits() == 0 && sim.waits == 0, "no host wait for two back-to-back uploads");
  check(ring.slots() == 2, "second upload took a second slot");
  check(sim.copies.size() == 2 && sim.copies[0] == a && sim.copies[1] == b, "copies carry each call's plan");
  // the stream reaches both copies: the next upload reuses a slot
  for (size_t i = 0; i < sim.complete.size(); ++i) sim.complete[i] = true;
  check(ring.upload(nullptr, a.data(), a.size(), 0, &what), "upload 3");
  check(ring.slots() == 2 && ring.host_waits() == 0, "completed slot reused");
  // a busy stream: uploads add slots up to the limit without waiting
  for (int i = 0; i < rnnt::StagingRing<FakeBackend>::kMaxSlots; ++i)
    check(ring.upload(nullptr, b.data(), b.size(), 0, &what), "upload while busy");
  check(ring.slots() == rnnt::StagingRing<FakeBackend>::kMaxSlots, "ring grew to its limit");
  check(ring.host_waits() == 1 && sim.waits == 1, "the first upload past the limit waited once");
  // a plan larger than every slot while all are busy: waits for the oldest and grows it
  std::vector<char> big(1 << 20, 'c');
  check(ring.upload(nullptr, big.data(), big.size(), 0, &what), "large upload");
  check(ring.host_waits() == 2 && sim.copies.back() == big, "large upload copied after one more wait");
  if (failures == 0) std::printf("ok\n");
  return failures ? 1 : 0;
}
