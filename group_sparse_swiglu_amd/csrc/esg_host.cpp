// Host-only pieces: the subsample draw and kernel timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "esg_internal.hpp"

namespace esg {

// ---------------------------------------------------------------------------
// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the state advances by the
// 64-bit golden-ratio increment and each output is the state passed through
// two xor-shift-multiply rounds and a final xor-shift (the mixing constants of
// Vigna's public splitmix64.c).
// ---------------------------------------------------------------------------
struct SplitMix64 {
  uint64_t state;
  explicit SplitMix64(uint64_t seed) : state(seed) {}
  uint64_t next() {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

// Per group: a partial Fisher-Yates shuffle of 0..gs-1 (draw i swaps
// position i with i + next() mod (gs - i)); the first spg ids, sorted and
// offset by g*gs, are the group's sampled rows.
void subsample_index(int d_ff, int group_size, int spg, uint64_t seed, int32_t* out) {
  const int groups = d_ff / group_size;
  SplitMix64 rng(seed);
  std::vector<int32_t> pool(group_size);
  for (int g = 0; g < groups; ++g) {
    for (int i = 0; i < group_size; ++i) pool[i] = i;
    for (int i = 0; i < spg; ++i) {
      const uint64_t r = rng.next() % (uint64_t)(group_size - i);
      std::swap(pool[i], pool[i + (int)r]);
    }
    std::sort(pool.begin(), pool.begin() + spg);
    for (int i = 0; i < spg; ++i) out[(size_t)g * spg + i] = g * group_size + pool[i];
  }
}

// ---------------------------------------------------------------------------
// Kernel timing
// ---------------------------------------------------------------------------
namespace {
struct TimedLaunch {
  std::string name;
  hipEvent_t start, stop;
};
// Per host thread: a thread times its own launches (no shared mutable state).
thread_local bool g_timing = false;
thread_local std::vector<TimedLaunch> g_launches;
thread_local std::vector<hipEvent_t> g_pool;  // events reused across resets: no creation in timed loops

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

bool timing_enabled() { return g_timing; }

LaunchTimer::LaunchTimer(const char* name, hipStream_t stream) : name_(name), stream_(stream), start_(nullptr) {
  if (!g_timing) return;
  hipEvent_t e = take_event();
  if (e == nullptr) return;
  if (hipEventRecord(e, stream) != hipSuccess) {
    g_pool.push_back(e);
    return;
  }
  start_ = (void*)e;
}

LaunchTimer::~LaunchTimer() {
  if (start_ == nullptr) return;
  hipEvent_t stop = take_event();
  if (stop == nullptr || hipEventRecord(stop, stream_) != hipSuccess) {
    g_pool.push_back((hipEvent_t)start_);
    if (stop) g_pool.push_back(stop);
    return;
  }
  g_launches.push_back({name_, (hipEvent_t)start_, stop});
}

void timing_set(bool on) { g_timing = on; }

void timing_reset() {
  for (auto& l : g_launches) {
    (void)hipEventSynchronize(l.stop);
    g_pool.push_back(l.start);
    g_pool.push_back(l.stop);
  }
  g_launches.clear();
}

int timing_read(const char* name, double* total_ms, int* launches) {
  double tot = 0.0;
  int n = 0;
  for (auto& l : g_launches) {
    if (l.name != name) continue;
    if (hipEventSynchronize(l.stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, l.start, l.stop) != hipSuccess) return -1;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return 0;
}

}  // namespace esg
