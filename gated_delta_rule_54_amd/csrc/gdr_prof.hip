// Optional per-kernel event timing behind gdr_profile_enable / _read.
#include <gdr.h>

#include <map>
#include <string>
#include <vector>

#include "gdr_internal.h"

namespace gdr {
namespace {

struct Pending {
  const char* name;
  hipEvent_t start, stop;
};

struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> free_events;
  std::vector<Pending> pending;
  Pending* open = nullptr;

  hipEvent_t get() {
    hipEvent_t e = nullptr;
    if (!free_events.empty()) {
      e = free_events.back();
      free_events.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
    }
    return e;
  }
  void drop() {
    for (auto& p : pending) {
      if (p.start) free_events.push_back(p.start);
      if (p.stop) free_events.push_back(p.stop);
    }
    pending.clear();
  }
};

thread_local Profiler g_prof;

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t st) : stream_(st), active_(g_prof.on) {
  if (!active_) return;
  Pending p{name, g_prof.get(), g_prof.get()};
  // an event that could not be recorded is returned to the pool, and a pair
  // missing either event is never read back
  if (p.start && hipEventRecord(p.start, st) != hipSuccess) {
    g_prof.free_events.push_back(p.start);
    p.start = nullptr;
  }
  g_prof.pending.push_back(p);
}

ProfScope::~ProfScope() {
  if (!active_ || g_prof.pending.empty()) return;
  Pending& p = g_prof.pending.back();
  if (p.stop && hipEventRecord(p.stop, stream_) != hipSuccess) {
    g_prof.free_events.push_back(p.stop);
    p.stop = nullptr;
  }
}

}  // namespace gdr

extern "C" {

gdr_status gdr_profile_enable(int on) {
  gdr::g_prof.on = on != 0;
  if (!on) gdr::g_prof.drop();
  return GDR_OK;
}

gdr_status gdr_profile_read(gdr_kernel_time* out, int cap, int* n) {
  if (!n || (cap > 0 && !out)) return GDR_ERR_NULL_ARG;
  struct Acc { double ms = 0; int64_t count = 0; };
  std::vector<std::pair<const char*, Acc>> acc;  // first-seen order
  for (auto& p : gdr::g_prof.pending) {
    float ms = 0.f;
    if (p.start && p.stop && hipEventSynchronize(p.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
      size_t i = 0;
      while (i < acc.size() && std::string(acc[i].first) != p.name) ++i;
      if (i == acc.size()) acc.push_back({p.name, Acc{}});
      acc[i].second.ms += ms;
      acc[i].second.count += 1;
    }
  }
  gdr::g_prof.drop();
  *n = static_cast<int>(acc.size());
  for (int i = 0; i < cap && i < *n; ++i) out[i] = gdr_kernel_time{acc[i].first, acc[i].second.ms, acc[i].second.count};
  return GDR_OK;
}

}  // extern "C"
