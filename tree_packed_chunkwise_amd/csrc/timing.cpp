// timing.cpp -- per-kernel launch timing behind kda_timing_enable / kda_timing_read.
#include "timing.h"

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kda_tree.h"

namespace kda {
namespace {

struct Rec {
  std::string name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;          // launches since the last reset
std::vector<hipEvent_t> g_pool;   // reusable events
std::string g_pending;
hipEvent_t g_pending_ev = nullptr;
std::string g_only;               // time only launches of this kernel class ("" = all)
bool g_skip = false;              // the launch in progress is not timed
// totals after kda_timing_read folds the records: name -> (launches, ms)
std::map<std::string, std::pair<int64_t, double>> g_tot;
std::vector<std::string> g_names;

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

void fold() {
  for (Rec& r : g_recs) {
    float ms = 0.f;
    if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess &&
        hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      auto& t = g_tot[r.name];
      t.first += 1;
      t.second += ms;
    }
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
}

}  // namespace

bool timing_on() { return g_on.load(std::memory_order_relaxed); }

void timing_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_skip = !g_only.empty() && g_only != name;
  if (g_skip) return;
  g_pending = name;
  g_pending_ev = take_event();
  if (g_pending_ev) (void)hipEventRecord(g_pending_ev, st);
}

void timing_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_skip) {
    g_skip = false;
    return;
  }
  hipEvent_t b = take_event();
  if (b) (void)hipEventRecord(b, st);
  g_recs.push_back({g_pending, g_pending_ev, b});
  g_pending_ev = nullptr;
}

}  // namespace kda

extern "C" {

int kda_timing_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(kda::g_mu);
  kda::fold();
  kda::g_tot.clear();
  kda::g_on.store(on != 0);
  return KDA_OK;
}

int kda_timing_filter(const char* name) {
  std::lock_guard<std::mutex> lk(kda::g_mu);
  kda::g_only = name ? name : "";
  return KDA_OK;
}

int kda_timing_read(int32_t idx, char* name, int32_t name_len, int64_t* launches,
                    double* total_ms) {
  std::lock_guard<std::mutex> lk(kda::g_mu);
  kda::fold();
  kda::g_names.clear();
  for (auto& kv : kda::g_tot) kda::g_names.push_back(kv.first);
  const int32_t n = (int32_t)kda::g_names.size();
  if (idx < 0) return n;
  if (idx >= n) return KDA_ERR_ARG;
  const auto& t = kda::g_tot[kda::g_names[idx]];
  if (name && name_len > 0) {
    std::strncpy(name, kda::g_names[idx].c_str(), (size_t)name_len - 1);
    name[name_len - 1] = 0;
  }
  if (launches) *launches = t.first;
  if (total_ms) *total_ms = t.second;
  return n;
}

}  // extern "C"
