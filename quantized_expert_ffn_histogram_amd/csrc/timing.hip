// Optional per-kernel device timing (off by default): when enabled, every
// kernel the library launches is bracketed by two HIP events recorded on the
// launch stream; a query sums the elapsed times per kernel name.  Timers that
// exist but stay off unless asked for follow the lqnn.cn static review §5.3
// (per-phase timing points, disabled by default).
#include <mutex>
#include <string>
#include <vector>

#include "moe_internal.h"

namespace strata {
namespace {

struct Record {
  const char *name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Record> g_records;   // in launch order
std::vector<hipEvent_t> g_pool;  // reusable events
size_t g_open = 0;               // index of the record awaiting its stop event

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

void release_all() {
  for (auto &r : g_records) {
    if (r.start) g_pool.push_back(r.start);
    if (r.stop) g_pool.push_back(r.stop);
  }
  g_records.clear();
}

}  // namespace

void timing_begin(const char *name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled) return;
  Record r{name, take_event(), nullptr};
  if (r.start) (void)hipEventRecord(r.start, s);
  g_open = g_records.size();
  g_records.push_back(r);
}

void timing_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_enabled || g_open >= g_records.size()) return;
  Record &r = g_records[g_open];
  r.stop = take_event();
  if (r.stop) (void)hipEventRecord(r.stop, s);
  g_open = g_records.size();
}

int timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  release_all();
  g_enabled = on != 0;
  g_open = 0;
  return 0;
}

int timing_query(const char *name, int *launches, double *total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  int n = 0;
  double ms = 0.0;
  for (auto &r : g_records) {
    if (!r.start || !r.stop) continue;
    if (name && std::string(name) != r.name) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return -1;
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return 0;
}

int timing_names(const char **names, int max_names) {
  std::lock_guard<std::mutex> lk(g_mu);
  std::vector<const char *> uniq;
  for (auto &r : g_records) {
    bool seen = false;
    for (const char *u : uniq) seen |= std::string(u) == r.name;
    if (!seen) uniq.push_back(r.name);
  }
  for (int i = 0; i < (int)uniq.size() && i < max_names; ++i) names[i] = uniq[i];
  return (int)uniq.size();
}

}  // namespace strata
