// Optional kernel tracing: HIP events around every library launch while
// enabled (usp_trace_enable / usp_trace_collect in usp.h).
#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "usp_internal.h"

namespace usp {

namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;

}  // namespace

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

TraceScope::TraceScope(const char* n, hipStream_t st) : name(n), s(st), start(nullptr) {
  if (!trace_on()) return;
  if (hipEventCreate(&start) != hipSuccess) {
    start = nullptr;
    return;
  }
  if (hipEventRecord(start, s) != hipSuccess) {
    (void)hipEventDestroy(start);
    start = nullptr;
  }
}

TraceScope::~TraceScope() {
  if (start == nullptr) return;
  hipEvent_t stop = nullptr;
  if (hipEventCreate(&stop) != hipSuccess || hipEventRecord(stop, s) != hipSuccess) {
    (void)hipEventDestroy(start);
    if (stop) (void)hipEventDestroy(stop);
    return;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back({name, start, stop});
}

}  // namespace usp

extern "C" {

int usp_trace_enable(int on) { return usp::g_on.exchange(on != 0) ? 1 : 0; }

int usp_trace_collect(usp_trace_entry* out, int max_entries) {
  if (out == nullptr && max_entries > 0) return USP_ERR_NULL;
  std::vector<usp::Rec> recs;
  {
    std::lock_guard<std::mutex> lk(usp::g_mu);
    recs.swap(usp::g_recs);
  }
  std::map<std::string, std::pair<long long, double>> agg;
  int rc = USP_OK;
  for (const usp::Rec& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      rc = USP_ERR_HIP;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  if (rc != USP_OK) return rc;
  std::vector<std::pair<std::string, std::pair<long long, double>>> v(agg.begin(), agg.end());
  std::sort(v.begin(), v.end(), [](const auto& a, const auto& b) { return a.second.second > b.second.second; });
  int n = 0;
  for (const auto& e : v) {
    if (n >= max_entries) break;
    std::memset(out[n].name, 0, sizeof(out[n].name));
    std::strncpy(out[n].name, e.first.c_str(), sizeof(out[n].name) - 1);
    out[n].launches = e.second.first;
    out[n].total_ms = e.second.second;
    ++n;
  }
  return n;
}

}  // extern "C"
