// Per-kernel timing with HIP events, for measurement.  Off by default; when
// on, every kernel launch of the library (or every launch of one kernel name)
// is bracketed by two events recorded on the launch's own stream, and
// durations are aggregated by kernel name.
#include <string.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tp_mlp.h"
#include "kernels.h"

namespace tpmlp {
namespace {

struct Record {
  const char* name;
  hipEvent_t start, stop;
};

struct Profiler {
  std::mutex mu;
  bool on = false;
  bool filtered = false;  // record only the kernels named `only`
  std::string only;
  std::vector<Record> records;
  std::vector<hipEvent_t> pool;
  struct Agg {
    std::string name;
    int64_t launches;
    double ms;
  };
  std::vector<Agg> agg;
  bool agg_valid = false;

  hipEvent_t take() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void recycle() {
    for (auto& r : records) {
      pool.push_back(r.start);
      pool.push_back(r.stop);
    }
    records.clear();
  }
};

Profiler& prof() {
  static Profiler* p = new Profiler();  // never destroyed: events outlive static teardown order
  return *p;
}

}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t s) : name_(name), stream_(s) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.on || (p.filtered && strcmp(name, p.only.c_str()) != 0)) return;
  start_ = p.take();
  stop_ = p.take();
  if (start_ && stop_ && hipEventRecord(start_, s) == hipSuccess) {
    active_ = true;
  }
}

KernelTimer::~KernelTimer() {
  if (!active_) return;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  (void)hipEventRecord(stop_, stream_);
  p.records.push_back(Record{name_, start_, stop_});
  p.agg_valid = false;
}

}  // namespace tpmlp

using namespace tpmlp;

extern "C" {

int tp_mlp_profile_enable(int32_t on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (on && !p.on) {
    p.recycle();
    p.agg.clear();
    p.agg_valid = false;
  }
  p.on = on != 0;
  return TP_MLP_OK;
}

int tp_mlp_profile_only(const char* name) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.filtered = name != nullptr;
  p.only = name ? name : "";
  return TP_MLP_OK;
}

int32_t tp_mlp_profile_count(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.agg_valid) {
    std::map<std::string, size_t> index;
    p.agg.clear();
    for (auto& r : p.records) {
      if (hipEventSynchronize(r.stop) != hipSuccess) return TP_MLP_EHIP;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return TP_MLP_EHIP;
      auto it = index.find(r.name);
      if (it == index.end()) {
        index[r.name] = p.agg.size();
        p.agg.push_back({r.name, 1, (double)ms});
      } else {
        p.agg[it->second].launches += 1;
        p.agg[it->second].ms += ms;
      }
    }
    p.agg_valid = true;
  }
  return (int32_t)p.agg.size();
}

int tp_mlp_profile_entry(int32_t i, const char** name, int64_t* launches, double* total_ms) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  if (!p.agg_valid || i < 0 || i >= (int32_t)p.agg.size() || !name || !launches || !total_ms) return TP_MLP_EINVAL;
  *name = p.agg[i].name.c_str();
  *launches = p.agg[i].launches;
  *total_ms = p.agg[i].ms;
  return TP_MLP_OK;
}

}  // extern "C"
