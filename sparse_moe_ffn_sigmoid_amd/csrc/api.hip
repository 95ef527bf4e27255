// Status strings and the optional stage-timing diagnostics.
#include <mutex>
#include <vector>

#include "prof.hpp"

namespace moe {
namespace prof {

namespace {
struct Pair {
  int stage;
  hipEvent_t start, end;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Pair> g_pending;
std::vector<hipEvent_t> g_pool;
Pair g_open[ST_COUNT];
bool g_is_open[ST_COUNT] = {};
double g_total[ST_COUNT] = {};
int32_t g_count[ST_COUNT] = {};

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

bool enabled() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on;
}

void record(int stage, bool start, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || stage < 0 || stage >= ST_COUNT) return;
  hipEvent_t e = take_event();
  if (!e) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    g_pool.push_back(e);
    return;
  }
  if (start) {
    g_open[stage] = Pair{stage, e, nullptr};
    g_is_open[stage] = true;
  } else if (g_is_open[stage]) {
    g_open[stage].end = e;
    g_pending.push_back(g_open[stage]);
    g_is_open[stage] = false;
  } else {
    g_pool.push_back(e);
  }
}

}  // namespace prof
}  // namespace moe

extern "C" const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype combination";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int moe_stage_timing(int enable) {
  using namespace moe::prof;
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = enable != 0;
  for (auto& p : g_pending) {
    g_pool.push_back(p.start);
    g_pool.push_back(p.end);
  }
  g_pending.clear();
  for (int i = 0; i < ST_COUNT; ++i) {
    g_total[i] = 0.0;
    g_count[i] = 0;
    g_is_open[i] = false;
  }
  return MOE_OK;
}

extern "C" int moe_stage_times(double* total_ms, int32_t* counts, int32_t max_stages) {
  using namespace moe::prof;
  std::lock_guard<std::mutex> lk(g_mu);
  for (auto& p : g_pending) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.start, p.end) != hipSuccess) return MOE_EHIP;
    g_total[p.stage] += ms;
    g_count[p.stage] += 1;
    g_pool.push_back(p.start);
    g_pool.push_back(p.end);
  }
  g_pending.clear();
  const int nst = max_stages < ST_COUNT ? max_stages : ST_COUNT;
  for (int i = 0; i < nst; ++i) {
    if (total_ms) total_ms[i] = g_total[i];
    if (counts) counts[i] = g_count[i];
  }
  return ST_COUNT;
}

extern "C" const char* moe_stage_name(int stage) {
  static const char* names[] = {"router",          "latent_down",   "shared_gate_up",
                                "routing",         "permute",       "routed_gate_up",
                                "routed_down",     "combine_rmsnorm", "up_proj_shared_down"};
  if (stage < 0 || stage >= moe::prof::ST_COUNT) return "unknown";
  return names[stage];
}
