// Optional per-kernel timing with HIP events.  While enabled, every kernel a
// spec_* call enqueues is launched with a start/stop event pair that the
// runtime stamps from that kernel's own dispatch (hipExtLaunchKernel), so an
// interval covers the kernel and not the queue gaps around it;
// spec_profile_read synchronises the recorded events and reports, per kernel
// kind, the launch count and the summed event time.  Disabled (the default),
// the hooks cost one branch per launch.
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/spec_verify.h"
#include "internal.h"

namespace specv {
namespace {

struct Pair {
  hipEvent_t a = nullptr, b = nullptr;
  int kind = -1;
  bool used = false;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<Pair> g_pairs;
size_t g_next = 0;
double g_ms[kProfKinds] = {0};
long g_count[kProfKinds] = {0};
std::vector<float> g_each[kProfKinds];  // every timed launch's duration, in order

// Fold every recorded pair into the totals (synchronising its end event).
void drain_locked() {
  for (auto& p : g_pairs) {
    if (!p.used) continue;
    float ms = 0.f;
    if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
      g_ms[p.kind] += ms;
      g_count[p.kind] += 1;
      g_each[p.kind].push_back(ms);
    }
    p.used = false;
  }
  g_next = 0;
}

}  // namespace

ProfEvents prof_begin(int kind) {
  ProfEvents ev;
  if (!g_on) return ev;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return ev;
  if (g_next == g_pairs.size()) drain_locked();
  Pair& p = g_pairs[g_next];
  p.kind = kind;
  ev.start = p.a;
  ev.stop = p.b;
  ev.slot = static_cast<int>(g_next);
  return ev;
}

void prof_end(const ProfEvents& ev, hipError_t launch_status) {
  if (ev.slot < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || ev.slot != static_cast<int>(g_next)) return;
  if (launch_status == hipSuccess) {
    g_pairs[g_next].used = true;
    ++g_next;
  }
}

}  // namespace specv

using namespace specv;

extern "C" {

int spec_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (on) {
    if (g_pairs.empty()) {
      g_pairs.resize(2048);
      for (auto& p : g_pairs) {
        if (hipEventCreate(&p.a) != hipSuccess || hipEventCreate(&p.b) != hipSuccess)
          return SPEC_EHIP;
      }
    }
    for (int i = 0; i < kProfKinds; ++i) {
      g_ms[i] = 0.0;
      g_count[i] = 0;
      g_each[i].clear();
    }
    for (auto& p : g_pairs) p.used = false;
    g_next = 0;
    g_on = true;
  } else {
    g_on = false;
  }
  return SPEC_OK;
}

int spec_profile_read(int kind, long* launches, double* total_ms) {
  if (kind < 0 || kind >= kProfKinds || launches == nullptr || total_ms == nullptr)
    return SPEC_EINVAL;
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  *launches = g_count[kind];
  *total_ms = g_ms[kind];
  return SPEC_OK;
}

int spec_profile_durations(int kind, float* ms_host, long cap, long* n_host) {
  if (kind < 0 || kind >= kProfKinds || n_host == nullptr || cap < 0 ||
      (cap > 0 && ms_host == nullptr))
    return SPEC_EINVAL;
  std::lock_guard<std::mutex> lk(g_mu);
  drain_locked();
  const auto& v = g_each[kind];
  const long n = static_cast<long>(v.size()) < cap ? static_cast<long>(v.size()) : cap;
  for (long i = 0; i < n; ++i) ms_host[i] = v[i];
  *n_host = static_cast<long>(v.size());
  return SPEC_OK;
}

}  // extern "C"
