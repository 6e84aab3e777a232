// Per-kernel timing with HIP events recorded on the launch stream.
//
// Disabled by default; moe_timing_enable(1) creates a fixed pool of events
// (no device memory) and every launch site brackets its kernel with a pair.
// moe_timing_report() waits for the recorded events, sums the elapsed times
// per kernel, and clears the record.  Used to measure each kernel's average
// duration inside a timed benchmark region.
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"

namespace {
const char* kNames[moe_launch::kNumTimers] = {"route", "index", "permute", "fc1", "quant_act",
                                              "fc2", "combine", "bwd_dA", "bwd_dW2",
                                              "bwd_dXp", "bwd_dW13", "pack", "xpose",
                                              "router_bwd", "router_aux", "capacity"};
struct Rec { int id; hipEvent_t a, b; };
std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_pool;
size_t g_next = 0;
std::vector<Rec> g_recs;
int g_open[moe_launch::kNumTimers];
hipEvent_t g_open_ev[moe_launch::kNumTimers];
}  // namespace

namespace moe_launch {
void timer_begin(int id, hipStream_t s) {
  if (!g_on || id < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_next + 2 > g_pool.size()) { g_open[id] = 0; return; }
  hipEvent_t a = g_pool[g_next++];
  (void)hipEventRecord(a, s);
  g_open[id] = 1;
  g_open_ev[id] = a;
}
void timer_end(int id, hipStream_t s) {
  if (!g_on || id < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_open[id] || g_next + 1 > g_pool.size()) return;
  hipEvent_t b = g_pool[g_next++];
  (void)hipEventRecord(b, s);
  g_recs.push_back({id, g_open_ev[id], b});
  g_open[id] = 0;
}
}  // namespace moe_launch

extern "C" {

int moe_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (on && g_pool.empty()) {
    g_pool.resize(16384);
    for (auto& e : g_pool)
      if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_HIP;
  }
  g_on = on != 0;
  g_next = 0;
  g_recs.clear();
  memset(g_open, 0, sizeof(g_open));
  return MOE_OK;
}

int moe_timing_report(char* buf, size_t len) {
  std::lock_guard<std::mutex> lk(g_mu);
  double tot[moe_launch::kNumTimers] = {0};
  int cnt[moe_launch::kNumTimers] = {0};
  for (auto& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return MOE_ERR_HIP;
    tot[r.id] += ms;
    cnt[r.id] += 1;
  }
  g_recs.clear();
  g_next = 0;
  size_t used = 0;
  if (buf && len) buf[0] = 0;
  for (int i = 0; i < moe_launch::kNumTimers; ++i) {
    if (!cnt[i] || !buf) continue;
    int n = snprintf(buf + used, len - used, "%s %d %.6f\n", kNames[i], cnt[i], tot[i]);
    if (n < 0 || size_t(n) >= len - used) break;
    used += size_t(n);
  }
  return MOE_OK;
}

}  // extern "C"
