// Optional per-kernel timing for benchmarks.  Off by default; when enabled
// every kernel launch of the library is bracketed by a pair of HIP events
// recorded on the launch stream, and the elapsed times can be read back per
// kernel.  Events come from a pool that is created on first use and kept for
// the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/docmask_gqa.h"
#include "kernels.hpp"

namespace dmgqa {
namespace {

struct Rec {
  int kernel;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_recs;       // records since the last enable
std::vector<hipEvent_t> g_pool;  // all events ever created
size_t g_used = 0;
int g_open[kNumKernels];

const char* kNames[kNumKernels] = {"prep",          "fwd",        "bwd_dq",
                                   "bwd_dkdv",      "bwd_reduce", "sched_rowstat",
                                   "tile_order",    "bwd_dq_rest", "scale_scan"};

hipEvent_t take_event() {
  if (g_used == g_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_used++];
}

}  // namespace

void timing_begin(int kernel, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  hipEvent_t e = take_event();
  if (!e || hipEventRecord(e, st) != hipSuccess) return;  // untimed, not an error
  g_recs.push_back({kernel, e, nullptr});
  g_open[kernel] = (int)g_recs.size() - 1;
}

void timing_end(int kernel, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_open[kernel] < 0) return;
  hipEvent_t e = take_event();
  if (!e || hipEventRecord(e, st) != hipSuccess) return;
  g_recs[g_open[kernel]].stop = e;
  g_open[kernel] = -1;
}

}  // namespace dmgqa

using namespace dmgqa;

extern "C" {

int docmask_gqa_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  g_recs.clear();
  g_used = 0;
  for (int i = 0; i < kNumKernels; ++i) g_open[i] = -1;
  return DMGQA_OK;
}

int docmask_gqa_timing_read(int kernel, double* total_ms, int* launches) {
  if (kernel < 0 || kernel >= kNumKernels || !total_ms || !launches) return DMGQA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  double tot = 0.0;
  int n = 0;
  for (const Rec& r : g_recs) {
    if (r.kernel != kernel || !r.stop) continue;
    if (hipEventSynchronize(r.stop) != hipSuccess) return DMGQA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return DMGQA_ERR_HIP;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return DMGQA_OK;
}

int docmask_gqa_kernel_count(void) { return kNumKernels; }

const char* docmask_gqa_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < kNumKernels) ? kNames[kernel] : "";
}

}  // extern "C"
