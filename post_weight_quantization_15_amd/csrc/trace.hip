// Per-phase GPU time (the tracing facility of the library): when enabled,
// every launch group of a phase -- the statistics kernels, one damping
// attempt's factorisation, each column-chain launch, each lazy block update,
// and the rest of the column loop (grid fits, working-copy set-up, output
// re-layout) -- is bracketed by two hipEvents recorded on the caller's
// stream; gptq_trace_read waits for them and adds up the elapsed times.
// Disabled (the default), nothing is recorded.
#include <mutex>
#include <vector>

#include "common.h"

namespace gptq {
namespace {

struct Mark {
  hipEvent_t a, b;
  int phase;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Mark> g_pending;                 // recorded, not yet read
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_free;
double g_ms[kTracePhases] = {};
int64_t g_n[kTracePhases] = {};

}  // namespace

bool trace_on() {
  std::lock_guard<std::mutex> lock(g_mu);
  return g_on;
}

int trace_begin(hipStream_t st, int phase) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_on) return -1;
  Mark mk{nullptr, nullptr, phase};
  if (!g_free.empty()) {
    mk.a = g_free.back().first;
    mk.b = g_free.back().second;
    g_free.pop_back();
  } else if (hipEventCreate(&mk.a) != hipSuccess || hipEventCreate(&mk.b) != hipSuccess) {
    return -1;
  }
  if (hipEventRecord(mk.a, st) != hipSuccess) {
    g_free.emplace_back(mk.a, mk.b);
    return -1;
  }
  g_pending.push_back(mk);
  return static_cast<int>(g_pending.size()) - 1;
}

void trace_end(hipStream_t st, int token) {
  if (token < 0) return;
  std::lock_guard<std::mutex> lock(g_mu);
  if (token < static_cast<int>(g_pending.size()))
    (void)hipEventRecord(g_pending[token].b, st);
}

}  // namespace gptq

using namespace gptq;

extern "C" {

gptq_status gptq_trace_enable(int32_t enable) {
  if (enable != 0 && enable != 1) return GPTQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  g_on = enable == 1;
  return GPTQ_OK;
}

gptq_status gptq_trace_read(double* ms, int64_t* launches, int32_t reset) {
  if (!ms || (reset != 0 && reset != 1)) return GPTQ_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  gptq_status rc = GPTQ_OK;
  for (Mark& mk : g_pending) {
    float t = 0.0f;
    if (hipEventSynchronize(mk.b) != hipSuccess ||
        hipEventElapsedTime(&t, mk.a, mk.b) != hipSuccess)
      rc = GPTQ_ERR_HIP;
    g_ms[mk.phase] += t;
    g_n[mk.phase] += 1;
    g_free.emplace_back(mk.a, mk.b);
  }
  g_pending.clear();
  for (int p = 0; p < kTracePhases; ++p) {
    ms[p] = g_ms[p];
    if (launches) launches[p] = g_n[p];
    if (reset) {
      g_ms[p] = 0.0;
      g_n[p] = 0;
    }
  }
  return rc;
}

}  // extern "C"
