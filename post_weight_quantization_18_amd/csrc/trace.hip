// Device-time tracing of the library's kernel launches (instrumentation; it
// changes no result). While a trace is active on a host thread, every launch
// the library enqueues from that thread is bracketed by two HIP events recorded
// on the launch stream; stopping the trace waits for the last event and sums
// the durations per kernel family. Inactive, a launch site only reads one
// thread-local flag.
#include <vector>

#include "common.h"

namespace gptq {

namespace {

struct TraceRec {
  int fam;
  double work;
  hipEvent_t a, b;
};

struct TraceState {
  bool on = false;
  std::vector<TraceRec> recs;
  std::vector<hipEvent_t> pool;  // events owned by this thread's trace, reused
  size_t used = 0;
  bool failed = false;
};

thread_local TraceState g_trace;

hipEvent_t take_event() {
  TraceState& t = g_trace;
  if (t.used < t.pool.size()) return t.pool[t.used++];
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) {
    t.failed = true;
    return nullptr;
  }
  t.pool.push_back(e);
  ++t.used;
  return e;
}

const char* const kFamilyNames[GPTQ_TRACE_FAMILIES] = {
    "syrk", "syrk_reduce", "chain_load", "chain_panel", "chain_update", "chain_merge", "chain_store",
    "quant_prep", "colloop", "esplit", "tgemm", "pack", "order", "gemv", "syrk_transpose"};

}  // namespace

TraceScope::TraceScope(hipStream_t st, int fam, double work) : st_(st), idx_(-1) {
  TraceState& t = g_trace;
  if (!t.on || t.failed) return;
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b || hipEventRecord(a, st) != hipSuccess) {
    t.failed = true;
    return;
  }
  idx_ = (int)t.recs.size();
  t.recs.push_back(TraceRec{fam, work, a, b});
}

void TraceScope::end() {
  if (idx_ < 0) return;
  TraceState& t = g_trace;
  if (hipEventRecord(t.recs[idx_].b, st_) != hipSuccess) t.failed = true;
  idx_ = -1;
}

TracePause::TracePause() : was_on_(g_trace.on) { g_trace.on = false; }
TracePause::~TracePause() { g_trace.on = was_on_; }

}  // namespace gptq

using namespace gptq;

extern "C" {

int32_t gptq_trace_start(void) {
  TraceState& t = g_trace;
  if (t.on) return GPTQ_ERR_INVALID_ARG;
  t.on = true;
  t.failed = false;
  t.recs.clear();
  t.used = 0;
  return GPTQ_OK;
}

int32_t gptq_trace_stop(int64_t* launches, double* ms, double* work, int32_t n) {
  TraceState& t = g_trace;
  if (!t.on) return GPTQ_ERR_INVALID_ARG;
  t.on = false;
  for (int32_t k = 0; k < n; ++k) {
    if (launches) launches[k] = 0;
    if (ms) ms[k] = 0.0;
    if (work) work[k] = 0.0;
  }
  gptq_status_t st = t.failed ? GPTQ_ERR_HIP : GPTQ_OK;
  for (const TraceRec& r : t.recs) {
    float dt = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&dt, r.a, r.b) != hipSuccess) {
      st = GPTQ_ERR_HIP;
      break;
    }
    if (r.fam < n) {
      if (launches) launches[r.fam] += 1;
      if (ms) ms[r.fam] += dt;
      if (work) work[r.fam] += r.work;
    }
  }
  t.recs.clear();
  t.used = 0;
  t.failed = false;
  return st;
}

const char* gptq_trace_family(int32_t k) {
  return (k >= 0 && k < GPTQ_TRACE_FAMILIES) ? kFamilyNames[k] : "unknown";
}

}  // extern "C"
