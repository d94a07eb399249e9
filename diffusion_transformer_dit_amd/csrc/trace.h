// Per-launch tracing of the library's kernels (internal header).
//
// With tracing on (dit_trace_begin, or DIT_TRACE=<path> in the environment),
// every launcher records a HIP event on its stream before and after its
// kernels, with the launcher's name and shape.  Nothing synchronises while
// recording: dit_trace_end waits for the recorded events, converts them to
// device times and writes Chrome trace JSON (one "X" event per launch, one
// track per stream), the per-operation GPU-time breakdown the ERNIE page's
// tracer produced (§IX "Per-Step Latency Breakdown").  Launches made while a
// stream is being captured into a HIP graph are not recorded (events inside a
// graph carry no timestamps).  DIT_DEBUG_SYNC=1 synchronises the stream after
// every launch and reports the first failing one (debugging only).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

namespace dit {

extern std::atomic<int> g_trace_flags;   // bit 0: tracing, bit 1: debug sync
void trace_init_from_env();

class TraceScope {
public:
    TraceScope(hipStream_t s, const char *name) {
        trace_init_from_env();
        if (g_trace_flags.load(std::memory_order_relaxed)) open(s, name);
    }
    ~TraceScope() {
        if (slot_ >= 0 || debug_) close();
    }
    bool on() const { return slot_ >= 0; }
    // shape annotation of the record (printf format); no-op when not tracing
    void args(const char *fmt, ...);

private:
    void open(hipStream_t s, const char *name);
    void close();
    hipStream_t s_ = nullptr;
    const char *name_ = nullptr;
    int slot_ = -1;
    bool debug_ = false;
};

}  // namespace dit
