// Per-launch tracing: event pairs per launcher, Chrome trace JSON on request.
#include "trace.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "dit.h"

namespace dit {

std::atomic<int> g_trace_flags{0};

namespace {

struct Record {
    char name[32];
    char args[96];
    hipEvent_t begin, end;
    hipStream_t stream;
};

std::mutex g_mu;
std::vector<Record> g_rec;          // capacity fixed at begin
size_t g_used = 0, g_dropped = 0;
hipEvent_t g_base = nullptr;
std::string g_env_path;
std::once_flag g_env_once;

bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(s, &st) == hipSuccess && st != hipStreamCaptureStatusNone;
}

void release_locked() {
    for (size_t i = 0; i < g_used; ++i) {
        (void)hipEventDestroy(g_rec[i].begin);
        (void)hipEventDestroy(g_rec[i].end);
    }
    if (g_base) (void)hipEventDestroy(g_base);
    g_base = nullptr;
    g_rec.clear();
    g_rec.shrink_to_fit();
    g_used = g_dropped = 0;
}

int begin_locked(int32_t capacity) {
    release_locked();
    if (hipEventCreate(&g_base) != hipSuccess) return DIT_ERR_HIP;
    if (hipEventRecord(g_base, nullptr) != hipSuccess) return DIT_ERR_HIP;
    g_rec.resize((size_t)capacity);
    g_trace_flags.fetch_or(1);
    return DIT_OK;
}

void json_escape(FILE *f, const char *s) {
    for (; *s; ++s) {
        if (*s == '"' || *s == '\\') fputc('\\', f);
        if ((unsigned char)*s >= 0x20) fputc(*s, f);
    }
}

}  // namespace

void trace_init_from_env() {
    std::call_once(g_env_once, [] {
        const char *dbg = getenv("DIT_DEBUG_SYNC");
        if (dbg && *dbg && strcmp(dbg, "0") != 0) g_trace_flags.fetch_or(2);
        const char *p = getenv("DIT_TRACE");
        if (p && *p && strcmp(p, "0") != 0) {
            g_env_path = strcmp(p, "1") == 0 ? "dit_trace.json" : p;
            std::lock_guard<std::mutex> lock(g_mu);
            (void)begin_locked(1 << 16);
        }
    });
}

void TraceScope::open(hipStream_t s, const char *name) {
    const int flags = g_trace_flags.load(std::memory_order_relaxed);
    const bool cap = capturing(s);
    debug_ = (flags & 2) && !cap;
    if (!(flags & 1) || cap) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!(g_trace_flags.load() & 1)) return;
    if (g_used >= g_rec.size()) {
        ++g_dropped;
        return;
    }
    Record &r = g_rec[g_used];
    if (hipEventCreate(&r.begin) != hipSuccess) return;
    if (hipEventCreate(&r.end) != hipSuccess) {
        (void)hipEventDestroy(r.begin);
        return;
    }
    snprintf(r.name, sizeof r.name, "%s", name);
    r.args[0] = 0;
    r.stream = s;
    (void)hipEventRecord(r.begin, s);
    slot_ = (int)g_used++;
    s_ = s;
    name_ = name;
}

void TraceScope::args(const char *fmt, ...) {
    if (slot_ < 0) return;
    std::lock_guard<std::mutex> lock(g_mu);
    if ((size_t)slot_ >= g_used) return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_rec[slot_].args, sizeof g_rec[slot_].args, fmt, ap);
    va_end(ap);
}

void TraceScope::close() {
    if (slot_ >= 0) {
        std::lock_guard<std::mutex> lock(g_mu);
        if ((size_t)slot_ < g_used) (void)hipEventRecord(g_rec[slot_].end, s_);
    }
    if (debug_) {
        const hipError_t e = hipStreamSynchronize(s_);
        if (e != hipSuccess)
            fprintf(stderr, "[dit] DIT_DEBUG_SYNC: %s failed: %s\n", name_ ? name_ : "launch", hipGetErrorString(e));
    }
}

}  // namespace dit

using namespace dit;

extern "C" {

int dit_trace_begin(int32_t capacity) {
    if (capacity <= 0 || capacity > (1 << 24)) return DIT_ERR_INVALID_ARG;
    trace_init_from_env();
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return DIT_ERR_NO_DEVICE;
    std::lock_guard<std::mutex> lock(g_mu);
    return begin_locked(capacity);
}

int dit_trace_end(const char *path) {
    trace_init_from_env();
    std::lock_guard<std::mutex> lock(g_mu);
    if (!(g_trace_flags.load() & 1)) return DIT_ERR_INVALID_ARG;   // not tracing
    g_trace_flags.fetch_and(~1);
    const char *out = path ? path : (g_env_path.empty() ? nullptr : g_env_path.c_str());
    int rc = DIT_OK;
    FILE *f = out ? fopen(out, "w") : nullptr;
    if (out && !f) rc = DIT_ERR_INVALID_ARG;
    if (f) {
        fprintf(f, "{\"displayTimeUnit\": \"ms\", \"otherData\": {\"library\": \"%s\", \"dropped\": %zu}, "
                   "\"traceEvents\": [\n", dit_version(), g_dropped);
        bool first = true;
        for (size_t i = 0; i < g_used; ++i) {
            const Record &r = g_rec[i];
            float t0 = 0.f, dt = 0.f;
            if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&t0, g_base, r.begin) != hipSuccess ||
                hipEventElapsedTime(&dt, r.begin, r.end) != hipSuccess) {
                rc = DIT_ERR_HIP;
                continue;
            }
            fprintf(f, "%s{\"name\": \"", first ? "" : ",\n");
            json_escape(f, r.name);
            fprintf(f, "\", \"ph\": \"X\", \"pid\": 0, \"tid\": %llu, \"ts\": %.3f, \"dur\": %.3f, \"args\": {\"shape\": \"",
                    (unsigned long long)(uintptr_t)r.stream, 1000.0 * t0, 1000.0 * dt);
            json_escape(f, r.args);
            fprintf(f, "\"}}");
            first = false;
        }
        fprintf(f, "\n]}\n");
        fclose(f);
    }
    release_locked();
    return rc;
}

}  // extern "C"
