// gdr_timing.hip -- opt-in per-kernel timing with HIP events.
//
// For the kernels selected by gdr_timing_enable's mask, every launch is
// bracketed by two hipEvents recorded on the same stream, so the durations
// measured are those of the kernels as they run in the caller's sequence.
// gdr_timing_read waits for the recorded events, returns the summed
// durations and launch counts per kernel, and forgets them.  Disabled (the
// default), the hooks cost one relaxed atomic load per launch.
#include "gdr.h"
#include "gdr_internal.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace gdr {
namespace {

struct Rec {
    int id;
    hipEvent_t begin, end;
};

std::atomic<int> g_mask{0};
std::mutex g_mu;
std::vector<Rec> g_recs;            // launches recorded since the last read
std::vector<hipEvent_t> g_free;     // events ready for reuse
thread_local hipEvent_t t_open[kKernelCount] = {};

hipEvent_t take_event() {
    hipEvent_t e = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_free.empty()) {
            e = g_free.back();
            g_free.pop_back();
        }
    }
    if (!e && hipEventCreate(&e) != hipSuccess) e = nullptr;
    return e;
}

}  // namespace

const char* kernel_name(int id) {
    static const char* names[kKernelCount] = {"gdr_chunkmap", "gdr_intra", "gdr_scan", "gdr_output",
                                              "gdr_decode"};
    return (id >= 0 && id < kKernelCount) ? names[id] : "";
}

void timing_begin(int id, hipStream_t s) {
    if (!((g_mask.load(std::memory_order_relaxed) >> id) & 1)) return;
    hipEvent_t e = take_event();
    if (e && hipEventRecord(e, s) == hipSuccess) t_open[id] = e;
}

void timing_end(int id, hipStream_t s) {
    hipEvent_t b = t_open[id];
    if (!b) return;
    t_open[id] = nullptr;
    hipEvent_t e = take_event();
    if (!e || hipEventRecord(e, s) != hipSuccess) return;
    std::lock_guard<std::mutex> lk(g_mu);
    g_recs.push_back(Rec{id, b, e});
}

}  // namespace gdr

extern "C" {

gdr_status gdr_timing_enable(int kernel_mask) {
    gdr::g_mask.store(kernel_mask);
    return GDR_OK;
}

const char* gdr_timing_kernel_name(int32_t id) { return gdr::kernel_name(id); }

gdr_status gdr_timing_read(double* total_ms, int32_t* launches, int32_t n) {
    if (!total_ms || !launches || n < 1) return GDR_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < n; ++i) {
        total_ms[i] = 0.0;
        launches[i] = 0;
    }
    std::vector<gdr::Rec> recs;
    {
        std::lock_guard<std::mutex> lk(gdr::g_mu);
        recs.swap(gdr::g_recs);
    }
    gdr_status st = GDR_OK;
    for (const gdr::Rec& r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess)
            st = GDR_ERR_HIP;
        else if (r.id < n) {
            total_ms[r.id] += ms;
            launches[r.id] += 1;
        }
    }
    std::lock_guard<std::mutex> lk(gdr::g_mu);
    for (const gdr::Rec& r : recs) {
        gdr::g_free.push_back(r.begin);
        gdr::g_free.push_back(r.end);
    }
    return st;
}

}  // extern "C"
