// timing.cpp -- optional per-kernel timing with HIP events.
//
// When enabled (selscan_timing_enable), every kernel launch made by the
// entry points is bracketed by two events recorded on the launch's own
// stream.  selscan_timing_collect waits for the recorded events, sums the
// elapsed times per kernel name and releases the events.  Disabled, the
// bracket costs one relaxed atomic load per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "selscan.h"

namespace {

struct Pending {
    const char* name;
    hipEvent_t start, stop;
};

std::atomic<int> g_enabled{0};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_free;
// open brackets per stream (a launch helper opens and closes on one thread)
thread_local std::vector<Pending> t_open;

hipEvent_t take_event() {
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

namespace selscan {

void ktime_mark(const char* kernel, hipStream_t stream, bool begin) {
    if (!g_enabled.load(std::memory_order_relaxed)) return;
    if (begin) {
        hipEvent_t e;
        {
            std::lock_guard<std::mutex> lk(g_mu);
            e = take_event();
        }
        if (!e) return;
        if (hipEventRecord(e, stream) != hipSuccess) {
            std::lock_guard<std::mutex> lk(g_mu);
            g_free.push_back(e);
            return;
        }
        t_open.push_back({kernel, e, nullptr});
        return;
    }
    if (t_open.empty() || t_open.back().name != kernel) return;
    Pending p = t_open.back();
    t_open.pop_back();
    std::lock_guard<std::mutex> lk(g_mu);
    p.stop = take_event();
    if (!p.stop) {
        g_free.push_back(p.start);
        return;
    }
    if (hipEventRecord(p.stop, stream) != hipSuccess) {
        g_free.push_back(p.start);
        g_free.push_back(p.stop);
        return;
    }
    g_pending.push_back(p);
}

}  // namespace selscan

extern "C" selscan_status_t selscan_timing_enable(int on) {
    if (on != 0 && on != 1) return SELSCAN_ERR_INVALID_ARG;
    g_enabled.store(on, std::memory_order_relaxed);
    return SELSCAN_OK;
}

extern "C" int selscan_timing_collect(selscan_kernel_time_t* out, int max_entries) {
    if (max_entries < 0 || (max_entries > 0 && !out)) return -1;
    std::vector<Pending> todo;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        todo.swap(g_pending);
    }
    // keyed by name; names are string literals of the launchers
    std::map<std::string, selscan_kernel_time_t> acc;
    std::vector<std::string> order;
    int rc = 0;
    for (const Pending& p : todo) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
            rc = -2;
            continue;
        }
        auto it = acc.find(p.name);
        if (it == acc.end()) {
            selscan_kernel_time_t k;
            k.name = p.name;
            k.launches = 0;
            k.total_ms = 0.0;
            k.min_ms = 1e300;
            k.max_ms = 0.0;
            it = acc.emplace(p.name, k).first;
            order.push_back(p.name);
        }
        it->second.launches += 1;
        it->second.total_ms += ms;
        if (ms < it->second.min_ms) it->second.min_ms = ms;
        if (ms > it->second.max_ms) it->second.max_ms = ms;
    }
    {
        std::lock_guard<std::mutex> lk(g_mu);
        for (const Pending& p : todo) {
            g_free.push_back(p.start);
            g_free.push_back(p.stop);
        }
    }
    (void)hipGetLastError();
    if (rc) return rc;
    int n = 0;
    for (const std::string& k : order) {
        if (n < max_entries) out[n] = acc[k];
        ++n;
    }
    return n;
}
