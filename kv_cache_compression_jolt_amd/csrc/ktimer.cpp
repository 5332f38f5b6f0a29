// Kernel launch timers (see ktimer.h).
#include "ktimer.h"

#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

namespace jolt {

struct KTimer {
    std::string name;
    bool on = false;
    std::vector<hipEvent_t> pending;     // start, stop, start, stop, ...
    double total_ms = 0.0;
    int64_t launches = 0;
};

namespace {
std::mutex g_mu;
std::vector<KTimer *> g_timers;          // never freed: launch sites may hold pointers
std::atomic<int> g_active{0};

KTimer *lookup(const char *kernel) {
    for (KTimer *t : g_timers)
        if (t->name == kernel) return t;
    return nullptr;
}

// fold completed event pairs into the totals (caller holds g_mu)
hipError_t drain(KTimer *t, bool wait) {
    size_t i = 0;
    for (; i + 1 < t->pending.size(); i += 2) {
        hipEvent_t a = t->pending[i], b = t->pending[i + 1];
        if (wait) {
            if (hipError_t e = hipEventSynchronize(b); e != hipSuccess) return e;
        } else if (hipEventQuery(b) != hipSuccess) {
            break;
        }
        float ms = 0.f;
        if (hipError_t e = hipEventElapsedTime(&ms, a, b); e != hipSuccess) return e;
        t->total_ms += ms;
        ++t->launches;
        (void)hipEventDestroy(a);
        (void)hipEventDestroy(b);
    }
    t->pending.erase(t->pending.begin(), t->pending.begin() + (ptrdiff_t)i);
    return hipSuccess;
}
}  // namespace

KTimer *ktimer_find(const char *kernel) {
    if (g_active.load(std::memory_order_relaxed) == 0) return nullptr;
    std::lock_guard<std::mutex> lk(g_mu);
    KTimer *t = lookup(kernel);
    return (t && t->on) ? t : nullptr;
}

void ktimer_record(KTimer *t, hipStream_t s, bool start) {
    hipEvent_t ev;
    if (hipEventCreate(&ev) != hipSuccess) return;
    if (hipEventRecord(ev, s) != hipSuccess) {
        (void)hipEventDestroy(ev);
        return;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    // a start without its stop (failed record) is dropped with the next start
    if (start && (t->pending.size() & 1)) {
        (void)hipEventDestroy(t->pending.back());
        t->pending.pop_back();
    }
    if (!start && !(t->pending.size() & 1)) {
        (void)hipEventDestroy(ev);
        return;
    }
    t->pending.push_back(ev);
    if (t->pending.size() > 512) (void)drain(t, false);
}

hipError_t ktimer_enable(const char *kernel, bool on) {
    std::lock_guard<std::mutex> lk(g_mu);
    KTimer *t = lookup(kernel);
    if (!t) {
        if (!on) return hipSuccess;
        t = new KTimer();
        t->name = kernel;
        g_timers.push_back(t);
    }
    if (on && !t->on) {
        hipError_t e = drain(t, true);
        t->total_ms = 0.0;
        t->launches = 0;
        t->on = true;
        g_active.fetch_add(1);
        return e;
    }
    if (!on && t->on) {
        t->on = false;
        g_active.fetch_sub(1);
    }
    return hipSuccess;
}

hipError_t ktimer_read(const char *kernel, double *total_ms, int64_t *launches) {
    std::lock_guard<std::mutex> lk(g_mu);
    KTimer *t = lookup(kernel);
    if (!t) {
        *total_ms = 0.0;
        *launches = 0;
        return hipSuccess;
    }
    hipError_t e = drain(t, true);
    *total_ms = t->total_ms;
    *launches = t->launches;
    return e;
}

}  // namespace jolt
