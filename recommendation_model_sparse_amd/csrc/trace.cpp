// Optional kernel timing: HIP events around every kernel the library launches (see
// dlrm_trace_enable in dlrm_sparse.h).  Off by default; when off, a launch costs one relaxed
// atomic load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "dlrm_sparse.h"

namespace dlrm {
namespace {

struct Pending {
    const char *name;
    hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;            // launched, not yet read
std::vector<hipEvent_t> g_free;            // event pool
std::map<std::string, std::pair<int64_t, double>> g_done;  // name -> (launches, ms)
thread_local hipEvent_t t_open = nullptr;  // start event of the launch in progress

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

void drain_locked() {
    for (const Pending &p : g_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            auto &slot = g_done[p.name];
            slot.first += 1;
            slot.second += ms;
        }
        g_free.push_back(p.start);
        g_free.push_back(p.stop);
    }
    g_pending.clear();
}

}  // namespace

bool trace_on() { return g_on.load(std::memory_order_relaxed); }

void trace_begin(hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    t_open = take_event();
    if (t_open && hipEventRecord(t_open, s) != hipSuccess) {  // no record for this launch
        g_free.push_back(t_open);
        t_open = nullptr;
    }
}

void trace_end(const char *name, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!t_open) return;
    hipEvent_t stop = take_event();
    if (!stop) {
        g_free.push_back(t_open);
        t_open = nullptr;
        return;
    }
    if (hipEventRecord(stop, s) != hipSuccess) {
        g_free.push_back(t_open);
        g_free.push_back(stop);
        t_open = nullptr;
        return;
    }
    g_pending.push_back(Pending{name, t_open, stop});
    t_open = nullptr;
}

}  // namespace dlrm

extern "C" int dlrm_trace_enable(int on) {
    dlrm::g_on.store(on != 0, std::memory_order_relaxed);
    return DLRM_OK;
}

extern "C" int dlrm_trace_read(int32_t max_entries, char *names, int64_t *launches, double *ms,
                               int32_t *n_entries) {
    using namespace dlrm;
    if (max_entries < 0 || !n_entries || (max_entries > 0 && (!names || !launches || !ms)))
        return DLRM_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    int32_t i = 0;
    for (const auto &kv : g_done) {
        if (i >= max_entries) break;
        std::strncpy(names + 64 * i, kv.first.c_str(), 63);
        names[64 * i + 63] = '\0';
        launches[i] = kv.second.first;
        ms[i] = kv.second.second;
        ++i;
    }
    *n_entries = i;
    g_done.clear();
    return DLRM_OK;
}
