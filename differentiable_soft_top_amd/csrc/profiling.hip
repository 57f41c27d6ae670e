// profiling.hip -- event pairs around selected kernel launches (diagnostic).
#include <atomic>
#include <mutex>
#include <string.h>
#include <vector>

#include "soft_topk.h"
#include "stk_prof.hpp"

namespace stk {

namespace {

const char* const kNames[kKernelCount] = {
    "sample", "filter", "select", "pass1", "band_hist", "band_scatter", "bucket_agg", "solve",
    "radix_upsweep", "radix_downsweep", "radix_scan", "tile_agg", "emit", "emit_finalize", "vjp_reduce", "vjp_apply", "reset",
    "rows_forward", "rows_backward", "curve_scan", "curve", "iterate",
};

struct Pair {
    int id;
    hipEvent_t start, stop;
};

std::atomic<uint32_t> g_mask{0};
std::mutex g_mu;
std::vector<Pair> g_pairs;        // recorded, unresolved
std::vector<hipEvent_t> g_free;   // reusable events
thread_local hipEvent_t t_open[kKernelCount];

hipEvent_t take_event()
{
    if (!g_free.empty()) {
        hipEvent_t e = g_free.back();
        g_free.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess)
        return nullptr;
    return e;
}

}  // namespace

const char* kernel_name(int id) { return (id >= 0 && id < kKernelCount) ? kNames[id] : "?"; }

void prof_before(int id, hipStream_t stream)
{
    if (!(g_mask.load(std::memory_order_relaxed) & (1u << id)))
        return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t e = take_event();
    t_open[id] = e;
    if (e)
        hipEventRecord(e, stream);
}

void prof_after(int id, hipStream_t stream)
{
    if (!(g_mask.load(std::memory_order_relaxed) & (1u << id)))
        return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t s = t_open[id];
    t_open[id] = nullptr;
    if (!s)
        return;
    hipEvent_t e = take_event();
    if (!e)
        return;
    hipEventRecord(e, stream);
    g_pairs.push_back(Pair{id, s, e});
}

}  // namespace stk

using namespace stk;

extern "C" {

int soft_topk_profile_kernel_count(void) { return kKernelCount; }

const char* soft_topk_profile_kernel_name(int id) { return kernel_name(id); }

int soft_topk_profile_begin(uint32_t kernel_mask)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Pair& p : g_pairs) {
        g_free.push_back(p.start);
        g_free.push_back(p.stop);
    }
    g_pairs.clear();
    g_mask.store(kernel_mask, std::memory_order_relaxed);
    return SOFT_TOPK_OK;
}

int soft_topk_profile_end(double* total_ms, int64_t* launches)
{
    g_mask.store(0, std::memory_order_relaxed);
    std::lock_guard<std::mutex> lk(g_mu);
    if (total_ms)
        memset(total_ms, 0, sizeof(double) * kKernelCount);
    if (launches)
        memset(launches, 0, sizeof(int64_t) * kKernelCount);
    int rc = SOFT_TOPK_OK;
    for (const Pair& p : g_pairs) {
        if (hipEventSynchronize(p.stop) != hipSuccess) {
            rc = SOFT_TOPK_EHIP;
            continue;
        }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
            rc = SOFT_TOPK_EHIP;
            continue;
        }
        if (total_ms)
            total_ms[p.id] += (double)ms;
        if (launches)
            launches[p.id] += 1;
        g_free.push_back(p.start);
        g_free.push_back(p.stop);
    }
    g_pairs.clear();
    return rc;
}

}  // extern "C"
