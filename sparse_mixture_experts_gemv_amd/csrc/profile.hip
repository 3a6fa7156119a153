// Event-pair profiler behind moe_profile_start / moe_profile_stop /
// moe_profile_read. Events are created up front by moe_profile_start, so the
// profiled region itself creates nothing; recording stops silently when the
// requested capacity is used up.
#include <atomic>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "profile.hpp"

namespace smoe {
namespace {

struct Record {
    int id;
    hipEvent_t start, stop;
};

struct Profiler {
    std::mutex mu;
    std::atomic<bool> enabled{false};
    std::vector<hipEvent_t> pool;
    std::vector<Record> recs;
    size_t next = 0;
    int open_id = -1;
    hipEvent_t open_start = nullptr;
    double total_ms[kNumKernelIds] = {};
    int launches[kNumKernelIds] = {};
};

Profiler &prof() {
    static Profiler p;
    return p;
}

const char *kNames[kNumKernelIds] = {"route_logits_gemm", "route_topk_softmax", "smap_hist",  "smap_rowscan",
                                     "smap_assign",       "smap_empty",         "ffn_tile_table", "ffn_acc_zero",
                                     "ffn_gate_up_gemm",  "ffn_down_scatter_gemm", "ffn_finalize",
                                     "ffn_combine",       "pl_gemm",            "pl_dx_gemm", "pl_wgrad_gemm",
                                     "pl_prep",           "pl_finalize",        "bwd_recompute_gemm",
                                     "bwd_dh_gemm",       "bwd_prep",           "bwd_wgrad_gemm", "bwd_dx_gemm",
                                     "smap_small"};

}  // namespace

const char *kernel_name(int id) { return (id >= 0 && id < kNumKernelIds) ? kNames[id] : "unknown"; }

void prof_begin(hipStream_t stream, int id) {
    Profiler &p = prof();
    if (!p.enabled.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.next + 2 > p.pool.size()) return;
    p.open_start = p.pool[p.next++];
    p.open_id = id;
    (void)hipEventRecord(p.open_start, stream);
}

void prof_end(hipStream_t stream, int id) {
    Profiler &p = prof();
    if (!p.enabled.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> g(p.mu);
    if (p.open_id != id || p.next + 1 > p.pool.size()) return;
    hipEvent_t stop = p.pool[p.next++];
    (void)hipEventRecord(stop, stream);
    p.recs.push_back(Record{id, p.open_start, stop});
    p.open_id = -1;
}

}  // namespace smoe

extern "C" {

int moe_profile_start(int capacity) {
    using namespace smoe;
    if (capacity < 1) return MOE_ERR_INVALID_ARGUMENT;
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    for (hipEvent_t e : p.pool) (void)hipEventDestroy(e);
    p.pool.clear();
    p.recs.clear();
    p.next = 0;
    p.open_id = -1;
    for (int i = 0; i < kNumKernelIds; ++i) {
        p.total_ms[i] = 0.0;
        p.launches[i] = 0;
    }
    p.pool.resize((size_t)capacity * 2);
    for (auto &e : p.pool)
        if (hipEventCreate(&e) != hipSuccess) return MOE_ERR_LAUNCH;
    p.recs.reserve((size_t)capacity);
    p.enabled.store(true);
    return MOE_OK;
}

int moe_profile_stop(void) {
    using namespace smoe;
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.enabled.store(false);
    for (const Record &r : p.recs) {
        if (hipEventSynchronize(r.stop) != hipSuccess) return MOE_ERR_LAUNCH;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return MOE_ERR_LAUNCH;
        p.total_ms[r.id] += ms;
        p.launches[r.id] += 1;
    }
    p.recs.clear();
    return MOE_OK;
}

int moe_profile_kinds(void) { return smoe::kNumKernelIds; }

int moe_profile_read(int kernel, const char **name, double *total_ms, int *launches) {
    using namespace smoe;
    if (kernel < 0 || kernel >= kNumKernelIds) return MOE_ERR_INVALID_ARGUMENT;
    Profiler &p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (name) *name = kernel_name(kernel);
    if (total_ms) *total_ms = p.total_ms[kernel];
    if (launches) *launches = p.launches[kernel];
    return MOE_OK;
}

}  // extern "C"
