// Live kernel timing: HIP events recorded around the launches of the timed
// kernel classes, on the launch's own stream, so that the average duration of
// a kernel can be measured while the training step runs.
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace mt {

namespace {
const char* kNames[PROF_N] = {"gemm_nt", "gemm_nn", "gemm_tn", "attn_fwd", "attn_bwd"};

struct Rec {
    int cls;
    double flops;
    hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
int64_t g_launches[PROF_N];
double g_ms[PROF_N], g_flops[PROF_N];

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) MT_FAIL(MT_E_HIP, "hipEventCreate failed");
    return e;
}
}  // namespace

ProfScope::ProfScope(ProfClass c, double flops, hipStream_t st) : s(st) {
    if (!g_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_mu);
    Rec r{(int)c, flops, take_event(), take_event()};
    if (hipEventRecord(r.a, s) != hipSuccess) MT_FAIL(MT_E_HIP, "hipEventRecord failed");
    g_recs.push_back(r);
    idx = (int)g_recs.size() - 1;
}

ProfScope::~ProfScope() {
    if (idx < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    (void)hipEventRecord(g_recs[idx].b, s);
}

}  // namespace mt

using namespace mt;

extern "C" {

int mt_prof_enable(int on) {
    return guard([&] { g_on.store(on != 0); });
}

int mt_prof_collect(mt_prof_entry* out, int max, int* n, int reset) {
    return guard([&] {
        MT_CHECK_ARG(n != nullptr && (max == 0 || out != nullptr), "bad arguments");
        std::lock_guard<std::mutex> lk(g_mu);
        for (auto& r : g_recs) {
            if (hipEventSynchronize(r.b) != hipSuccess) MT_FAIL(MT_E_HIP, "hipEventSynchronize failed");
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) MT_FAIL(MT_E_HIP, "hipEventElapsedTime failed");
            g_launches[r.cls] += 1;
            g_ms[r.cls] += ms;
            g_flops[r.cls] += r.flops;
            g_pool.push_back(r.a);
            g_pool.push_back(r.b);
        }
        g_recs.clear();
        int k = 0;
        for (int c = 0; c < PROF_N && k < max; ++c) {
            if (!g_launches[c]) continue;
            memset(&out[k], 0, sizeof(out[k]));
            strncpy(out[k].name, kNames[c], sizeof(out[k].name) - 1);
            out[k].launches = g_launches[c];
            out[k].ms = g_ms[c];
            out[k].flops = g_flops[c];
            ++k;
        }
        *n = k;
        if (reset) {
            memset(g_launches, 0, sizeof(g_launches));
            memset(g_ms, 0, sizeof(g_ms));
            memset(g_flops, 0, sizeof(g_flops));
        }
    });
}

}  // extern "C"
