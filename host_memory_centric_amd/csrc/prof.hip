// Live kernel timing: HIP events recorded around the launches of the timed
// kernel classes, on the launch's own stream, so that the average duration of
// a kernel can be measured while the training step runs.
#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"
#include "device.h"
#include "kernels.h"

namespace mt {

namespace {
const char* kNames[PROF_N] = {"gemm_nt", "gemm_nn", "gemm_tn", "attn_fwd", "attn_bwd", "gemm_fwd16"};

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

// The timing events skip the system-scope fence that a default event
// performs when it is recorded (a cache writeback and invalidation): they
// only order the timestamps around a launch on its own stream, and the
// fence would perturb the kernels they time and the copies running beside
// them.
hipEvent_t new_event() {
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
        MT_FAIL(MT_E_HIP, "hipEventCreateWithFlags failed");
    return e;
}

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    return new_event();
}

// events created up front when timing is switched on, so that the timed
// launches do not create events (the pool grows on demand past this)
constexpr size_t PROF_POOL = 4096;
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

// MFMA probe: every wave runs four independent accumulator chains of
// v_mfma_f32_32x32x16_bf16 on register operands (no memory traffic), so the
// rate it reaches is what the matrix cores sustain at the clock the chip holds
// under that load.  The sink is written only if the sum of the accumulators
// equals a value it cannot take (the chains stay live).
constexpr int PROBE_WGS = 2048;  // 8 workgroups of 4 waves per CU on 256 CUs
constexpr int PROBE_CHAINS = 4;

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.125f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.0625f * (float)((lane * 3 + e) & 7));
    }
    f32x16 acc[PROBE_CHAINS];
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < PROBE_CHAINS; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < PROBE_CHAINS; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += acc[k][r];
    if (sum == -1.0f) sink[blockIdx.x] = sum;  // the products are non-negative
}

}  // namespace mt

using namespace mt;

extern "C" {

int mt_probe_mfma(int32_t iters, float* sink, void* stream, double* tflops) {
    return guard([&] {
        MT_CHECK_ARG(iters > 0 && sink != nullptr && tflops != nullptr, "bad arguments");
        const hipStream_t s = (hipStream_t)stream;
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess)
            MT_FAIL(MT_E_HIP, "hipEventCreate failed");
        // a warm-up fifth of the work, then the timed run
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(PROBE_WGS), dim3(256), 0, s, sink, std::max(1, iters / 5));
        hipError_t e = hipEventRecord(a, s);
        hipLaunchKernelGGL(mfma_probe_kernel, dim3(PROBE_WGS), dim3(256), 0, s, sink, iters);
        if (e == hipSuccess) e = hipGetLastError();
        if (e == hipSuccess) e = hipEventRecord(b, s);
        if (e == hipSuccess) e = hipEventSynchronize(b);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
        (void)hipEventDestroy(a);
        (void)hipEventDestroy(b);
        if (e != hipSuccess) MT_FAIL(MT_E_HIP, "mfma probe: %s", hipGetErrorString(e));
        const double flops = (double)PROBE_WGS * 4 * PROBE_CHAINS * (double)iters * 2.0 * 32 * 32 * 16;
        *tflops = flops / (ms * 1e-3) / 1e12;
    });
}

int mt_prof_enable(int on) {
    return guard([&] {
        if (on) {
            std::lock_guard<std::mutex> lk(g_mu);
            while (g_pool.size() < PROF_POOL) g_pool.push_back(new_event());
        }
        g_on.store(on != 0);
    });
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
