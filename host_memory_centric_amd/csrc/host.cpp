// Host side of the layer-streamed trainer: unit layout, the pageable master
// store, the just-in-time packer, pinned buffers and asynchronous copies, the
// SIMD host Adam, the embedding gather/scatter and the RoPE tables.
//
// Design notes (MegaTrain paper page, appendix A.1 "Host (CPU) Memory
// Management" and A.3 "GPU Buffer Management"; hyper.ai summary, method):
// every unit's state is one contiguous block with 4 KB-aligned regions so a
// layer moves in one DMA burst; the store itself is pageable and only a few
// fixed-size staging buffers are pinned, so pinned memory does not grow with
// depth.
#include <hip/hip_runtime_api.h>
#include <immintrin.h>
#include <fcntl.h>
#include <sys/mman.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <cmath>
#include <cerrno>
#include <cstdarg>
#include <cstring>
#include <mutex>
#include <thread>
#include <vector>

#include "common.h"

namespace mt {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

static void hip_check(hipError_t e, const char* what) {
    if (e != hipSuccess) MT_FAIL(MT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// layout
// ---------------------------------------------------------------------------
void check_cfg(const mt_model_cfg* cfg) {
    MT_CHECK_ARG(cfg != nullptr, "cfg is NULL");
    if (cfg->layers < 1 || cfg->hidden < 8 || cfg->heads < 1 || cfg->head_dim < 8 || cfg->ffn < 8 ||
        cfg->vocab < 8)
        MT_FAIL(MT_E_SHAPE, "non-positive model dimension");
    if ((int64_t)cfg->heads * cfg->head_dim != cfg->hidden)
        MT_FAIL(MT_E_SHAPE, "hidden (%d) != heads (%d) * head_dim (%d)", cfg->hidden, cfg->heads,
                cfg->head_dim);
    if (cfg->hidden % 8 || cfg->ffn % 8 || cfg->vocab % 8 || cfg->head_dim % 8)
        MT_FAIL(MT_E_SHAPE, "hidden, ffn, vocab and head_dim must be multiples of 8");
    if (!(cfg->eps > 0.f) || !(cfg->rope_base > 1.f)) MT_FAIL(MT_E_ARG, "bad eps or rope_base");
    if (cfg->tied != 0 && cfg->tied != 1) MT_FAIL(MT_E_ARG, "tied must be 0 or 1");
}

mt_unit_layout layout_of(const mt_model_cfg* cfg, int unit, uint32_t flags) {
    check_cfg(cfg);
    MT_CHECK_ARG((flags & ~(uint32_t)(MT_STORE_MASTER_FP32 | MT_STORE_GRAD_ACCUM | MT_STORE_PINNED_DMA)) == 0,
                 "unknown store flags %u", flags);
    mt_unit_layout L;
    memset(&L, 0, sizeof(L));
    const uint64_t h = cfg->hidden, f = cfg->ffn, V = cfg->vocab;
    uint64_t numel[6] = {0, 0, 0, 0, 0, 0};
    if (unit >= 0) {
        MT_CHECK_ARG(unit < cfg->layers, "unit %d out of range", unit);
        L.n_tensors = 6;
        numel[0] = h;          // attention RMSNorm gain
        numel[1] = 3 * h * h;  // fused QKV
        numel[2] = h * h;      // output projection
        numel[3] = h;          // MLP RMSNorm gain
        numel[4] = 2 * f * h;  // fused gate/up
        numel[5] = h * f;      // down projection
    } else if (unit == MT_UNIT_EMBED) {
        L.n_tensors = 1;
        numel[0] = V * h;
    } else if (unit == MT_UNIT_HEAD) {
        L.n_tensors = cfg->tied ? 1 : 2;
        numel[0] = h;                    // final RMSNorm gain
        numel[1] = cfg->tied ? 0 : V * h;  // LM head (the embedding when tied)
    } else {
        MT_FAIL(MT_E_ARG, "unknown unit %d", unit);
    }
    uint64_t off = 0;
    for (int j = 0; j < L.n_tensors; ++j) {
        L.tensor_off[j] = off;
        L.tensor_numel[j] = numel[j];
        L.params += numel[j];
        off = round_up(off + 2 * numel[j], MT_TENSOR_ALIGN);
    }
    L.w_bytes = off;
    const uint64_t elems = L.w_bytes / 2;
    const uint64_t rb[6] = {L.w_bytes, L.w_bytes, 4 * elems, 4 * elems,
                            (flags & MT_STORE_MASTER_FP32) ? 4 * elems : 0,
                            (flags & MT_STORE_GRAD_ACCUM) ? 4 * elems : 0};
    uint64_t pos = 0;
    for (int r = 0; r < 6; ++r) {
        L.region_off[r] = pos;
        L.region_bytes[r] = round_up(rb[r], MT_BLOCK_ALIGN);
        pos += L.region_bytes[r];
    }
    L.block_bytes = pos;
    return L;
}

// ---------------------------------------------------------------------------
// host worker threads: a blocking parallel-for over [0, n)
// ---------------------------------------------------------------------------
static std::atomic<int> g_threads{0};

static int n_threads() {
    int t = g_threads.load();
    if (t > 0) return t;
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof(set), &set) == 0) t = CPU_COUNT(&set);
    if (t <= 0) t = (int)std::thread::hardware_concurrency();
    return std::max(1, t);
}

// Threads of the optimizer calls (mt_step, mt_grad_accumulate); 0: n_threads().
static std::atomic<int> g_opt_threads{0};

// One persistent pool of host workers shared by every parallel host pass
// (packer copies, Adam, accumulation, embedding gradient, fill, save/load).
// A pass is a job split into chunks; the calling thread works on its own
// job's chunks and the pool's workers help, taking chunks from the active
// job of highest priority: the packer's copies (priority 1, on the weight
// stream's critical path) go before optimizer work (priority 0) when both
// run at once.  No thread is created per call; passes from several host
// threads run concurrently on the same workers.
class WorkerPool {
  public:
    struct Job {
        uint64_t n = 0, grain = 1, chunks = 0;
        const std::function<void(uint64_t, uint64_t)>* fn = nullptr;
        int prio = 0;
        int max_helpers = 0;               // workers allowed on the job at once (besides the caller)
        std::atomic<uint64_t> next{0};
        std::atomic<uint64_t> done{0};
        int helpers = 0;                   // workers inside a chunk of this job (pool mutex)
        std::exception_ptr err;
        std::mutex err_mu;

        // Runs chunks until none is left; returns the number run.
        uint64_t work(bool one) {
            uint64_t ran = 0;
            for (;;) {
                const uint64_t c = next.fetch_add(1);
                if (c >= chunks) break;
                try {
                    (*fn)(c * grain, std::min(n, (c + 1) * grain));
                } catch (...) {
                    std::lock_guard<std::mutex> lk(err_mu);
                    if (!err) err = std::current_exception();
                }
                done.fetch_add(1);
                ++ran;
                if (one) break;
            }
            return ran;
        }
    };

    static WorkerPool& get() {
        static WorkerPool* pool = new WorkerPool();  // never destroyed: workers may outlive static destructors
        return *pool;
    }

    void run(Job& j) {
        ensure_workers();
        {
            std::lock_guard<std::mutex> lk(mu_);
            active_.push_back(&j);
        }
        cv_work_.notify_all();
        j.work(false);
        std::unique_lock<std::mutex> lk(mu_);
        cv_done_.wait(lk, [&] { return j.done.load() == j.chunks && j.helpers == 0; });
        active_.erase(std::find(active_.begin(), active_.end(), &j));
    }

  private:
    std::mutex mu_;
    std::condition_variable cv_work_, cv_done_;
    std::vector<Job*> active_;
    std::vector<std::thread> workers_;

    // Grows the pool to n_threads() - 1 workers (the caller is the n-th).
    void ensure_workers() {
        const int want = n_threads() - 1;
        std::lock_guard<std::mutex> lk(mu_);
        while ((int)workers_.size() < want) {
            workers_.emplace_back([this] { loop(); });
            workers_.back().detach();
        }
    }

    Job* pick() {  // under mu_: the highest-priority job with chunks left and room for a helper
        Job* best = nullptr;
        for (Job* j : active_)
            if (j->next.load() < j->chunks && j->helpers < j->max_helpers && (!best || j->prio > best->prio))
                best = j;
        return best;
    }

    void loop() {
        for (;;) {
            Job* j;
            {
                std::unique_lock<std::mutex> lk(mu_);
                cv_work_.wait(lk, [&] { return (j = pick()) != nullptr; });
                ++j->helpers;
            }
            j->work(true);  // one chunk, then look again: a higher-priority job may have arrived
            bool finished;
            {
                std::lock_guard<std::mutex> lk(mu_);
                --j->helpers;
                finished = j->done.load() == j->chunks && j->helpers == 0;
            }
            if (finished) cv_done_.notify_all();
        }
    }
};

// Blocking parallel-for over [0, n) in chunks of `grain` on the worker pool;
// at most max_threads threads (0: all) work on it, the caller included.
template <class F>
static void parallel_for(uint64_t n, uint64_t grain, F&& fn, int max_threads = 0, int prio = 0) {
    if (n == 0) return;
    const uint64_t chunks = (n + grain - 1) / grain;
    const int nt = (int)std::min<uint64_t>(chunks, (uint64_t)(max_threads > 0 ? max_threads : n_threads()));
    if (nt <= 1) {
        fn(0, n);
        return;
    }
    const std::function<void(uint64_t, uint64_t)> f = [&](uint64_t b, uint64_t e) { fn(b, e); };
    WorkerPool::Job j;
    j.n = n;
    j.grain = grain;
    j.chunks = chunks;
    j.fn = &f;
    j.prio = prio;
    j.max_helpers = nt - 1;
    WorkerPool::get().run(j);
    if (j.err) std::rethrow_exception(j.err);
}

static bool have_avx512();

// Copy with non-temporal stores: the destination (a pinned staging buffer read
// next by the DMA engine) is not read back into the caches first, which saves
// a third of the copy's DRAM traffic.
__attribute__((target("avx512f"))) static void stream_copy(char* dst, const char* src, uint64_t n) {
    uint64_t i = 0;
    for (; i + 256 <= n; i += 256) {
        const __m512i a = _mm512_loadu_si512(src + i), b = _mm512_loadu_si512(src + i + 64),
                      c = _mm512_loadu_si512(src + i + 128), d = _mm512_loadu_si512(src + i + 192);
        _mm512_stream_si512((__m512i*)(dst + i), a);
        _mm512_stream_si512((__m512i*)(dst + i + 64), b);
        _mm512_stream_si512((__m512i*)(dst + i + 128), c);
        _mm512_stream_si512((__m512i*)(dst + i + 192), d);
    }
    if (i < n) memcpy(dst + i, src + i, n - i);
    _mm_sfence();
}

static void par_memcpy(void* dst, const void* src, uint64_t bytes) {
    const uint64_t grain = 4ull << 20;
    const bool nt = have_avx512() && ((uintptr_t)dst & 63) == 0;
    parallel_for(bytes, grain, [&](uint64_t b, uint64_t e) {
        if (nt)
            stream_copy((char*)dst + b, (const char*)src + b, e - b);
        else
            memcpy((char*)dst + b, (const char*)src + b, e - b);
    }, 0, /*prio=*/1);
}

// ---------------------------------------------------------------------------
// store
// ---------------------------------------------------------------------------
}  // namespace mt

// Each unit's block is held as two segments: [W | G], the part the DMA
// engines read and write, and [M | V | P | A], the optimizer's part.  In a
// pageable store both lie in one mapping (seg1 = seg0 + region_off[2]); with
// MT_STORE_PINNED_DMA the first is page-locked (hipHostMalloc) and the second
// a separate pageable mapping.  Index: unit + 2 (embed, head, layers...).
struct mt_store {
    mt_model_cfg cfg;
    uint32_t flags = 0;                  // MT_STORE_* flags
    std::vector<char*> seg0, seg1;
    std::vector<uint64_t> mapped_bytes;  // mmap length of each unit's pageable mapping
    std::vector<mt_unit_layout> layouts;
    std::vector<int64_t> n_accum;        // micro-batch gradients in A since the unit's last step
};

namespace mt {

static int unit_index(const mt_store* st, int unit) {
    MT_CHECK_ARG(st != nullptr, "store is NULL");
    MT_CHECK_ARG(unit >= MT_UNIT_HEAD && unit < st->cfg.layers, "unit %d out of range", unit);
    return unit + 2;
}

// Address of region r (0..5: W, G, M, V, P, A) of the unit at index idx.
static char* region_ptr(const mt_store* st, size_t idx, int r) {
    const mt_unit_layout& L = st->layouts[idx];
    return r < 2 ? st->seg0[idx] + L.region_off[r] : st->seg1[idx] + (L.region_off[r] - L.region_off[2]);
}

static void* map_block(uint64_t bytes) {
    void* p = mmap(nullptr, bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1,
                   0);
    if (p == MAP_FAILED) MT_FAIL(MT_E_NOMEM, "mmap of %llu bytes failed", (unsigned long long)bytes);
    madvise(p, bytes, MADV_HUGEPAGE);
    return p;
}

// ---------------------------------------------------------------------------
// seeded generator (SplitMix64 in counter form; Box-Muller normals)
// ---------------------------------------------------------------------------
static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static inline uint64_t rng_u(uint32_t seed, uint32_t stream, uint64_t i) {
    const uint64_t key = ((uint64_t)seed << 48) | ((uint64_t)stream << 32) | i;
    return mix64(key * 0x9E3779B97F4A7C15ull);
}
static inline uint16_t f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static inline float bf16_to_f32(uint16_t b) {
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static void fill_normal(uint16_t* dst, uint64_t n, uint32_t seed, uint32_t stream, double std) {
    parallel_for(n, 1 << 16, [&](uint64_t b, uint64_t e) {
        for (uint64_t i = b; i < e; ++i) {
            const uint64_t a = rng_u(seed, stream, 2 * i), c = rng_u(seed, stream, 2 * i + 1);
            const double u1 = (double)((a >> 11) + 1) * 0x1.0p-53;
            const double u2 = (double)(c >> 11) * 0x1.0p-53;
            const double z = std::sqrt(-2.0 * std::log(u1)) * std::cos(2.0 * M_PI * u2);
            dst[i] = f32_to_bf16((float)(std * z));
        }
    });
}

// ---------------------------------------------------------------------------
// Adam (fp32, one IEEE rounding per operation; no contraction)
// ---------------------------------------------------------------------------
// Adam constants, each computed in fp64 and rounded once to fp32.  The bias
// corrections are folded into the step size and epsilon:
// alpha = lr * sqrt(c2) / c1, eps_hat = eps * sqrt(c2) with c1 = 1 - beta1^t,
// c2 = 1 - beta2^t, which is the bias-corrected update
// lr * (m / c1) / (sqrt(v / c2) + eps) rewritten with one division and one
// square root per element.
struct AdamK {
    float b1, b2, omb1, omb2, alpha, eps_hat, decay;
    bool wd;
};

static AdamK adam_consts(const mt_adam_cfg* a, int64_t t) {
    AdamK k;
    const double c1 = 1.0 - std::pow(a->beta1, (double)t), c2 = 1.0 - std::pow(a->beta2, (double)t);
    k.b1 = (float)a->beta1;
    k.b2 = (float)a->beta2;
    k.omb1 = (float)(1.0 - a->beta1);
    k.omb2 = (float)(1.0 - a->beta2);
    k.alpha = (float)(a->lr * std::sqrt(c2) / c1);
    k.eps_hat = (float)(a->eps * std::sqrt(c2));
    k.decay = (float)(1.0 - a->lr * a->weight_decay);
    k.wd = a->weight_decay != 0.0;
    return k;
}

#pragma clang fp contract(off)
static void adam_scalar(uint16_t* W, uint16_t* G, float* M, float* Vv, const uint16_t* src, float* wout,
                        uint64_t b, uint64_t e, const AdamK& k) {
    for (uint64_t i = b; i < e; ++i) {
        if (src) G[i] = src[i];
        float w = bf16_to_f32(W[i]);
        if (k.wd) w = w * k.decay;
        const float g = bf16_to_f32(G[i]);
        const float m = k.b1 * M[i] + k.omb1 * g;
        const float v = k.b2 * Vv[i] + k.omb2 * (g * g);
        M[i] = m;
        Vv[i] = v;
        const float denom = std::sqrt(v) + k.eps_hat;
        const float step = k.alpha * m;
        const float wn = w - step / denom;
        if (wout) wout[i] = wn;
        W[i] = f32_to_bf16(wn);
    }
}

__attribute__((target("avx512f,avx512bw"))) static void adam_avx512(uint16_t* W, uint16_t* G, float* M,
                                                                      float* Vv, const uint16_t* src,
                                                                      float* wout, uint64_t b, uint64_t e,
                                                                      const AdamK& k) {
    const __m512 b1 = _mm512_set1_ps(k.b1), b2 = _mm512_set1_ps(k.b2), omb1 = _mm512_set1_ps(k.omb1),
                 omb2 = _mm512_set1_ps(k.omb2), alpha = _mm512_set1_ps(k.alpha), eps = _mm512_set1_ps(k.eps_hat),
                 dec = _mm512_set1_ps(k.decay);
    const __m512i rnd = _mm512_set1_epi32(0x7fff), one = _mm512_set1_epi32(1);
    const bool g_aligned = ((uintptr_t)(G + b) & 31) == 0;
    uint64_t i = b;
    for (; i + 16 <= e; i += 16) {
        __m256i gb;
        if (src) {
            gb = _mm256_loadu_si256((const __m256i*)(src + i));
            if (g_aligned)
                _mm256_stream_si256((__m256i*)(G + i), gb);  // G is not read again here
            else
                _mm256_storeu_si256((__m256i*)(G + i), gb);
        } else {
            gb = _mm256_loadu_si256((const __m256i*)(G + i));
        }
        const __m256i wb = _mm256_loadu_si256((const __m256i*)(W + i));
        __m512 w = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(wb), 16));
        if (k.wd) w = _mm512_mul_ps(w, dec);
        const __m512 g = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(gb), 16));
        const __m512 m = _mm512_add_ps(_mm512_mul_ps(b1, _mm512_loadu_ps(M + i)), _mm512_mul_ps(omb1, g));
        const __m512 v = _mm512_add_ps(_mm512_mul_ps(b2, _mm512_loadu_ps(Vv + i)),
                                       _mm512_mul_ps(omb2, _mm512_mul_ps(g, g)));
        _mm512_storeu_ps(M + i, m);
        _mm512_storeu_ps(Vv + i, v);
        const __m512 denom = _mm512_add_ps(_mm512_sqrt_ps(v), eps);
        const __m512 step = _mm512_mul_ps(alpha, m);
        const __m512 wn = _mm512_sub_ps(w, _mm512_div_ps(step, denom));
        if (wout) _mm512_storeu_ps(wout + i, wn);
        // round to nearest even (weights are finite)
        __m512i u = _mm512_castps_si512(wn);
        u = _mm512_add_epi32(u, _mm512_add_epi32(rnd, _mm512_and_si512(_mm512_srli_epi32(u, 16), one)));
        _mm256_storeu_si256((__m256i*)(W + i), _mm512_cvtepi32_epi16(_mm512_srli_epi32(u, 16)));
    }
    if (src && g_aligned) _mm_sfence();
    if (i < e) adam_scalar(W, G, M, Vv, src, wout, i, e, k);
}
// Adam with the optional regions (same operation order as adam_scalar): P,
// the fp32 master weights, replaces W as the weight read and receives w';
// with A (k >= 1 accumulated micro-batches) the gradient landed in G is
// bf16((A + bf16 src) / nf), nf = k + 1, src = the last micro-batch's
// gradient (the slab, or G itself).
static void adam_ex_scalar(uint16_t* W, uint16_t* G, float* M, float* Vv, float* P, const float* A, float nf,
                           const uint16_t* src, float* wout, uint64_t b, uint64_t e, const AdamK& k) {
    for (uint64_t i = b; i < e; ++i) {
        if (A) {
            const float s = A[i] + bf16_to_f32(src ? src[i] : G[i]);
            G[i] = f32_to_bf16(s / nf);
        } else if (src) {
            G[i] = src[i];
        }
        float w = P ? P[i] : bf16_to_f32(W[i]);
        if (k.wd) w = w * k.decay;
        const float g = bf16_to_f32(G[i]);
        const float m = k.b1 * M[i] + k.omb1 * g;
        const float v = k.b2 * Vv[i] + k.omb2 * (g * g);
        M[i] = m;
        Vv[i] = v;
        const float denom = std::sqrt(v) + k.eps_hat;
        const float step = k.alpha * m;
        const float wn = w - step / denom;
        if (wout) wout[i] = wn;
        if (P) P[i] = wn;
        W[i] = f32_to_bf16(wn);
    }
}

__attribute__((target("avx512f,avx512bw"))) static inline __m512 bf16x16_to_f32(__m256i b) {
    return _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(b), 16));
}
// round to nearest even (finite values)
__attribute__((target("avx512f,avx512bw"))) static inline __m256i f32x16_to_bf16(__m512 x) {
    __m512i u = _mm512_castps_si512(x);
    u = _mm512_add_epi32(u, _mm512_add_epi32(_mm512_set1_epi32(0x7fff),
                                              _mm512_and_si512(_mm512_srli_epi32(u, 16), _mm512_set1_epi32(1))));
    return _mm512_cvtepi32_epi16(_mm512_srli_epi32(u, 16));
}

__attribute__((target("avx512f,avx512bw"))) static void adam_ex_avx512(uint16_t* W, uint16_t* G, float* M,
                                                                         float* Vv, float* P, const float* A,
                                                                         float nf, const uint16_t* src,
                                                                         float* wout, uint64_t b, uint64_t e,
                                                                         const AdamK& k) {
    const __m512 b1 = _mm512_set1_ps(k.b1), b2 = _mm512_set1_ps(k.b2), omb1 = _mm512_set1_ps(k.omb1),
                 omb2 = _mm512_set1_ps(k.omb2), alpha = _mm512_set1_ps(k.alpha), eps = _mm512_set1_ps(k.eps_hat),
                 dec = _mm512_set1_ps(k.decay), nfv = _mm512_set1_ps(nf);
    uint64_t i = b;
    for (; i + 16 <= e; i += 16) {
        __m256i gb;
        if (A) {
            const __m256i lb = _mm256_loadu_si256((const __m256i*)((src ? src : G) + i));
            const __m512 s = _mm512_add_ps(_mm512_loadu_ps(A + i), bf16x16_to_f32(lb));
            gb = f32x16_to_bf16(_mm512_div_ps(s, nfv));
            _mm256_storeu_si256((__m256i*)(G + i), gb);
        } else if (src) {
            gb = _mm256_loadu_si256((const __m256i*)(src + i));
            _mm256_storeu_si256((__m256i*)(G + i), gb);
        } else {
            gb = _mm256_loadu_si256((const __m256i*)(G + i));
        }
        __m512 w = P ? _mm512_loadu_ps(P + i) : bf16x16_to_f32(_mm256_loadu_si256((const __m256i*)(W + i)));
        if (k.wd) w = _mm512_mul_ps(w, dec);
        const __m512 g = bf16x16_to_f32(gb);
        const __m512 m = _mm512_add_ps(_mm512_mul_ps(b1, _mm512_loadu_ps(M + i)), _mm512_mul_ps(omb1, g));
        const __m512 v = _mm512_add_ps(_mm512_mul_ps(b2, _mm512_loadu_ps(Vv + i)),
                                       _mm512_mul_ps(omb2, _mm512_mul_ps(g, g)));
        _mm512_storeu_ps(M + i, m);
        _mm512_storeu_ps(Vv + i, v);
        const __m512 denom = _mm512_add_ps(_mm512_sqrt_ps(v), eps);
        const __m512 step = _mm512_mul_ps(alpha, m);
        const __m512 wn = _mm512_sub_ps(w, _mm512_div_ps(step, denom));
        if (wout) _mm512_storeu_ps(wout + i, wn);
        if (P) _mm512_storeu_ps(P + i, wn);
        _mm256_storeu_si256((__m256i*)(W + i), f32x16_to_bf16(wn));
    }
    if (i < e) adam_ex_scalar(W, G, M, Vv, P, A, nf, src, wout, i, e, k);
}

// A = bf16 src (first micro-batch after a step) or A + bf16 src
static void accum_scalar(float* A, const uint16_t* src, bool first, uint64_t b, uint64_t e) {
    for (uint64_t i = b; i < e; ++i) A[i] = first ? bf16_to_f32(src[i]) : A[i] + bf16_to_f32(src[i]);
}

__attribute__((target("avx512f,avx512bw"))) static void accum_avx512(float* A, const uint16_t* src, bool first,
                                                                       uint64_t b, uint64_t e) {
    uint64_t i = b;
    for (; i + 16 <= e; i += 16) {
        const __m512 g = bf16x16_to_f32(_mm256_loadu_si256((const __m256i*)(src + i)));
        _mm512_storeu_ps(A + i, first ? g : _mm512_add_ps(_mm512_loadu_ps(A + i), g));
    }
    if (i < e) accum_scalar(A, src, first, i, e);
}
#pragma clang fp contract(on)

static bool have_avx512() {
    static const bool ok = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                           getenv("MT_NO_AVX512") == nullptr;
    return ok;
}

// P = fp32(W) for every unit of a master-weight store
static void sync_master(mt_store* st) {
    for (size_t idx = 0; idx < st->layouts.size(); ++idx) {
        const mt_unit_layout& L = st->layouts[idx];
        const uint16_t* W = (const uint16_t*)region_ptr(st, idx, 0);
        float* P = (float*)region_ptr(st, idx, 4);
        parallel_for(L.w_bytes / 2, 1 << 20, [&](uint64_t b, uint64_t e) {
            for (uint64_t i = b; i < e; ++i) P[i] = bf16_to_f32(W[i]);
        });
    }
}

// ---- checkpoint / resume ---------------------------------------------------
struct CkptHeader {
    char magic[8];  // "MTSTORE1"
    uint32_t version, flags;
    mt_model_cfg cfg;
    int64_t t;
    uint64_t n_units, total_bytes;
};
constexpr uint64_t kIoChunk = 64ull << 20;

struct Fd {
    int fd;
    ~Fd() {
        if (fd >= 0) close(fd);
    }
};

static void io_fail(const char* what, const char* path) { MT_FAIL(MT_E_IO, "%s %s: %s", what, path, strerror(errno)); }

// pread/pwrite of [off, off + n) in full, retrying short transfers
template <bool WRITE>
void io_all(int fd, char* buf, uint64_t n, uint64_t off, const char* path) {
    while (n > 0) {
        const ssize_t r = WRITE ? pwrite(fd, buf, n, (off_t)off) : pread(fd, buf, n, (off_t)off);
        if (r < 0 && errno == EINTR) continue;
        if (r <= 0) {
            if (r == 0) errno = EIO;
            io_fail(WRITE ? "write" : "read", path);
        }
        buf += r;
        off += (uint64_t)r;
        n -= (uint64_t)r;
    }
}

// Transfers every block to/from the file after the header (blocks in unit
// order, each in its layout's byte order whatever the store's segments), in
// chunks of at most 64 MB spread over the worker threads.
template <bool WRITE>
void io_blocks(mt_store* st, int fd, const char* path) {
    struct Job {
        char* mem;
        uint64_t n, file_off;
    };
    std::vector<Job> jobs;
    uint64_t pos = sizeof(CkptHeader);
    for (size_t i = 0; i < st->layouts.size(); ++i) {
        const mt_unit_layout& L = st->layouts[i];
        const uint64_t seg_lo[2] = {0, L.region_off[2]}, seg_hi[2] = {L.region_off[2], L.block_bytes};
        char* seg[2] = {st->seg0[i], st->seg1[i]};
        for (int k = 0; k < 2; ++k)
            for (uint64_t o = seg_lo[k]; o < seg_hi[k]; o += kIoChunk)
                jobs.push_back({seg[k] + (o - seg_lo[k]), std::min(kIoChunk, seg_hi[k] - o), pos + o});
        pos += L.block_bytes;
    }
    parallel_for(jobs.size(), 1, [&](uint64_t b, uint64_t e) {
        for (uint64_t j = b; j < e; ++j) io_all<WRITE>(fd, jobs[j].mem, jobs[j].n, jobs[j].file_off, path);
    });
}

}  // namespace mt

using namespace mt;

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* mt_last_error(void) { return g_err; }

int mt_set_threads(int n) {
    return guard([&] {
        MT_CHECK_ARG(n >= 0 && n <= 4096, "bad thread count %d", n);
        g_threads.store(n);
    });
}

int mt_set_optimizer_threads(int n) {
    return guard([&] {
        MT_CHECK_ARG(n >= 0 && n <= 4096, "bad thread count %d", n);
        g_opt_threads.store(n);
    });
}

int mt_unit_layout_get(const mt_model_cfg* cfg, int unit, mt_unit_layout* out) {
    return mt_unit_layout_get_ex(cfg, 0, unit, out);
}

int mt_unit_layout_get_ex(const mt_model_cfg* cfg, uint32_t flags, int unit, mt_unit_layout* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        *out = layout_of(cfg, unit, flags);
    });
}

int mt_store_create(const mt_model_cfg* cfg, mt_store** out) { return mt_store_create_ex(cfg, 0, out); }

int mt_store_create_ex(const mt_model_cfg* cfg, uint32_t flags, mt_store** out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        check_cfg(cfg);
        layout_of(cfg, 0, flags);  // validates the flags
        auto* st = new mt_store();
        st->cfg = *cfg;
        st->flags = flags;
        const bool pinned = flags & MT_STORE_PINNED_DMA;
        try {
            for (int u = MT_UNIT_HEAD; u < cfg->layers; ++u) {
                mt_unit_layout L = layout_of(cfg, u, flags);
                const uint64_t dma = L.region_off[2];  // [W | G]
                const uint64_t len = round_up(pinned ? L.block_bytes - dma : L.block_bytes, 2ull << 20);
                st->layouts.push_back(L);
                st->seg0.push_back(nullptr);
                st->seg1.push_back(nullptr);
                st->mapped_bytes.push_back(0);
                st->n_accum.push_back(0);
                char* m = (char*)map_block(len);
                st->mapped_bytes.back() = len;
                if (pinned) {
                    st->seg1.back() = m;
                    void* p = nullptr;
                    const hipError_t e = hipHostMalloc(&p, dma, hipHostMallocDefault);
                    if (e != hipSuccess)
                        MT_FAIL(e == hipErrorOutOfMemory ? MT_E_NOMEM : MT_E_HIP,
                                "page-locking the W and G regions of unit %d (%llu bytes): %s", u,
                                (unsigned long long)dma, hipGetErrorString(e));
                    st->seg0.back() = (char*)p;
                    parallel_for(dma, 8ull << 20, [&](uint64_t b, uint64_t e2) { memset((char*)p + b, 0, e2 - b); });
                } else {
                    st->seg0.back() = m;
                    st->seg1.back() = m + dma;
                }
            }
        } catch (...) {
            mt_store_destroy(st);
            throw;
        }
        *out = st;
    });
}

void mt_store_destroy(mt_store* st) {
    if (!st) return;
    const bool pinned = st->flags & MT_STORE_PINNED_DMA;
    for (size_t i = 0; i < st->layouts.size(); ++i) {
        if (pinned) {
            if (st->seg0[i]) (void)hipHostFree(st->seg0[i]);
            if (st->seg1[i]) munmap(st->seg1[i], st->mapped_bytes[i]);
        } else if (st->seg0[i]) {
            munmap(st->seg0[i], st->mapped_bytes[i]);
        }
    }
    delete st;
}

int mt_store_block(mt_store* st, int unit, void** block) {
    return guard([&] {
        MT_CHECK_ARG(block != nullptr, "block is NULL");
        const int idx = unit_index(st, unit);
        if (st->flags & MT_STORE_PINNED_DMA)
            MT_FAIL(MT_E_STATE, "a pinned-DMA store has no contiguous block; address regions with mt_store_region");
        *block = st->seg0[idx];
    });
}

int mt_store_region(mt_store* st, int unit, int region, void** ptr) {
    return guard([&] {
        MT_CHECK_ARG(ptr != nullptr, "ptr is NULL");
        const int idx = unit_index(st, unit);
        MT_CHECK_ARG(region >= 0 && region < 6, "region %d out of range", region);
        if (st->layouts[idx].region_bytes[region] == 0)
            MT_FAIL(MT_E_STATE, "region %d is not present in this store", region);
        *ptr = region_ptr(st, idx, region);
    });
}

int mt_store_bytes(const mt_store* st, uint64_t* out) {
    return guard([&] {
        MT_CHECK_ARG(st && out, "NULL argument");
        uint64_t s = 0;
        for (auto& L : st->layouts) s += L.block_bytes;
        *out = s;
    });
}

int mt_store_fill_normal(mt_store* st, uint32_t seed, double std_) {
    return guard([&] {
        MT_CHECK_ARG(st != nullptr, "store is NULL");
        MT_CHECK_ARG(seed < 65536, "seed must fit in 16 bits");
        for (int u = MT_UNIT_HEAD; u < st->cfg.layers; ++u) {
            const int idx = unit_index(st, u);
            const mt_unit_layout& L = st->layouts[idx];
            // zero every region first (first touch happens here, in parallel)
            const uint64_t dma = L.region_off[2];
            parallel_for(dma, 8ull << 20, [&](uint64_t b, uint64_t e) { memset(st->seg0[idx] + b, 0, e - b); });
            parallel_for(L.block_bytes - dma, 8ull << 20,
                         [&](uint64_t b, uint64_t e) { memset(st->seg1[idx] + b, 0, e - b); });
            char* w = region_ptr(st, idx, 0);
            for (int j = 0; j < L.n_tensors; ++j) {
                uint16_t* t = (uint16_t*)(w + L.tensor_off[j]);
                const uint64_t n = L.tensor_numel[j];
                const bool gain = (u >= 0 && (j == 0 || j == 3)) || (u == MT_UNIT_HEAD && j == 0);
                if (gain) {
                    for (uint64_t i = 0; i < n; ++i) t[i] = 0x3F80;  // 1.0
                } else {
                    uint32_t stream = u >= 0 ? 16u + 8u * (uint32_t)u + (uint32_t)j
                                             : (u == MT_UNIT_EMBED ? 1u : 3u);
                    fill_normal(t, n, seed, stream, std_);
                }
            }
        }
        if (st->flags & MT_STORE_MASTER_FP32) sync_master(st);
    });
}

int mt_store_sync_master(mt_store* st) {
    return guard([&] {
        MT_CHECK_ARG(st != nullptr, "store is NULL");
        if (!(st->flags & MT_STORE_MASTER_FP32)) MT_FAIL(MT_E_STATE, "the store has no master weights");
        sync_master(st);
    });
}

int mt_grad_accumulate(mt_store* st, int unit, const void* grad_src) {
    return guard([&] {
        const int idx = unit_index(st, unit);
        if (!(st->flags & MT_STORE_GRAD_ACCUM)) MT_FAIL(MT_E_STATE, "the store has no gradient accumulator");
        const mt_unit_layout& L = st->layouts[idx];
        float* A = (float*)region_ptr(st, idx, 5);
        const uint16_t* src = grad_src ? (const uint16_t*)grad_src : (const uint16_t*)region_ptr(st, idx, 1);
        const bool first = st->n_accum[idx] == 0;
        const bool simd = have_avx512();
        parallel_for(L.w_bytes / 2, 1 << 18, [&](uint64_t b, uint64_t e) {
            if (simd)
                accum_avx512(A, src, first, b, e);
            else
                accum_scalar(A, src, first, b, e);
        }, g_opt_threads.load());
        ++st->n_accum[idx];
    });
}


int mt_store_save(const mt_store* cst, const char* path, int64_t t) {
    return guard([&] {
        MT_CHECK_ARG(cst != nullptr && path != nullptr, "NULL argument");
        mt_store* st = const_cast<mt_store*>(cst);
        Fd f{open(path, O_WRONLY | O_CREAT | O_TRUNC, 0644)};
        if (f.fd < 0) io_fail("open", path);
        CkptHeader h;
        memset(&h, 0, sizeof(h));
        memcpy(h.magic, "MTSTORE1", 8);
        h.version = 1;
        h.flags = st->flags & ~(uint32_t)MT_STORE_PINNED_DMA;  // placement is not part of the format
        h.cfg = st->cfg;
        h.t = t;
        h.n_units = st->layouts.size();
        for (auto& L : st->layouts) h.total_bytes += L.block_bytes;
        io_all<true>(f.fd, (char*)&h, sizeof(h), 0, path);
        io_blocks<true>(st, f.fd, path);
        io_all<true>(f.fd, (char*)st->n_accum.data(), 8 * st->n_accum.size(), sizeof(h) + h.total_bytes, path);
        if (fsync(f.fd) != 0) io_fail("fsync", path);
    });
}

int mt_store_load(mt_store* st, const char* path, int64_t* t_out) {
    return guard([&] {
        MT_CHECK_ARG(st != nullptr && path != nullptr && t_out != nullptr, "NULL argument");
        Fd f{open(path, O_RDONLY)};
        if (f.fd < 0) io_fail("open", path);
        CkptHeader h;
        io_all<false>(f.fd, (char*)&h, sizeof(h), 0, path);
        uint64_t total = 0;
        for (auto& L : st->layouts) total += L.block_bytes;
        if (memcmp(h.magic, "MTSTORE1", 8) != 0 || h.version != 1)
            MT_FAIL(MT_E_ARG, "%s is not a store checkpoint", path);
        if (memcmp(&h.cfg, &st->cfg, sizeof(mt_model_cfg)) != 0 || h.flags != (st->flags & ~(uint32_t)MT_STORE_PINNED_DMA) ||
            h.n_units != st->layouts.size() || h.total_bytes != total)
            MT_FAIL(MT_E_ARG, "%s was written for another model config or store flags", path);
        io_blocks<false>(st, f.fd, path);
        io_all<false>(f.fd, (char*)st->n_accum.data(), 8 * st->n_accum.size(), sizeof(h) + total, path);
        *t_out = h.t;
    });
}

int mt_pack_layer(mt_store* st, int unit, void* dst, size_t dst_bytes) {
    return guard([&] {
        const int idx = unit_index(st, unit);
        const mt_unit_layout& L = st->layouts[idx];
        MT_CHECK_ARG(dst != nullptr, "dst is NULL");
        MT_CHECK_ARG(dst_bytes >= L.w_bytes, "dst holds %zu bytes, unit needs %llu", dst_bytes,
                     (unsigned long long)L.w_bytes);
        par_memcpy(dst, region_ptr(st, idx, 0), L.w_bytes);
    });
}

int mt_pack_head_tied(mt_store* st, void* dst, size_t dst_bytes) {
    return guard([&] {
        MT_CHECK_ARG(st != nullptr && dst != nullptr, "NULL argument");
        MT_CHECK_ARG(st->cfg.tied, "the model does not tie its embedding and head");
        mt_model_cfg untied = st->cfg;
        untied.tied = 0;
        const mt_unit_layout D = layout_of(&untied, MT_UNIT_HEAD);
        MT_CHECK_ARG(dst_bytes >= D.w_bytes, "dst holds %zu bytes, the head slot needs %llu", dst_bytes,
                     (unsigned long long)D.w_bytes);
        const int hi = unit_index(st, MT_UNIT_HEAD), ei = unit_index(st, MT_UNIT_EMBED);
        const char* hw = region_ptr(st, hi, 0);
        const char* ew = region_ptr(st, ei, 0);
        memset(dst, 0, D.tensor_off[1]);                                   // gain and its padding
        memcpy((char*)dst, hw, 2 * D.tensor_numel[0]);                     // final gain
        par_memcpy((char*)dst + D.tensor_off[1], ew, 2 * D.tensor_numel[1]);  // E as the LM head
    });
}

int mt_pinned_alloc(size_t bytes, void** out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr && bytes > 0, "bad arguments");
        void* p = nullptr;
        hip_check(hipHostMalloc(&p, bytes, hipHostMallocDefault), "hipHostMalloc");
        *out = p;
    });
}

int mt_pinned_free(void* p) {
    return guard([&] {
        if (p) hip_check(hipHostFree(p), "hipHostFree");
    });
}

int mt_host_copy(void* dst, const void* src, size_t bytes) {
    return guard([&] {
        MT_CHECK_ARG(dst && src, "NULL pointer");
        MT_CHECK_ARG((char*)dst + bytes <= (const char*)src || (const char*)src + bytes <= (char*)dst,
                     "the buffers overlap");
        if (bytes) par_memcpy(dst, src, bytes);
    });
}

int mt_copy_h2d(void* dst_dev, const void* src_host, size_t bytes, void* stream) {
    return guard([&] {
        MT_CHECK_ARG(dst_dev && src_host, "NULL pointer");
        hip_check(hipMemcpyAsync(dst_dev, src_host, bytes, hipMemcpyHostToDevice, (hipStream_t)stream),
                  "hipMemcpyAsync H2D");
    });
}

int mt_copy_d2h(void* dst_host, const void* src_dev, size_t bytes, void* stream) {
    return guard([&] {
        MT_CHECK_ARG(dst_host && src_dev, "NULL pointer");
        hip_check(hipMemcpyAsync(dst_host, src_dev, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream),
                  "hipMemcpyAsync D2H");
    });
}

int mt_step(mt_store* st, int unit, const void* grad_src, const mt_adam_cfg* adam, int64_t t,
            float* w_fp32_out) {
    return guard([&] {
        const int idx = unit_index(st, unit);
        MT_CHECK_ARG(adam != nullptr, "adam is NULL");
        MT_CHECK_ARG(t >= 1, "step counter must be >= 1");
        const mt_unit_layout& L = st->layouts[idx];
        uint16_t* W = (uint16_t*)region_ptr(st, idx, 0);
        uint16_t* G = (uint16_t*)region_ptr(st, idx, 1);
        float* M = (float*)region_ptr(st, idx, 2);
        float* Vv = (float*)region_ptr(st, idx, 3);
        const AdamK k = adam_consts(adam, t);
        const uint64_t n = L.w_bytes / 2;
        const uint16_t* src = (const uint16_t*)grad_src;
        const bool simd = have_avx512();
        float* P = (st->flags & MT_STORE_MASTER_FP32) ? (float*)region_ptr(st, idx, 4) : nullptr;
        const int64_t k_acc = st->n_accum[idx];
        const float* A = k_acc > 0 ? (const float*)region_ptr(st, idx, 5) : nullptr;
        if (!P && !A) {
            parallel_for(n, 1 << 18, [&](uint64_t b, uint64_t e) {
                if (simd)
                    adam_avx512(W, G, M, Vv, src, w_fp32_out, b, e, k);
                else
                    adam_scalar(W, G, M, Vv, src, w_fp32_out, b, e, k);
            }, g_opt_threads.load());
        } else {
            const float nf = (float)(k_acc + 1);
            parallel_for(n, 1 << 18, [&](uint64_t b, uint64_t e) {
                if (simd)
                    adam_ex_avx512(W, G, M, Vv, P, A, nf, src, w_fp32_out, b, e, k);
                else
                    adam_ex_scalar(W, G, M, Vv, P, A, nf, src, w_fp32_out, b, e, k);
            }, g_opt_threads.load());
        }
        st->n_accum[idx] = 0;
    });
}

int mt_embed_gather(mt_store* st, const int32_t* tok, int64_t T, void* dst) {
    return guard([&] {
        const int idx = unit_index(st, MT_UNIT_EMBED);
        MT_CHECK_ARG(tok && dst && T >= 0, "bad arguments");
        const uint64_t h = st->cfg.hidden;
        const uint16_t* E = (const uint16_t*)region_ptr(st, idx, 0);
        for (int64_t t = 0; t < T; ++t)
            MT_CHECK_ARG(tok[t] >= 0 && tok[t] < st->cfg.vocab, "token %d at %lld out of range", tok[t],
                         (long long)t);
        parallel_for((uint64_t)T, 256, [&](uint64_t b, uint64_t e) {
            for (uint64_t t = b; t < e; ++t) memcpy((uint16_t*)dst + t * h, E + (uint64_t)tok[t] * h, 2 * h);
        });
    });
}

// Embedding gradient into G: row v = bf16 of (init[v], or 0) + the rows
// dx0[t] with tok[t] = v taken in ascending t, accumulated in fp32.
static void embed_grad_rows(mt_store* st, const int32_t* tok, int64_t T, const float* dx0, const uint16_t* init) {
    const int idx = unit_index(st, MT_UNIT_EMBED);
    MT_CHECK_ARG(tok && dx0 && T >= 0, "bad arguments");
    const uint64_t h = st->cfg.hidden, V = st->cfg.vocab;
    for (int64_t t = 0; t < T; ++t)
        MT_CHECK_ARG(tok[t] >= 0 && tok[t] < st->cfg.vocab, "token out of range");
    uint16_t* G = (uint16_t*)region_ptr(st, idx, 1);
    // Positions grouped by token id, ascending position inside a group (a
    // stable counting sort), then one fp32 row sum per token.
    std::vector<int64_t> start(V + 1, 0), pos(T);
    for (int64_t t = 0; t < T; ++t) ++start[tok[t] + 1];
    for (uint64_t v = 0; v < V; ++v) start[v + 1] += start[v];
    {
        std::vector<int64_t> fill(start.begin(), start.end() - 1);
        for (int64_t t = 0; t < T; ++t) pos[fill[tok[t]]++] = t;
    }
    parallel_for(V, 64, [&](uint64_t v0, uint64_t v1) {
        std::vector<float> acc(h);
        for (uint64_t v = v0; v < v1; ++v) {
            uint16_t* g = G + v * h;
            const int64_t b = start[v], e = start[v + 1];
            if (b == e) {
                if (init)
                    memcpy(g, init + v * h, 2 * h);
                else
                    memset(g, 0, 2 * h);
                continue;
            }
            for (uint64_t c = 0; c < h; ++c) acc[c] = init ? bf16_to_f32(init[v * h + c]) : 0.f;
            for (int64_t i = b; i < e; ++i) {
                const float* src = dx0 + (uint64_t)pos[i] * h;
                for (uint64_t c = 0; c < h; ++c) acc[c] += src[c];
            }
            for (uint64_t c = 0; c < h; ++c) g[c] = f32_to_bf16(acc[c]);
        }
    });
}

int mt_embed_grad(mt_store* st, const int32_t* tok, int64_t T, const float* dx0) {
    return guard([&] { embed_grad_rows(st, tok, T, dx0, nullptr); });
}

int mt_embed_grad_tied(mt_store* st, const int32_t* tok, int64_t T, const float* dx0, const void* head_grad) {
    return guard([&] {
        MT_CHECK_ARG(st != nullptr && head_grad != nullptr, "NULL argument");
        MT_CHECK_ARG(st->cfg.tied, "the model does not tie its embedding and head");
        embed_grad_rows(st, tok, T, dx0, (const uint16_t*)head_grad);
    });
}

int mt_rope_tables(const mt_model_cfg* cfg, int32_t seq, float* cos_out, float* sin_out) {
    return guard([&] {
        check_cfg(cfg);
        MT_CHECK_ARG(seq >= 1 && cos_out && sin_out, "bad arguments");
        const int half = cfg->head_dim / 2;
        std::vector<double> theta(half);
        for (int i = 0; i < half; ++i)
            theta[i] = std::pow((double)cfg->rope_base, (-2.0 * (double)i) / (double)cfg->head_dim);
        parallel_for((uint64_t)seq, 1024, [&](uint64_t b, uint64_t e) {
            for (uint64_t s = b; s < e; ++s)
                for (int i = 0; i < half; ++i) {
                    const double a = (double)s * theta[i];
                    cos_out[s * half + i] = (float)std::cos(a);
                    sin_out[s * half + i] = (float)std::sin(a);
                }
        });
    });
}

}  // extern "C"
