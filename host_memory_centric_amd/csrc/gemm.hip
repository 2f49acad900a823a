// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation, for the layer template's linear maps (QKV, output, gate/up and
// down projections and the LM head) in the three orientations the forward and
// backward need:
//   forward      Y[T, out]  = X[T, in] * W[out, in]^T   A K-major, B K-major
//   input grad   dX[T, in]  = dY[T, out] * W[out, in]   A K-major, B N-major
//   weight grad  dW[out,in] = dY[T, out]^T * X[T, in]   A M-major, B N-major
// Tiles are staged global -> registers -> LDS (double buffered, one barrier
// per K step).  An operand whose contraction index is not contiguous is
// loaded as 8x8 sub-blocks along its contiguous index (coalesced) and
// transposed in registers so the LDS tile is always [row][k], which is what
// the MFMA operand fetch wants.  The weight-gradient GEMMs reduce over all
// tokens; when their tile grid is too small to fill 256 CUs they split K into
// fixed slices whose fp32 partials are summed in slice order by a second
// kernel: results never depend on scheduling (no atomics).
#include "common.h"
#include "device.h"
#include "kernels.h"

namespace mt {

struct GemmArgs {
    int64_t M, N, K;
    const uint16_t* A;
    int64_t lda;
    const uint16_t* B;
    int64_t ldb;
    float* Cf;
    uint16_t* Cb;
    const uint16_t* R;
    int64_t ldc;
    int accumulate;
    int64_t k_per_split;   // multiple of BK; K slice of blockIdx.y
    int64_t split_stride;  // elements between partial outputs of successive slices (0: no split)
    int tiles_m, tiles_n;
};

// ---------------------------------------------------------------------------
// operand tile loaders
// ---------------------------------------------------------------------------
// K-major operand: rows [r0, r0+ROWS) of a [rows][K] matrix, k in [k0, k0+BK).
template <int ROWS, int BK, int NT>
struct KMajorLoader {
    static constexpr int VEC = ROWS * BK / 8;
    static constexpr int PER = (VEC + NT - 1) / NT;
    uint4 v[PER];
    __device__ __forceinline__ void load(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                         int64_t kend, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            v[i] = make_uint4(0, 0, 0, 0);
            if (u < VEC) {
                const int row = u / (BK / 8), kc = u % (BK / 8);
                const int64_t gr = r0 + row, gk = k0 + kc * 8;
                if (gr < rows && gk < kend) v[i] = *(const uint4*)(P + gr * ld + gk);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t* S, int tid, int ldsw) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < VEC) {
                const int row = u / (BK / 8), kc = u % (BK / 8);
                *(uint4*)(S + row * ldsw + kc * 8) = v[i];
            }
        }
    }
};

// MN-major operand: a [K][rows] matrix (rows contiguous).  Work unit = 8 k
// rows x 8 contiguous elements; lane -> (kq fastest, then column chunk).
template <int ROWS, int BK, int NT>
struct MNMajorLoader {
    static constexpr int UNITS = (BK / 8) * (ROWS / 8);
    static constexpr int PER = (UNITS + NT - 1) / NT;
    uint4 v[PER][8];
    __device__ __forceinline__ void load(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                         int64_t kend, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
#pragma unroll
            for (int r = 0; r < 8; ++r) v[i][r] = make_uint4(0, 0, 0, 0);
            if (u < UNITS) {
                const int kq = u % (BK / 8), mc = u / (BK / 8);
                const int64_t gm = r0 + mc * 8;
                if (gm < rows) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const int64_t gk = k0 + kq * 8 + r;
                        if (gk < kend) v[i][r] = *(const uint4*)(P + gk * ld + gm);
                    }
                }
            }
        }
    }
    __device__ __forceinline__ static uint32_t pick(const uint4& a, int e) {
        const uint32_t d = (e >> 1) == 0 ? a.x : (e >> 1) == 1 ? a.y : (e >> 1) == 2 ? a.z : a.w;
        return (e & 1) ? (d >> 16) : (d & 0xffffu);
    }
    __device__ __forceinline__ void store(uint16_t* S, int tid, int ldsw) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = tid + i * NT;
            if (u < UNITS) {
                const int kq = u % (BK / 8), mc = u / (BK / 8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint4 w;
                    w.x = pick(v[i][0], e) | (pick(v[i][1], e) << 16);
                    w.y = pick(v[i][2], e) | (pick(v[i][3], e) << 16);
                    w.z = pick(v[i][4], e) | (pick(v[i][5], e) << 16);
                    w.w = pick(v[i][6], e) | (pick(v[i][7], e) << 16);
                    *(uint4*)(S + (mc * 8 + e) * ldsw + kq * 8) = w;
                }
            }
        }
    }
};

template <bool KMAJ, int ROWS, int BK, int NT>
struct LoaderSel;
template <int ROWS, int BK, int NT>
struct LoaderSel<true, ROWS, BK, NT> {
    using type = KMajorLoader<ROWS, BK, NT>;
};
template <int ROWS, int BK, int NT>
struct LoaderSel<false, ROWS, BK, NT> {
    using type = MNMajorLoader<ROWS, BK, NT>;
};

// Tile order: blocks are dispatched round-robin over the 8 XCDs; give each
// XCD a contiguous run of tiles, and walk tiles in groups of GROUP_M tile rows
// so that concurrently running tiles share A rows and B columns in L2.
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tm, int tn, int& pm, int& pn) {
    constexpr int XCD = 8, GROUP_M = 8;
    if (nblk % XCD == 0) bid = (bid % XCD) * (nblk / XCD) + bid / XCD;
    const int in_group = GROUP_M * tn;
    const int g = bid / in_group;
    const int first = g * GROUP_M;
    const int gsz = min(tm - first, GROUP_M);
    const int r = bid % in_group;
    pm = first + r % gsz;
    pn = r / gsz;
}

template <int BM, int BN, int BK, int WM, int WN, bool AK, bool BKM>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int PAD = 8;
    constexpr int LDSW = BK + PAD;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1 && BK % 16 == 0, "bad tile");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][(BM + BN) * LDSW];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int pm, pn;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, pm, pn);
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const int64_t kbeg = (int64_t)blockIdx.y * p.k_per_split;
    const int64_t kend = min(p.K, kbeg + p.k_per_split);
    const int nk = (int)((kend - kbeg + BK - 1) / BK);

    typename LoaderSel<AK, BM, BK, NT>::type la;
    typename LoaderSel<BKM, BN, BK, NT>::type lb;
    const int tidb = (tid + NT / 2) % NT;  // spread A and B loads over different threads

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (nk > 0) {
        la.load(p.A, p.lda, p.M, m0, kbeg, kend, tid);
        lb.load(p.B, p.ldb, p.N, n0, kbeg, kend, tidb);
        la.store(smem[0], tid, LDSW);
        lb.store(smem[0] + BM * LDSW, tidb, LDSW);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int64_t k0 = kbeg + (int64_t)(kt + 1) * BK;
            la.load(p.A, p.lda, p.M, m0, k0, kend, tid);
            lb.load(p.B, p.ldb, p.N, n0, k0, kend, tidb);
        }
        const uint16_t* As = smem[cur];
        const uint16_t* Bs = smem[cur] + BM * LDSW;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            bf16x8 af[TM], bfm[TN];
            const int kc = kk * 16 + 8 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = as_bf16x8(*(const uint4*)(As + (wm * WTM + i * 32 + (lane & 31)) * LDSW + kc));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfm[j] = as_bf16x8(*(const uint4*)(Bs + (wn * WTN + j * 32 + (lane & 31)) * LDSW + kc));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfm[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) {
            la.store(smem[cur ^ 1], tid, LDSW);
            lb.store(smem[cur ^ 1] + BM * LDSW, tidb, LDSW);
        }
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
    float* Cf = p.Cf ? p.Cf + (int64_t)blockIdx.y * p.split_stride : nullptr;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + wn * WTN + j * 32 + (lane & 31);
            if (n >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m >= p.M) continue;
                const int64_t o = m * p.ldc + n;
                float v = acc[i][j][r];
                if (p.R) v += bf2f(p.R[o]);
                if (Cf) Cf[o] = p.accumulate ? Cf[o] + v : v;
                if (p.Cb) p.Cb[o] = f2bf(v);
            }
        }
}

// Sum split-K partials in slice order: out = sum_s part[s] (+R), then the
// same output semantics as the GEMM epilogue.
__global__ void splitk_reduce_kernel(const float* part, int splits, int64_t M, int64_t N, float* Cf,
                                     uint16_t* Cb, const uint16_t* R, int64_t ldc, int accumulate) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = M * N;
    if (idx >= total) return;
    const int64_t m = idx / N, n = idx % N;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += part[(int64_t)s * total + idx];
    const int64_t o = m * ldc + n;
    if (R) v += bf2f(R[o]);
    if (Cf) Cf[o] = accumulate ? Cf[o] + v : v;
    if (Cb) Cb[o] = f2bf(v);
}

template <int BM, int BN, int BK, int WM, int WN>
static void launch_tiles(const GemmDesc& d, hipStream_t s, float* part, int splits, int64_t kps) {
    GemmArgs p;
    p.M = d.M;
    p.N = d.N;
    p.K = d.K;
    p.A = (const uint16_t*)d.A;
    p.lda = d.lda;
    p.B = (const uint16_t*)d.B;
    p.ldb = d.ldb;
    p.tiles_m = (int)((d.M + BM - 1) / BM);
    p.tiles_n = (int)((d.N + BN - 1) / BN);
    p.k_per_split = kps;
    if (splits > 1) {
        p.Cf = part;
        p.Cb = nullptr;
        p.R = nullptr;
        p.ldc = d.N;
        p.accumulate = 0;
        p.split_stride = d.M * d.N;
    } else {
        p.Cf = d.Cf;
        p.Cb = (uint16_t*)d.Cb;
        p.R = (const uint16_t*)d.R;
        p.ldc = d.ldc;
        p.accumulate = d.accumulate;
        p.split_stride = 0;
    }
    dim3 grid(p.tiles_m * p.tiles_n, splits);
    dim3 block(WM * WN * 64);
    if (d.a_kmajor && d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, true, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, true, false>), grid, block, 0, s, p);
    else if (!d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, false, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, BK, WM, WN, false, true>), grid, block, 0, s, p);
}

size_t gemm_splitk_bytes(int64_t M, int64_t N, int64_t K) {
    const int s = gemm_pick_splits(M, N, K);
    return s > 1 ? (size_t)s * M * N * 4 : 0;
}

static bool use_big(int64_t M, int64_t N) { return M >= 1024 && N >= 1024; }

int gemm_pick_splits(int64_t M, int64_t N, int64_t K) {
    const int64_t bm = use_big(M, N) ? 256 : 128, bn = bm;
    const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int64_t target = 512;  // two waves of workgroups over 256 CUs
    if (tiles >= target) return 1;
    int64_t s = (target + tiles - 1) / tiles;
    s = std::min<int64_t>(s, K / 1024);  // keep >= 16 K steps of 64 per slice
    return (int)std::max<int64_t>(1, std::min<int64_t>(s, 16));
}

void gemm(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0 || d.M % 8 || d.N % 8 || d.K % 8 || d.lda % 8 || d.ldb % 8 ||
        d.ldc % 8)
        MT_FAIL(MT_E_SHAPE, "gemm: M=%lld N=%lld K=%lld lda=%lld ldb=%lld ldc=%lld must be positive multiples of 8",
                (long long)d.M, (long long)d.N, (long long)d.K, (long long)d.lda, (long long)d.ldb,
                (long long)d.ldc);
    if (!d.A || !d.B || (!d.Cf && !d.Cb)) MT_FAIL(MT_E_ARG, "gemm: NULL operand");
    if (((uintptr_t)d.A | (uintptr_t)d.B | (uintptr_t)d.Cf | (uintptr_t)d.Cb | (uintptr_t)d.R) & 15)
        MT_FAIL(MT_E_ALIGN, "gemm: operands must be 16-byte aligned");
    const int64_t a_rows_ld = d.a_kmajor ? d.K : d.M, b_rows_ld = d.b_kmajor ? d.K : d.N;
    if (d.lda < a_rows_ld || d.ldb < b_rows_ld || d.ldc < d.N) MT_FAIL(MT_E_SHAPE, "gemm: leading dimension too small");
    int splits = gemm_pick_splits(d.M, d.N, d.K);
    if (splits > 1 && (!d.ws || d.ws_bytes < (size_t)splits * d.M * d.N * 4)) splits = 1;
    const int BK = 64;
    int64_t kps = d.K;
    if (splits > 1) {
        kps = ((d.K + splits - 1) / splits + BK - 1) / BK * BK;
        splits = (int)((d.K + kps - 1) / kps);
    }
    float* part = splits > 1 ? (float*)d.ws : nullptr;
    const ProfClass pc = d.a_kmajor ? (d.b_kmajor ? PROF_GEMM_NT : PROF_GEMM_NN) : PROF_GEMM_TN;
    ProfScope prof(pc, 2.0 * (double)d.M * (double)d.N * (double)d.K, s);
    if (use_big(d.M, d.N))
        launch_tiles<256, 256, 64, 2, 4>(d, s, part, splits, kps);
    else
        launch_tiles<128, 128, 64, 2, 2>(d, s, part, splits, kps);
    if (splits > 1) {
        const int64_t total = d.M * d.N;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, part,
                           splits, d.M, d.N, d.Cf, (uint16_t*)d.Cb, (const uint16_t*)d.R, d.ldc, d.accumulate);
    }
    launch_check("gemm");
}

}  // namespace mt
