// bf16 GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation (and the same kernels on fp16 operands, v_mfma_f32_32x32x16_f16,
// for the forward maps, whose activations are kept in fp16 and whose weights
// are converted to fp16 and transposed to [in, out], so that the forward runs
// in the input-gradient orientation below), for the layer
// template's linear maps (QKV, output, gate/up and
// down projections and the LM head) in the three orientations the forward and
// backward need:
//   forward      Y[T, out]  = X[T, in] * W[out, in]^T   A K-major, B K-major
//   input grad   dX[T, in]  = dY[T, out] * W[out, in]   A K-major, B N-major
//   weight grad  dW[out,in] = dY[T, out]^T * X[T, in]   A M-major, B N-major
//
// Large operands (M, N >= 256, K in whole steps of 32) run gemm_pp_kernel
// (gemm_pp.h): 256x256 output tiles, one workgroup of 8 waves per CU, each
// wave 128x64, two waves per SIMD that take turns: one reads its fragments
// from LDS and issues the direct global->LDS loads of a later K sub-step
// while the other runs its MFMAs, with one workgroup barrier per phase.  K
// advances in sub-steps of 32 through a four-slot LDS ring that the loads
// keep three sub-steps ahead.  The output tile is written through LDS as
// whole 512-byte rows (per-lane scattered stores cost a fifth of the kernel).
// gemm_pipe_kernel (gemm_pipe.h; MT_GEMM_IMPL=pipe) is the earlier design of
// the same tiles with one wave per SIMD (4 waves of 128x128) interleaving its
// own loads, reads and MFMAs; it is 12-20 % slower on the 7B layer shapes.
// Smaller operands use gemm_kernel (gemm_kernel.h): 256x256 or 128x128
// tiles of 8 or 4 waves and a two-slot ring of 64-wide K steps, with
// zero-filled partial K steps.
//
// Either way an operand whose contraction index is strided (the N-major
// weight in dX, both operands of dW) is copied into LDS as it lies and read
// with the transposing ds_read_b64_tr_b16, so no orientation needs register
// staging.  Every output element accumulates its products in the same K order
// in every kernel, so results do not depend on which kernel runs.  The
// weight-gradient GEMMs reduce over all tokens; when their tile grid is too
// small to fill 256 CUs they split K into fixed slices whose fp32 partials
// are summed in slice order by a second kernel: results never depend on
// scheduling (no atomics).
#include <cstdlib>
#include <cstring>

#include "gemm_pp.h"

namespace mt {

// Sum split-K partials in slice order: out = sum_s part[s] (+R), then the
// same output semantics as the GEMM epilogue; 4 consecutive outputs of a row
// per thread (N is a multiple of 8).
__global__ void splitk_reduce_kernel(const float* part, int splits, int64_t M, int64_t N, float* Cf,
                                     uint16_t* Cb, const uint16_t* R, int64_t ldc, int accumulate) {
    const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int64_t total = M * N;
    if (idx >= total) return;
    const int64_t m = idx / N, n = idx % N;
    float4 v = *(const float4*)(part + idx);
    for (int s = 1; s < splits; ++s) {
        const float4 w = *(const float4*)(part + (int64_t)s * total + idx);
        v.x += w.x;
        v.y += w.y;
        v.z += w.z;
        v.w += w.w;
    }
    const int64_t o = m * ldc + n;
    if (R) {
        const uint2 r = *(const uint2*)(R + o);
        v.x += bf_lo(r.x);
        v.y += bf_hi(r.x);
        v.z += bf_lo(r.y);
        v.w += bf_hi(r.y);
    }
    if (Cf) {
        if (accumulate) {
            const float4 c = *(const float4*)(Cf + o);
            *(float4*)(Cf + o) = make_float4(c.x + v.x, c.y + v.y, c.z + v.z, c.w + v.w);
        } else {
            *(float4*)(Cf + o) = v;
        }
    }
    if (Cb) *(uint2*)(Cb + o) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
}

static GemmArgs make_args(const GemmDesc& d, float* part, int splits, int64_t kps, int bm, int bn) {
    GemmArgs p;
    p.M = d.M;
    p.N = d.N;
    p.K = d.K;
    p.A = (const uint16_t*)d.A;
    p.lda = d.lda;
    p.B = (const uint16_t*)d.B;
    p.ldb = d.ldb;
    p.tiles_m = (int)((d.M + bm - 1) / bm);
    p.tiles_n = (int)((d.N + bn - 1) / bn);
    p.k_per_split = kps;
    p.epi = d.epi;
    p.rope_cos = d.rope_cos;
    p.rope_sin = d.rope_sin;
    p.rope_S = d.rope_S;
    p.rope_hd = d.rope_hd;
    p.rope_t0 = d.rope_t0;
    p.rope_cols = d.rope_cols;
    p.Ca = (uint16_t*)d.Ca;
    p.Ca16 = (uint16_t*)d.Ca16;
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
    return p;
}

template <int BM, int BN, int WM, int WN>
static void launch_tiles(const GemmDesc& d, hipStream_t s, float* part, int splits, int64_t kps) {
    const GemmArgs p = make_args(d, part, splits, kps, BM, BN);
    dim3 grid(p.tiles_m * p.tiles_n, splits);
    dim3 block(WM * WN * 64);
    if (d.f16 && d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true, true, true>), grid, block, 0, s, p);
    else if (d.f16)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true, false, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, true, false>), grid, block, 0, s, p);
    else if (!d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, false, true>), grid, block, 0, s, p);
}

static void launch_pipe(const GemmDesc& d, hipStream_t s, float* part, int splits, int64_t kps) {
    const GemmArgs p = make_args(d, part, splits, kps, 256, 256);
    dim3 grid(p.tiles_m * p.tiles_n, splits);
    dim3 block(256);
    if (d.a_kmajor && d.b_kmajor)
        hipLaunchKernelGGL((gemm_pipe_kernel<true, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_pipe_kernel<true, false>), grid, block, 0, s, p);
    else if (!d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_pipe_kernel<false, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((gemm_pipe_kernel<false, true>), grid, block, 0, s, p);
}

static void launch_pp(const GemmDesc& d, hipStream_t s, float* part, int splits, int64_t kps) {
    const GemmArgs p = make_args(d, part, splits, kps, 256, 256);
    dim3 grid(p.tiles_m * p.tiles_n, splits);
    dim3 block(512);
    if (d.f16 && d.b_kmajor)
        hipLaunchKernelGGL((gemm_pp_kernel<true, true, true>), grid, block, 0, s, p);
    else if (d.f16)
        hipLaunchKernelGGL((gemm_pp_kernel<true, false, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && d.b_kmajor)
        hipLaunchKernelGGL((gemm_pp_kernel<true, true>), grid, block, 0, s, p);
    else if (d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_pp_kernel<true, false>), grid, block, 0, s, p);
    else if (!d.a_kmajor && !d.b_kmajor)
        hipLaunchKernelGGL((gemm_pp_kernel<false, false>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((gemm_pp_kernel<false, true>), grid, block, 0, s, p);
}

// Kernel for large operands: MT_GEMM_IMPL=pipe selects the 4-wave pipelined
// kernel, anything else the 8-wave ping-pong kernel (read once per process).
static bool use_pp() {
    static const bool v = [] {
        const char* e = getenv("MT_GEMM_IMPL");
        return !(e && strcmp(e, "pipe") == 0);
    }();
    return v;
}

// The large-operand kernels need whole 256x256 tiles inside the operands (the
// last tile is moved back to the edge), K slices of whole 32-wide sub-steps,
// and per-lane byte offsets below 2^31 (256 rows or 64 k-rows of an operand).
static bool pipe_ok(const GemmDesc& d, int64_t kps) {
    return d.M >= 256 && d.N >= 256 && d.K % PBK == 0 && kps % PBK == 0 && d.lda < (1 << 22) &&
           d.ldb < (1 << 22);
}

bool gemm_epi_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb) {
    return M >= 256 && N >= 256 && N % 256 == 0 && K % PBK == 0 && lda < (1 << 22) && ldb < (1 << 22) &&
           gemm_pick_splits(M, N, K) == 1;
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

// Enqueue one GEMM (checked by gemm()) with the given K slices.
static void run_gemm(const GemmDesc& d, int splits, int64_t kps, hipStream_t s) {
    float* part = splits > 1 ? (float*)d.ws : nullptr;
    if (pipe_ok(d, kps)) {
        if (use_pp() || d.f16 || d.epi) launch_pp(d, s, part, splits, kps);
        else launch_pipe(d, s, part, splits, kps);
    }
    else if (use_big(d.M, d.N))
        launch_tiles<256, 256, 2, 4>(d, s, part, splits, kps);
    else
        launch_tiles<128, 128, 2, 2>(d, s, part, splits, kps);
    if (splits > 1) {
        const int64_t total = d.M * d.N;
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total / 4 + 255) / 256)), dim3(256), 0, s, part,
                           splits, d.M, d.N, d.Cf, (uint16_t*)d.Cb, (const uint16_t*)d.R, d.ldc, d.accumulate);
    }
}

static int compute_units() {
    static const int n = [] {
        int dev = 0, cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        return cu;
    }();
    return n;
}

// Tile columns of a GEMM that the last, partly filled round of workgroups
// holds, when it is worth running them apart; 0 otherwise.  The large-operand
// kernel runs one 256x256 tile per CU, so 640 tiles on 256 CUs are 2.5 rounds
// with half the machine idle in the third.  With a long contraction (K >= 8192)
// the columns of whole rounds go first and the remaining columns run with K
// split in two, which fills the last round with half-length tiles (-6 % to
// -12 % at 8192 x 5120 and K = 13824..27648; shorter K loses to the partial
// sums' extra traffic).  Needs whole tiles, a plain epilogue and a workspace
// for the partials.
static int64_t tail_columns(const GemmDesc& d) {
    if (d.epi || !d.ws || d.M % 256 || d.N % 256 || d.K < 8192 || d.K % (2 * PBK)) return 0;
    if (gemm_pick_splits(d.M, d.N, d.K) != 1 || !pipe_ok(d, d.K)) return 0;
    const int64_t tm = d.M / 256, tn = d.N / 256, cu = compute_units();
    const int64_t rem = (tm * tn) % cu;
    if (tm * tn < cu || rem == 0 || rem > cu / 2 || rem % tm) return 0;
    const int64_t nt = rem / tm;
    if (nt >= tn || d.ws_bytes < (size_t)(2 * d.M * nt * 256 * 4)) return 0;
    return nt * 256;
}

void gemm(const GemmDesc& d, hipStream_t s) {
    if (d.M <= 0 || d.N <= 0 || d.K <= 0 || d.M % 8 || d.N % 8 || d.K % 8 || d.lda % 8 || d.ldb % 8 ||
        d.ldc % 8)
        MT_FAIL(MT_E_SHAPE, "gemm: M=%lld N=%lld K=%lld lda=%lld ldb=%lld ldc=%lld must be positive multiples of 8",
                (long long)d.M, (long long)d.N, (long long)d.K, (long long)d.lda, (long long)d.ldb,
                (long long)d.ldc);
    if (!d.A || !d.B || (!d.Cf && !d.Cb && !d.epi)) MT_FAIL(MT_E_ARG, "gemm: NULL operand");
    if (((uintptr_t)d.A | (uintptr_t)d.B | (uintptr_t)d.Cf | (uintptr_t)d.Cb | (uintptr_t)d.R) & 15)
        MT_FAIL(MT_E_ALIGN, "gemm: operands must be 16-byte aligned");
    const int64_t a_rows_ld = d.a_kmajor ? d.K : d.M, b_rows_ld = d.b_kmajor ? d.K : d.N;
    if (d.lda < a_rows_ld || d.ldb < b_rows_ld || d.ldc < d.N) MT_FAIL(MT_E_SHAPE, "gemm: leading dimension too small");
    if (d.epi) {
        if (!d.f16 || d.epi > 2 || d.Cf || d.R || d.accumulate || !gemm_epi_ok(d.M, d.N, d.K, d.lda, d.ldb))
            MT_FAIL(MT_E_ARG, "gemm: fused epilogue %d not available for M=%lld N=%lld K=%lld", d.epi, (long long)d.M,
                    (long long)d.N, (long long)d.K);
        if (((uintptr_t)d.Ca | (uintptr_t)d.Ca16) & 15) MT_FAIL(MT_E_ALIGN, "gemm: outputs must be 16-byte aligned");
        if (d.epi == 1 && (!d.Cb || !d.rope_cos || !d.rope_sin || d.rope_S < 1 || (d.rope_hd != 64 && d.rope_hd != 128) ||
                           d.rope_cols % d.rope_hd || d.rope_cols > d.N))
            MT_FAIL(MT_E_ARG, "gemm: bad RoPE epilogue arguments");
        if (d.epi == 2 && !d.Cb && !d.Ca && !d.Ca16) MT_FAIL(MT_E_ARG, "gemm: SwiGLU epilogue without outputs");
    }
    if (d.f16 && !d.a_kmajor) MT_FAIL(MT_E_ARG, "gemm: fp16 operands need a K-major A");
    const ProfClass pc =
        d.f16 ? PROF_GEMM_FWD16 : d.a_kmajor ? (d.b_kmajor ? PROF_GEMM_NT : PROF_GEMM_NN) : PROF_GEMM_TN;
    ProfScope prof(pc, 2.0 * (double)d.M * (double)d.N * (double)d.K, s);
    const int64_t nt = tail_columns(d);
    if (nt > 0) {
        // columns [0, N - nt) in whole rounds, then [N - nt, N) with K in two halves
        GemmDesc head = d, tail = d;
        const int64_t n0 = d.N - nt;
        head.N = n0;
        tail.N = nt;
        tail.B = (const uint16_t*)d.B + (d.b_kmajor ? n0 * d.ldb : n0);
        if (d.Cf) tail.Cf = d.Cf + n0;
        if (d.Cb) tail.Cb = (uint16_t*)d.Cb + n0;
        if (d.R) tail.R = (const uint16_t*)d.R + n0;
        run_gemm(head, 1, d.K, s);
        run_gemm(tail, 2, d.K / 2, s);
        launch_check("gemm");
        return;
    }
    int splits = d.epi ? 1 : gemm_pick_splits(d.M, d.N, d.K);
    if (splits > 1 && (!d.ws || d.ws_bytes < (size_t)splits * d.M * d.N * 4)) splits = 1;
    const int BK = GBK;
    int64_t kps = d.K;
    if (splits > 1) {
        kps = ((d.K + splits - 1) / splits + BK - 1) / BK * BK;
        splits = (int)((d.K + kps - 1) / kps);
    }
    run_gemm(d, splits, kps, s);
    launch_check("gemm");
}

}  // namespace mt
