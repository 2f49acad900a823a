// The bf16 MFMA GEMM kernel template and its LDS tile helpers, shared by the
// translation units that instantiate it (see gemm.hip for the design).
#pragma once
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
    // Fused epilogues of the fp16 forward (gemm_pp_kernel only; whole 256-column tiles):
    //  epi 1: RoPE.  Output columns below rope_cols come in interleaved pairs, column
    //    2j + e of a head being feature j + e*hd/2; they are rotated by the angle of
    //    pair j at position (rope_t0 + row) % rope_S and stored de-interleaved, every
    //    column as fp16, into Cb.
    //  epi 2: SwiGLU.  Output column 2j + e is gate (e = 0) or up (e = 1) of feature j;
    //    Cb receives gate | up de-interleaved as bf16 ([M, N], optional), Ca silu(gate)*up
    //    as bf16 and Ca16 the same as fp16 ([M, N/2], optional).
    int epi;
    const float* rope_cos;
    const float* rope_sin;
    int rope_S, rope_hd;
    int64_t rope_t0, rope_cols;
    uint16_t* Ca;
    uint16_t* Ca16;
};

// ---------------------------------------------------------------------------
// LDS tiles.  Every operand tile holds 64 k values x ROWS rows, 32 KB for 256
// rows, and reaches LDS by direct global->LDS loads (global_load_lds_dwordx4:
// lane l of a wave instruction lands at byte 16*l of a contiguous 1 KB).
//
// K-major operand ([rows][K] in memory): LDS [row][64 k], 128-byte rows, the
// 16-byte chunk kc of row r at chunk kc ^ ((r >> 1) & 7).  MFMA fragments are
// plain 16-byte reads.
//
// MN-major operand ([K][rows] in memory): LDS [k][ROWS] as in memory, chunk c
// (8 rows) of k-row k at chunk c ^ (4 * (k & 3)).  Fragments come from
// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4r+q supplies 4
// consecutive rows of k-row kb+r and lane i receives row i of k-rows kb..kb+3,
// so two such reads give a lane its 8 contraction values.
//
// Both swizzles make the fragment reads bank-conflict free.
// ---------------------------------------------------------------------------
constexpr int GBK = 64;  // K step

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4s_t lds_v4s;

__device__ __forceinline__ int kswz(int kc, int row) { return kc ^ ((row >> 1) & 7); }
__device__ __forceinline__ int mswz(int c, int k) { return c ^ (4 * (k & 3)); }

template <int ROWS>
struct Tile {
    static constexpr int BYTES = ROWS * GBK * 2;
    static constexpr int INSTR = BYTES / 1024;  // 1 KB wave instructions per tile

    // Direct loads of a K-major tile; rows past `rows` are clamped (their
    // products land in rows/columns that are never stored).
    template <int NSW>
    __device__ __forceinline__ static void dma_k(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                                 uint16_t* T, int sw, int lane) {
#pragma unroll
        for (int jj = 0; jj < INSTR / NSW; ++jj) {
            const int j = sw + jj * NSW;  // 8-row group
            const int row = 8 * j + (lane >> 3);
            const int64_t gr = min(r0 + row, rows - 1);
            const uint16_t* g = P + gr * ld + k0 + 8 * kswz(lane & 7, row);
            __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(T + j * 512), 16, 0, 0);
        }
    }
    // Direct loads of an MN-major tile (2 k-rows per instruction).
    template <int NSW>
    __device__ __forceinline__ static void dma_mn(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                                  uint16_t* T, int sw, int lane) {
        constexpr int CPR = ROWS / 8;             // chunks per k-row
        constexpr int KPI = 64 / CPR;             // k-rows per instruction
        static_assert(KPI >= 1 && 64 % CPR == 0, "rows per tile");
#pragma unroll
        for (int jj = 0; jj < INSTR / NSW; ++jj) {
            const int j = sw + jj * NSW;
            const int k = KPI * j + lane / CPR;
            const int c = mswz(lane % CPR, k);
            const int64_t gm = min(r0 + 8 * c, rows - 8);
            const uint16_t* g = P + (k0 + k) * ld + gm;
            __builtin_amdgcn_global_load_lds((const void*)g, (lds_void*)(T + j * 512), 16, 0, 0);
        }
    }
    // Register path with zero fill for the last, partial K step.
    __device__ __forceinline__ static void sync_k(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                                  int64_t kend, uint16_t* T, int t, int nth) {
        for (int u = t; u < ROWS * GBK / 8; u += nth) {
            const int row = u / (GBK / 8), kc = u % (GBK / 8);
            const int64_t gr = r0 + row, gk = k0 + kc * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (gr < rows && gk < kend) v = *(const uint4*)(P + gr * ld + gk);
            *(uint4*)(T + row * GBK + 8 * kswz(kc, row)) = v;
        }
    }
    __device__ __forceinline__ static void sync_mn(const uint16_t* P, int64_t ld, int64_t rows, int64_t r0, int64_t k0,
                                                   int64_t kend, uint16_t* T, int t, int nth) {
        constexpr int CPR = ROWS / 8;
        for (int u = t; u < GBK * CPR; u += nth) {
            const int k = u / CPR, c = u % CPR;
            const int64_t gm = r0 + 8 * c;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (gm < rows && k0 + k < kend) v = *(const uint4*)(P + (k0 + k) * ld + gm);
            *(uint4*)(T + k * ROWS + 8 * mswz(c, k)) = v;
        }
    }
    // MFMA operand fragment (rows rbase .. rbase+31 of the tile, k step kk)
    __device__ __forceinline__ static bf16x8 frag_k(const uint16_t* T, int rbase, int kk, int lane) {
        const int row = rbase + (lane & 31);
        const int kc = kk * 2 + (lane >> 5);
        return as_bf16x8(*(const uint4*)(T + row * GBK + 8 * kswz(kc, row)));
    }
    __device__ __forceinline__ static bf16x8 frag_mn(const uint16_t* T, int rbase, int kk, int lane) {
        const int g = lane >> 4, j = lane & 15;
        const int r = j >> 2, q = j & 3;
        const int m = rbase + 16 * (g & 1) + 4 * q;     // 4 rows this lane supplies
        const int kb = kk * 16 + 8 * (g >> 1) + r;      // its k-row (first read)
        const int c = m >> 3, sub = (m & 7);            // chunk and offset (0 or 4)
        const uint16_t* a0 = T + kb * ROWS + 8 * mswz(c, kb) + sub;
        const uint16_t* a1 = T + (kb + 4) * ROWS + 8 * mswz(c, kb + 4) + sub;
        const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)a0);
        const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)a1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// Tile order: blocks are dispatched round-robin over the 8 XCDs; give each
// XCD a contiguous run of tiles, and walk tiles in groups of GROUP_M tile rows
// so that concurrently running tiles share A rows and B columns in L2.
template <int GROUP_M = 8>
__device__ __forceinline__ void tile_coords(int bid, int nblk, int tm, int tn, int& pm, int& pn) {
    constexpr int XCD = 8;
    if (nblk % XCD == 0) bid = (bid % XCD) * (nblk / XCD) + bid / XCD;
    const int in_group = GROUP_M * tn;
    const int g = bid / in_group;
    const int first = g * GROUP_M;
    const int gsz = min(tm - first, GROUP_M);
    const int r = bid % in_group;
    pm = first + r % gsz;
    pn = r / gsz;
}

// Store one 32x32 accumulator tile; (mb, n) = this lane's first row and its column.
__device__ __forceinline__ void store_acc(const f32x16& a, const GemmArgs& p, float* Cf, int64_t mb, int64_t n) {
    if (n >= p.N) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = mb + 8 * (r >> 2) + (r & 3);
        if (m < p.M) {
            const int64_t o = m * p.ldc + n;
            float v = a[r];
            if (p.R) v += bf2f(p.R[o]);
            if (Cf) Cf[o] = p.accumulate ? Cf[o] + v : v;
            if (p.Cb) p.Cb[o] = f2bf(v);
        }
    }
}

template <int BM, int BN, int WM, int WN, bool AK, bool BKM, bool F16 = false>
__global__ __launch_bounds__(WM* WN * 64) void gemm_kernel(GemmArgs p) {
    constexpr int NT = WM * WN * 64, NW = NT / 64, SW = NW / 2;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM >= 1 && TN >= 1 && NW % 2 == 0, "bad tile");
    using TA = Tile<BM>;
    using TB = Tile<BN>;
    static_assert(TA::INSTR % SW == 0 && TB::INSTR % SW == 0, "staging waves");
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2][(BM + BN) * GBK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    int pm, pn;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, pm, pn);
    const int64_t m0 = (int64_t)pm * BM, n0 = (int64_t)pn * BN;
    const int64_t kbeg = (int64_t)blockIdx.y * p.k_per_split;
    const int64_t kend = min(p.K, kbeg + p.k_per_split);
    const int nk = (int)((kend - kbeg + GBK - 1) / GBK);

    // waves 0 .. SW-1 load operand A, the others operand B (wave-uniform)
    const bool stage_a = wave < SW;
    const int sw = stage_a ? wave : wave - SW;
    auto issue = [&](int64_t k0, uint16_t* buf) {
        if (k0 + GBK <= kend) {
            if (stage_a) {
                if constexpr (AK) TA::template dma_k<SW>(p.A, p.lda, p.M, m0, k0, buf, sw, lane);
                else TA::template dma_mn<SW>(p.A, p.lda, p.M, m0, k0, buf, sw, lane);
            } else {
                if constexpr (BKM) TB::template dma_k<SW>(p.B, p.ldb, p.N, n0, k0, buf + BM * GBK, sw, lane);
                else TB::template dma_mn<SW>(p.B, p.ldb, p.N, n0, k0, buf + BM * GBK, sw, lane);
            }
        } else {  // last, partial K step: zero-filled register path over all threads
            if constexpr (AK) TA::sync_k(p.A, p.lda, p.M, m0, k0, kend, buf, tid, NT);
            else TA::sync_mn(p.A, p.lda, p.M, m0, k0, kend, buf, tid, NT);
            if constexpr (BKM) TB::sync_k(p.B, p.ldb, p.N, n0, k0, kend, buf + BM * GBK, tid, NT);
            else TB::sync_mn(p.B, p.ldb, p.N, n0, k0, kend, buf + BM * GBK, tid, NT);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto mfma_k = [&](const uint16_t* As, const uint16_t* Bs, int kk) {
        bf16x8 af[TM], bfm[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (AK) af[i] = TA::frag_k(As, wm * WTM + i * 32, kk, lane);
            else af[i] = TA::frag_mn(As, wm * WTM + i * 32, kk, lane);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (BKM) bfm[j] = TB::frag_k(Bs, wn * WTN + j * 32, kk, lane);
            else bfm[j] = TB::frag_mn(Bs, wn * WTN + j * 32, kk, lane);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = mfma32x16<F16>(af[i], bfm[j], acc[i][j]);
    };

    // One K step: start the direct loads of the next tile into the other
    // buffer, then consume this one.  The two buffers are passed as
    // restrict-qualified pointers: the compiler's wait insertion otherwise
    // assumes the in-flight global->LDS loads may alias this step's LDS reads
    // and waits for them (vmcnt(0)) before the first read, which serialises
    // the copy and the MFMAs.  The loads are waited for explicitly below.
    auto step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ nxt, bool more, int64_t knext) {
        if (more) issue(knext, nxt);
#pragma unroll
        for (int kk = 0; kk < GBK / 16; ++kk) mfma_k(cur, cur + BM * GBK, kk);
    };

    if (nk > 0) issue(kbeg, smem[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        // the other buffer was last read in the previous step, before the barrier
        step(smem[cur], smem[cur ^ 1], kt + 1 < nk, kbeg + (int64_t)(kt + 1) * GBK);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
    float* Cf = p.Cf ? p.Cf + (int64_t)blockIdx.y * p.split_stride : nullptr;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            store_acc(acc[i][j], p, Cf, m0 + wm * WTM + i * 32 + 4 * (lane >> 5), n0 + wn * WTN + j * 32 + (lane & 31));
}

}  // namespace mt
