// The pipelined bf16 GEMM kernel for large operands (M, N >= 256, K slices in
// whole steps of 32): 256x256 output tiles, 4 waves of 128x128, a four-stage
// ring of K sub-steps in LDS fed by direct global->LDS buffer loads, and a
// coalesced epilogue staged through LDS.  Design notes in gemm.hip.
#pragma once
#include "gemm_kernel.h"

namespace mt {

constexpr int PBK = 32;     // K sub-step
constexpr int PSTAGES = 4;  // LDS ring depth (3 sub-steps of loads in flight)

// Operand tiles of one sub-step, 256 rows x 32 k (16 KB):
//  K-major  ([rows][K] in memory): LDS [row][32 k], 64-byte rows, the 16-byte
//    chunk c of row r at position c ^ ((r >> 2) & 3): fragment reads (32
//    rows, one chunk) hit 16 distinct 16-byte bank groups per 16 lanes.
//  MN-major ([K][rows] in memory): LDS [k][256] as in memory, chunk c of
//    k-row k at c ^ 4 (k & 3), read with ds_read_b64_tr_b16 as in gemm_kernel.h.
struct PTile {
    static __device__ __forceinline__ int kpos(int c, int row) { return c ^ ((row >> 2) & 3); }
    static __device__ __forceinline__ bf16x8 frag_k(const uint16_t* T, int rbase, int kk, int lane) {
        const int row = rbase + (lane & 31);
        const int c = kk * 2 + (lane >> 5);
        return as_bf16x8(*(const uint4*)(T + row * PBK + 8 * kpos(c, row)));
    }
    static __device__ __forceinline__ bf16x8 frag_mn(const uint16_t* T, int rbase, int kk, int lane) {
        const int g = lane >> 4, j = lane & 15;
        const int r = j >> 2, q = j & 3;
        const int m = rbase + 16 * (g & 1) + 4 * q;  // the 4 rows this lane supplies
        const int kb = kk * 16 + 8 * (g >> 1) + r;   // its k-row (first read)
        const int c = m >> 3, sub = m & 7;
        const uint16_t* a0 = T + kb * 256 + 8 * mswz(c, kb) + sub;
        const uint16_t* a1 = T + (kb + 4) * 256 + 8 * mswz(c, kb + 4) + sub;
        const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)a0);
        const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)a1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base) {
    // raw buffer over the tile's rows; every offset used stays inside the
    // operand (tile origins are clamped so whole tiles are in bounds)
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)0x7fffffff, 0x00020000);
}

template <bool AK, bool BKM>
__global__ __launch_bounds__(256) void gemm_pipe_kernel(GemmArgs p) {
    constexpr int BM = 256, BN = 256;
    constexpr int TE = 256 * PBK;  // elements per operand tile
    __shared__ __attribute__((aligned(1024))) uint16_t smem[PSTAGES][2 * TE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    int pm, pn;
    tile_coords(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, pm, pn);
    // The last tile row / column is moved back to end at the matrix edge so
    // that every load is in bounds; its rows / columns below the unmoved
    // origin belong to the previous tile and are not stored.
    const int64_t m_lo = (int64_t)pm * BM, n_lo = (int64_t)pn * BN;
    const int64_t m0 = min(m_lo, p.M - BM), n0 = min(n_lo, p.N - BN);
    const int64_t kbeg = (int64_t)blockIdx.y * p.k_per_split;
    const int64_t kend = min(p.K, kbeg + p.k_per_split);
    const int ns = (int)((kend - kbeg) / PBK);  // >= 1 (checked by the launcher)

    // Per-lane byte offsets of the direct loads.  Wave w issues instructions
    // j = w + 4i (i < 4) of each operand tile, 1 KB each, landing at j KB.
    //  K-major: instruction j = rows 16j .. 16j+15, 4 lanes (64 bytes) per
    //    row; LDS position q holds chunk q ^ ((row >> 2) & 3), which depends
    //    on the lane only ((16j + lane/4) >> 2 = 4j + lane/16).
    //  MN-major: instruction j = k-rows 2j, 2j+1, 32 lanes per k-row;
    //    position q holds chunk q ^ 4 (k & 3), k & 3 = 2 (j & 1) + lane/32,
    //    and j & 1 = w & 1.
    auto lane_off = [&](bool kmaj, int64_t ld) -> uint32_t {
        if (kmaj) {
            const int row = lane >> 2, q = lane & 3;
            return (uint32_t)(row * ld * 2 + 16 * (q ^ ((lane >> 4) & 3)));
        }
        const int kr = lane >> 5, q = lane & 31;
        return (uint32_t)(kr * ld * 2 + 16 * (q ^ (4 * (2 * (wave & 1) + kr))));
    };
    const uint32_t a_lo = lane_off(AK, p.lda), b_lo = lane_off(BKM, p.ldb);
    const uint32_t a_js = (uint32_t)((AK ? 16 : 2) * p.lda * 2), b_js = (uint32_t)((BKM ? 16 : 2) * p.ldb * 2);

    // Loads of sub-step s into ring slot s % PSTAGES.  Past the last sub-step
    // the last one is loaded again (never read): every wave issues the same
    // number of loads per sub-step, so the wait counts below are static.
    auto issue = [&](int s) {
        const int64_t k0 = kbeg + (int64_t)min(s, ns - 1) * PBK;
        uint16_t* buf = smem[s % PSTAGES];
        const auto ra = tile_rsrc(AK ? p.A + m0 * p.lda + k0 : p.A + k0 * p.lda + m0);
        const auto rb = tile_rsrc(BKM ? p.B + n0 * p.ldb + k0 : p.B + k0 * p.ldb + n0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = wave + 4 * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(buf + j * 512), 16, a_lo + j * a_js, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(buf + TE + j * 512), 16, b_lo + j * b_js, 0, 0, 0);
        }
    };

    // acc[i][j] = the transposed 32x32 block (i, j) of this wave's 128x128:
    // the B fragment is the MFMA's first operand, so a lane holds one output
    // row (lane % 32) and runs of 4 consecutive columns.
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
    auto read_frags = [&](const uint16_t* __restrict__ S, int kk, bf16x8* a, bf16x8* b) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (AK) a[i] = PTile::frag_k(S, wm * 128 + i * 32, kk, lane);
            else a[i] = PTile::frag_mn(S, wm * 128 + i * 32, kk, lane);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (BKM) b[j] = PTile::frag_k(S + TE, wn * 128 + j * 32, kk, lane);
            else b[j] = PTile::frag_mn(S + TE, wn * 128 + j * 32, kk, lane);
        }
    };
    auto mma = [&](const bf16x8* a, const bf16x8* b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    };
    // Wait until at most 8 (PSTAGES - 2) of this wave's loads are in flight
    // (those of the next sub-step have landed) and its LDS reads are done.
    constexpr int WV = 8 * (PSTAGES - 2);
    constexpr int WAIT = (WV & 15) | ((WV >> 4) << 14) | (7 << 4);
    // One sub-step: refill the slot freed by the previous sub-step, read the
    // second half's fragments while the first half's MFMAs run, then (after
    // every wave's next slot has landed and every read of this slot is done)
    // read the next sub-step's first fragments under the second half's MFMAs.
    // The scheduling barriers keep the MFMAs of the first half ahead of the
    // wait and the workgroup barrier.  The slots are restrict-qualified so
    // that the compiler does not wait for the in-flight loads before reads.
    auto body = [&](const uint16_t* __restrict__ cur, const uint16_t* __restrict__ nxt, int s) {
        issue(s + PSTAGES - 1);
        read_frags(cur, 1, fa1, fb1);
        mma(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(WAIT);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (s + 1 < ns) read_frags(nxt, 0, fa0, fb0);
        mma(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s = 0; s < PSTAGES - 1; ++s) issue(s);
    __builtin_amdgcn_s_waitcnt(WAIT);
    __builtin_amdgcn_s_barrier();
    read_frags(smem[0], 0, fa0, fb0);
    for (int s = 0; s < ns; ++s) body(smem[s % PSTAGES], smem[(s + 1) % PSTAGES], s);
    __builtin_amdgcn_s_waitcnt(0);  // the trailing repeated loads, before LDS is reused

    float* Cf = p.Cf ? p.Cf + (int64_t)blockIdx.y * p.split_stride : nullptr;
    if (!Cf) {
        // bf16 output: add the residual (read in the accumulator layout), round,
        // stage the tile in LDS as [256][256] (16-byte chunk c of row r at
        // c ^ (r & 31)) and write whole rows, 2 x 512 bytes per store.
        __syncthreads();
        uint16_t* st = &smem[0][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + (lane & 31);
            const int64_t m = m0 + r;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);  // first column in the tile
                    float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                          v3 = acc[i][j][4 * q + 3];
                    if (p.R && m < p.M && n0 + cl < p.N) {
                        const uint2 rr = *(const uint2*)(p.R + m * p.ldc + n0 + cl);
                        v0 += bf_lo(rr.x);
                        v1 += bf_hi(rr.x);
                        v2 += bf_lo(rr.y);
                        v3 += bf_hi(rr.y);
                    }
                    const int c = cl >> 3;
                    *(uint2*)(st + r * 256 + 8 * (c ^ (r & 31)) + 4 * (lane >> 5)) =
                        make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
                }
        }
        __syncthreads();
        const int c = tid & 31;
        const int64_t n = n0 + 8 * c;
        if (n < n_lo || n >= p.N) return;
#pragma unroll 4
        for (int it = 0; it < 32; ++it) {
            const int r = 8 * it + (tid >> 5);
            const int64_t m = m0 + r;
            if (m < m_lo || m >= p.M) continue;
            *(uint4*)(p.Cb + m * p.ldc + n) = *(const uint4*)(st + r * 256 + 8 * (c ^ (r & 31)));
        }
        return;
    }
    // fp32 output (optionally accumulated; the bf16 copy, if any, is of the
    // product plus residual, not of the accumulated sum): straight from the
    // accumulators, 4 consecutive columns per store.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
        if (m < m_lo || m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * 128 + j * 32 + 8 * q + 4 * (lane >> 5);
                if (n < n_lo || n >= p.N) continue;
                const int64_t o = m * p.ldc + n;
                float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                      v3 = acc[i][j][4 * q + 3];
                if (p.R) {
                    const uint2 rr = *(const uint2*)(p.R + o);
                    v0 += bf_lo(rr.x);
                    v1 += bf_hi(rr.x);
                    v2 += bf_lo(rr.y);
                    v3 += bf_hi(rr.y);
                }
                float4* cp = (float4*)(Cf + o);
                float4 w = make_float4(v0, v1, v2, v3);
                if (p.accumulate) {
                    const float4 cv = *cp;
                    w.x += cv.x;
                    w.y += cv.y;
                    w.z += cv.z;
                    w.w += cv.w;
                }
                *cp = w;
                if (p.Cb) *(uint2*)(p.Cb + o) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
            }
    }
}

}  // namespace mt
