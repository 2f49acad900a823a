// Ping-pong bf16 GEMM kernel for large operands (M, N >= 256, K slices in
// whole steps of 32): 256x256 output tiles, 8 waves of 128x64, two waves per
// SIMD.  The two waves of a SIMD alternate between a memory phase
// (LDS->register fragment reads of the current sub-step, then direct
// global->LDS loads three sub-steps ahead) and a compute phase (16 MFMAs on
// those fragments), one phase apart, with one workgroup barrier between
// phases: while one wave of the SIMD reads and loads, the other keeps the
// matrix core busy.  The LDS tile layouts and the ring are those of
// gemm_pipe.h; the per-output K order is the same, so the results are
// bit-identical to the other kernels.
#pragma once
#include "gemm_pipe.h"

namespace mt {

// Staging of a 256 x 256 tile of 16-bit values in LDS: 16-byte chunk c of row
// r at chunk c ^ (r & 31), so that both the per-lane stores (32 rows, one
// chunk) and the row reads of the write-out are conflict free.
__device__ __forceinline__ int stage_off(int r, int col) { return r * 256 + 8 * ((col >> 3) ^ (r & 31)) + (col & 7); }

// Write the staged tile's rows m0 + r (r < 256, rows below m_lo belong to the
// previous tile) as 16-byte pieces: the thread's chunk c (0..31) goes to
// lo + m * ld + 8c for c < 16, else to hi + m * ld + 8(c - 16) (either base NULL:
// skipped).
__device__ __forceinline__ void write_halves(const uint16_t* st, uint16_t* lo, uint16_t* hi, int64_t ld, int64_t m0,
                                             int64_t m_lo, int64_t M, int tid) {
    const int c = tid & 31;
    uint16_t* base = c < 16 ? lo : hi;
    if (!base) return;
    const int cc = c & 15;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
        const int r = 16 * it + (tid >> 5);
        const int64_t m = m0 + r;
        if (m < m_lo || m >= M) continue;
        *(uint4*)(base + m * ld + 8 * cc) = *(const uint4*)(st + r * 256 + 8 * (c ^ (r & 31)));
    }
}

// The fused epilogues (GemmArgs::epi) of a 256 x 256 tile at (m0, n0); N is a
// multiple of 256, so n0 is the tile's own origin and every head (or gate/up
// pair block) lies inside the tile.
__device__ __forceinline__ void epilogue_fused(const GemmArgs& p, const f32x16 (&acc)[4][2], int64_t m0, int64_t n0,
                                               int64_t m_lo, int wm, int wn, int lane, int tid, uint16_t* st) {
    __syncthreads();  // every wave is past its last fragment read: LDS is free
    if (p.epi == 1) {
        const int hd = p.rope_hd, half = hd / 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + (lane & 31);
            const int64_t pos = (p.rope_t0 + m0 + r) % p.rope_S;
            const float* cs = p.rope_cos + pos * half;
            const float* sn = p.rope_sin + pos * half;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5);
                    const float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2],
                                v3 = acc[i][j][4 * q + 3];
                    if (n0 + cl < p.rope_cols) {
                        // (v0, v1) = features (pr, pr + hd/2) of pair pr, (v2, v3) pair pr + 1
                        const int o = (int)((n0 + cl) % hd), pr = o / 2;
                        const int la = cl - o + pr;  // local column of feature pr of this head
                        const float2 c2 = *(const float2*)(cs + pr), s2 = *(const float2*)(sn + pr);
                        const float ra0 = v0 * c2.x - v1 * s2.x, rb0 = v1 * c2.x + v0 * s2.x;
                        const float ra1 = v2 * c2.y - v3 * s2.y, rb1 = v3 * c2.y + v2 * s2.y;
                        *(uint32_t*)(st + stage_off(r, la)) = pack_h2(ra0, ra1);
                        *(uint32_t*)(st + stage_off(r, la + half)) = pack_h2(rb0, rb1);
                    } else {
                        *(uint2*)(st + stage_off(r, cl)) = make_uint2(pack_h2(v0, v1), pack_h2(v2, v3));
                    }
                }
        }
        __syncthreads();
        write_halves(st, p.Cb + n0, p.Cb + n0 + 128, p.ldc, m0, m_lo, p.M, tid);
        return;
    }
    // SwiGLU: (v0, v1, v2, v3) = gate, up of feature jf and of jf + 1, jf = (n0 + cl) / 2
    const int64_t f = p.N / 2, j0 = n0 / 2;
    if (p.Cb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5), lg = cl / 2;
                    *(uint32_t*)(st + stage_off(r, lg)) = pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 2]);
                    *(uint32_t*)(st + stage_off(r, 128 + lg)) = pack_bf2(acc[i][j][4 * q + 1], acc[i][j][4 * q + 3]);
                }
        }
        __syncthreads();
        write_halves(st, p.Cb + j0, p.Cb + f + j0, p.ldc, m0, m_lo, p.M, tid);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cl = wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5), lg = cl / 2;
                const float a0 = swiglu_f(acc[i][j][4 * q], acc[i][j][4 * q + 1]);
                const float a1 = swiglu_f(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
                *(uint32_t*)(st + stage_off(r, lg)) = pack_bf2(a0, a1);
                *(uint32_t*)(st + stage_off(r, 128 + lg)) = pack_h2(a0, a1);
            }
    }
    __syncthreads();
    write_halves(st, p.Ca ? p.Ca + j0 : nullptr, p.Ca16 ? p.Ca16 + j0 : nullptr, f, m0, m_lo, p.M, tid);
}

template <bool AK, bool BKM, bool F16 = false>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs p) {
    constexpr int BM = 256, BN = 256;
    constexpr int TE = 256 * PBK;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[PSTAGES][2 * TE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Waves w and w + 4 share a SIMD (wave i of a workgroup is placed on SIMD
    // i mod 4; correctness does not depend on it); group 0 (waves 0-3) runs
    // one phase ahead of group 1.  Wave tile: rows wm*128 .. +127, columns
    // wn*64 .. +63.
    const int grp = wave >> 2, w4 = wave & 3;
    const int wm = w4 & 1, wn = 2 * grp + (w4 >> 1);
    int pm, pn;
    tile_coords<4>(blockIdx.x, gridDim.x, p.tiles_m, p.tiles_n, pm, pn);
    const int64_t m_lo = (int64_t)pm * BM, n_lo = (int64_t)pn * BN;
    const int64_t m0 = min(m_lo, p.M - BM), n0 = min(n_lo, p.N - BN);
    const int64_t kbeg = (int64_t)blockIdx.y * p.k_per_split;
    const int64_t kend = min(p.K, kbeg + p.k_per_split);
    const int ns = (int)((kend - kbeg) / PBK);  // >= 1 (checked by the launcher)

    // Group 0 loads the A tile of each sub-step, group 1 the B tile: wave w4
    // of the group issues the 1 KB instructions j = w4 + 4i (i < 4) of that
    // operand, with the lane offsets of gemm_pipe_kernel.
    const bool load_a = grp == 0;
    const bool kmaj = load_a ? AK : BKM;
    const uint16_t* P = load_a ? p.A : p.B;
    const int64_t ld = load_a ? p.lda : p.ldb;
    const int64_t r0 = load_a ? m0 : n0;
    uint32_t lo, js;
    if (kmaj) {
        const int row = lane >> 2, q = lane & 3;
        lo = (uint32_t)(row * ld * 2 + 16 * (q ^ ((lane >> 4) & 3)));
        js = (uint32_t)(16 * ld * 2);
    } else {
        const int kr = lane >> 5, q = lane & 31;
        lo = (uint32_t)(kr * ld * 2 + 16 * (q ^ (4 * (2 * (w4 & 1) + kr))));
        js = (uint32_t)(2 * ld * 2);
    }
    const int dst_off = load_a ? 0 : TE;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Loads of sub-step s (past the last one, the last one again: every wave
    // issues four loads per sub-step, so the wait counts are static).
    auto issue = [&](uint16_t* __restrict__ buf, int s) {
        const int64_t k0 = kbeg + (int64_t)min(s, ns - 1) * PBK;
        const auto rs = tile_rsrc(kmaj ? P + r0 * ld + k0 : P + k0 * ld + r0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = w4 + 4 * i;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(buf + dst_off + j * 512), 16, lo + j * js, 0, 0,
                                                     0);
        }
    };
    bf16x8 fa[2][4], fb[2][2];
    auto read_frags = [&](const uint16_t* __restrict__ S) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (AK) fa[kk][i] = PTile::frag_k(S, wm * 128 + i * 32, kk, lane);
                else fa[kk][i] = PTile::frag_mn(S, wm * 128 + i * 32, kk, lane);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (BKM) fb[kk][j] = PTile::frag_k(S + TE, wn * 64 + j * 32, kk, lane);
                else fb[kk][j] = PTile::frag_mn(S + TE, wn * 64 + j * 32, kk, lane);
            }
        }
    };
    // Memory phase of sub-step s: read this sub-step's fragments, then
    // refill the slot that sub-step s - 1 used (both groups finished reading
    // it before the previous barrier), then wait for the reads and for this
    // wave's loads of sub-step s + 1, so that after the barrier every wave's
    // share of it is in LDS.  The slots are restrict-qualified so that the
    // compiler does not wait for the in-flight loads before the reads.
    auto mem = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ refill, int s) {
        read_frags(cur);
        issue(refill, s + PSTAGES - 1);
    };
    constexpr int WV = 4 * (PSTAGES - 2);
    constexpr int WAIT = (WV & 15) | ((WV >> 4) << 14) | (7 << 4);

#pragma unroll
    for (int s = 0; s < PSTAGES - 1; ++s) issue(smem[s], s);
    __builtin_amdgcn_s_waitcnt(WAIT);
    __builtin_amdgcn_s_barrier();
    // Stagger: group 1 starts one phase behind, so that in every phase one
    // wave of each SIMD runs its memory phase and the other its MFMAs.
    if (grp == 1) __builtin_amdgcn_s_barrier();
    for (int s = 0; s < ns; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        mem(smem[s % PSTAGES], smem[(s + PSTAGES - 1) % PSTAGES], s);
        __builtin_amdgcn_s_waitcnt(WAIT);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32x16<F16>(fb[kk][j], fa[kk][i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_s_waitcnt(0);  // the trailing repeated loads, before LDS is reused

    // acc[i][j] is the transposed 32x32 block (i, j) of the wave tile: a lane
    // holds output row (lane % 32) and runs of 4 consecutive columns.
    if constexpr (F16) {
        if (p.epi) {
            epilogue_fused(p, acc, m0, n0, m_lo, wm, wn, lane, tid, &smem[0][0]);
            return;
        }
    }
    float* Cf = p.Cf ? p.Cf + (int64_t)blockIdx.y * p.split_stride : nullptr;
    if (!Cf) {
        // bf16 output: residual, round, stage [256][256] in LDS (16-byte chunk
        // c of row r at c ^ (r & 31)), write whole 512-byte rows.
        __syncthreads();
        uint16_t* st = &smem[0][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * 128 + i * 32 + (lane & 31);
            const int64_t m = m0 + r;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int cl = wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5);
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
        for (int it = 0; it < 16; ++it) {
            const int r = 16 * it + (tid >> 5);
            const int64_t m = m0 + r;
            if (m < m_lo || m >= p.M) continue;
            *(uint4*)(p.Cb + m * p.ldc + n) = *(const uint4*)(st + r * 256 + 8 * (c ^ (r & 31)));
        }
        return;
    }
    // fp32 output (optionally accumulated; the bf16 copy, if any, is of the
    // product plus residual): straight from the accumulators.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
        if (m < m_lo || m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n0 + wn * 64 + j * 32 + 8 * q + 4 * (lane >> 5);
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
