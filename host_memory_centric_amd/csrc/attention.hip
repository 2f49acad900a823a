// Causal attention on gfx950 matrix cores: tiled online-softmax forward and a
// two-kernel backward (dK/dV over key tiles, dQ over query tiles), so no
// gradient is ever accumulated with atomics.
//
// Scores are computed transposed where that keeps each query's softmax state
// inside one lane: with S^T = K Q^T on v_mfma_f32_32x32x16_bf16 a lane owns
// one query column and 16 key rows of each 32x32 tile, so the row max / row
// sum need one cross-half shuffle, the running rescale of O^T = V^T P^T is a
// per-lane multiply, and the probabilities are already laid out as the B
// operand of the next MFMA.  The 8 contraction elements a lane feeds are the
// same (lane half, element) -> key mapping in both operands, which is all the
// MFMA needs.  The dK/dV kernel uses the untransposed S = Q K^T so that each
// lane owns one key column.
//
// Layout: qkv is the fused projection output [B*S, 3*H] (q | k | v, head h at
// columns h*hd .. h*hd + hd - 1 of each third), o is [B*S, H], lse is
// [B, heads, S] natural-log row logsumexp of the scaled scores.
#include "common.h"
#include "device.h"
#include "kernels.h"

namespace mt {

constexpr int ATT_WAVES = 4;
constexpr int ATT_THREADS = ATT_WAVES * 64;
constexpr int ATT_BQ = ATT_WAVES * 32;  // queries per workgroup (fwd, dQ)
constexpr int ATT_BKV = 64;             // keys per step (fwd, dQ)
constexpr int ATT_BK = ATT_WAVES * 32;  // keys per workgroup (dK/dV)
constexpr int ATT_QT = 64;              // queries per step (dK/dV)
constexpr int RPAD = 8;                 // padding of [rows][hd] tiles
constexpr int TPAD = 4;                 // padding of transposed [hd][rows] tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// rows [r0, r0 + ROWS) of a [S][hd] matrix (row stride ld) -> Ts[r][d]
template <int ROWS, int HD>
__device__ __forceinline__ void load_rows(const uint16_t* G, int64_t ld, int r0, int S, uint16_t (*Ts)[HD + RPAD]) {
    for (int u = threadIdx.x; u < ROWS * HD / 8; u += ATT_THREADS) {
        const int row = u / (HD / 8), c = (u % (HD / 8)) * 8;
        const int r = r0 + row;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < S) v = *(const uint4*)(G + (int64_t)r * ld + c);
        *(uint4*)&Ts[row][c] = v;
    }
}

// rows [r0, r0 + ROWS) of a [S][hd] matrix -> transposed Tt[d][r]
template <int ROWS, int HD>
__device__ __forceinline__ void load_rows_t(const uint16_t* G, int64_t ld, int r0, int S, uint16_t (*Tt)[ROWS + TPAD]) {
    for (int u = threadIdx.x; u < (ROWS / 4) * (HD / 8); u += ATT_THREADS) {
        const int dc = (u % (HD / 8)) * 8, rq = u / (HD / 8);
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + rq * 4 + i;
            v[i] = make_uint4(0, 0, 0, 0);
            if (r < S) v[i] = *(const uint4*)(G + (int64_t)r * ld + dc);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int sh = (e & 1) * 16;
            const int q = e >> 1;
            const uint32_t a0 = ((const uint32_t*)&v[0])[q] >> sh & 0xffffu, a1 = ((const uint32_t*)&v[1])[q] >> sh & 0xffffu,
                           a2 = ((const uint32_t*)&v[2])[q] >> sh & 0xffffu, a3 = ((const uint32_t*)&v[3])[q] >> sh & 0xffffu;
            *(uint2*)&Tt[dc + e][rq * 4] = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        }
    }
}

// A-operand fragment of a transposed tile: row i (d), the 8 contraction
// elements (keys or queries) c0 + {4h..4h+3} and c0 + 8 + {4h..4h+3}.
template <int W>
__device__ __forceinline__ bf16x8 frag_t(const uint16_t (*Tt)[W], int row, int c0, int half) {
    const uint2 lo = *(const uint2*)&Tt[row][c0 + 4 * half];
    const uint2 hi = *(const uint2*)&Tt[row][c0 + 8 + 4 * half];
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// B-operand fragment from 8 accumulator values (elements r0 .. r0+7 of a tile)
__device__ __forceinline__ bf16x8 frag_acc(const f32x16& a, int r0) {
    return as_bf16x8(make_uint4(pack_bf2(a[r0 + 0], a[r0 + 1]), pack_bf2(a[r0 + 2], a[r0 + 3]),
                                pack_bf2(a[r0 + 4], a[r0 + 5]), pack_bf2(a[r0 + 6], a[r0 + 7])));
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(ATT_THREADS) void attn_fwd_kernel(const uint16_t* __restrict__ qkv, uint16_t* __restrict__ o,
                                                               float* __restrict__ lse, int S, int heads, float sl2) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[HD][ATT_BKV + TPAD];
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    const int qb = nqb - 1 - (int)blockIdx.x;  // most work first
    const int b = blockIdx.y / heads, head = blockIdx.y % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const int q0 = qb * ATT_BQ + wave * 32;
    const int qi = q0 + (lane & 31);

    uint4 qf[HD / 16];
#pragma unroll
    for (int ds = 0; ds < HD / 16; ++ds) {
        qf[ds] = make_uint4(0, 0, 0, 0);
        if (qi < S) qf[ds] = *(const uint4*)(Qg + (int64_t)qi * ld + ds * 16 + 8 * half);
    }
    f32x16 oacc[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_BKV - 1) / ATT_BKV;
    for (int kb = 0; kb < nkv; ++kb) {
        const int k0 = kb * ATT_BKV;
        __syncthreads();
        load_rows<ATT_BKV, HD>(Kg, ld, k0, S, Ks);
        load_rows_t<ATT_BKV, HD>(Vg, ld, k0, S, Vt);
        __syncthreads();
        if (k0 > q0 + 31) continue;  // every key of this tile is in this wave's future

        f32x16 st[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) st[kt][r] = 0.f;
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds) {
                const bf16x8 a = as_bf16x8(*(const uint4*)&Ks[kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qf[ds]), st[kt], 0, 0, 0);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kt * 32 + acc_row(r, half);
                float v = st[kt][r] * sl2;
                if (key > qi || key >= S) v = -INFINITY;
                st[kt][r] = v;
                mx = fmaxf(mx, v);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = exp2f(st[kt][r] - m_new);
                st[kt][r] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pb = frag_acc(st[kt], ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt) {
                    const bf16x8 va = frag_t<ATT_BKV + TPAD>(Vt, dt * 32 + (lane & 31), kt * 32 + ks * 16, half);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
                }
            }
    }
    if (qi < S) {
        const float inv_l = 1.0f / l_run;
        uint16_t* orow = o + ((int64_t)b * S + qi) * H + (int64_t)head * HD;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                *(uint2*)(orow + d) = make_uint2(pack_bf2(oacc[dt][4 * g] * inv_l, oacc[dt][4 * g + 1] * inv_l),
                                                 pack_bf2(oacc[dt][4 * g + 2] * inv_l, oacc[dt][4 * g + 3] * inv_l));
            }
        if (half == 0) lse[((int64_t)b * heads + head) * S + qi] = (m_run + log2f(l_run)) * LN2;
    }
}

// ---------------------------------------------------------------------------
// backward: D = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int HD>
__global__ void attn_bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                    float* __restrict__ dvec, int64_t T, int S, int heads) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= T * heads) return;
    const int64_t t = idx / heads;
    const int head = (int)(idx % heads);
    const int64_t H = (int64_t)heads * HD;
    const uint16_t* a = o + t * H + (int64_t)head * HD;
    const uint16_t* c = dout + t * H + (int64_t)head * HD;
    float s = 0.f;
#pragma unroll 4
    for (int d = 0; d < HD; d += 8) {
        const uint4 x = *(const uint4*)(a + d), y = *(const uint4*)(c + d);
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) s += bf_lo(xw[q]) * bf_lo(yw[q]) + bf_hi(xw[q]) * bf_hi(yw[q]);
    }
    const int64_t b = t / S, sidx = t % S;
    dvec[(b * heads + head) * S + sidx] = s;
}

// ---------------------------------------------------------------------------
// backward: dQ, one workgroup per 128 queries, loop over key tiles
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(ATT_THREADS) void attn_bwd_dq_kernel(const uint16_t* __restrict__ qkv,
                                                                  const float* __restrict__ lse,
                                                                  const uint16_t* __restrict__ dout,
                                                                  const float* __restrict__ dvec,
                                                                  uint16_t* __restrict__ dqkv, int S, int heads,
                                                                  float sl2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Kt[HD][ATT_BKV + TPAD];
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    const int qb = nqb - 1 - (int)blockIdx.x;
    const int b = blockIdx.y / heads, head = blockIdx.y % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const uint16_t* dOg = dout + (int64_t)b * S * H + (int64_t)head * HD;
    const int q0 = qb * ATT_BQ + wave * 32;
    const int qi = q0 + (lane & 31);

    uint4 qf[HD / 16], df[HD / 16];
#pragma unroll
    for (int ds = 0; ds < HD / 16; ++ds) {
        qf[ds] = make_uint4(0, 0, 0, 0);
        df[ds] = make_uint4(0, 0, 0, 0);
        if (qi < S) {
            qf[ds] = *(const uint4*)(Qg + (int64_t)qi * ld + ds * 16 + 8 * half);
            df[ds] = *(const uint4*)(dOg + (int64_t)qi * H + ds * 16 + 8 * half);
        }
    }
    const int64_t rowbase = ((int64_t)b * heads + head) * S;
    const float lse2 = qi < S ? lse[rowbase + qi] * LOG2E : 0.f;
    const float Dq = qi < S ? dvec[rowbase + qi] : 0.f;
    f32x16 dq[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_BKV - 1) / ATT_BKV;
    for (int kb = 0; kb < nkv; ++kb) {
        const int k0 = kb * ATT_BKV;
        __syncthreads();
        load_rows<ATT_BKV, HD>(Kg, ld, k0, S, Ks);
        load_rows<ATT_BKV, HD>(Vg, ld, k0, S, Vs);
        load_rows_t<ATT_BKV, HD>(Kg, ld, k0, S, Kt);
        __syncthreads();
        if (k0 > q0 + 31) continue;
        f32x16 st[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                st[kt][r] = 0.f;
                dp[kt][r] = 0.f;
            }
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds) {
                const bf16x8 ka = as_bf16x8(*(const uint4*)&Ks[kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, as_bf16x8(qf[ds]), st[kt], 0, 0, 0);
                const bf16x8 va = as_bf16x8(*(const uint4*)&Vs[kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                dp[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(df[ds]), dp[kt], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + kt * 32 + acc_row(r, half);
                const bool ok = key <= qi && key < S && qi < S;
                const float p = ok ? exp2f(st[kt][r] * sl2 - lse2) : 0.f;
                st[kt][r] = p * (dp[kt][r] - Dq);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 sb = frag_acc(st[kt], ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt) {
                    const bf16x8 ka = frag_t<ATT_BKV + TPAD>(Kt, dt * 32 + (lane & 31), kt * 32 + ks * 16, half);
                    dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sb, dq[dt], 0, 0, 0);
                }
            }
    }
    if (qi < S) {
        uint16_t* row = dqkv + ((int64_t)b * S + qi) * ld + (int64_t)head * HD;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                *(uint2*)(row + d) = make_uint2(pack_bf2(dq[dt][4 * g] * scale, dq[dt][4 * g + 1] * scale),
                                                pack_bf2(dq[dt][4 * g + 2] * scale, dq[dt][4 * g + 3] * scale));
            }
    }
}

// ---------------------------------------------------------------------------
// backward: dK and dV, one workgroup per 128 keys, loop over query tiles
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(ATT_THREADS) void attn_bwd_dkdv_kernel(const uint16_t* __restrict__ qkv,
                                                                    const float* __restrict__ lse,
                                                                    const uint16_t* __restrict__ dout,
                                                                    const float* __restrict__ dvec,
                                                                    uint16_t* __restrict__ dqkv, int S, int heads,
                                                                    float sl2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t Qs[ATT_QT][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t dOs[ATT_QT][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Qt[HD][ATT_QT + TPAD];
    __shared__ __attribute__((aligned(16))) uint16_t dOt[HD][ATT_QT + TPAD];
    __shared__ float lse_s[ATT_QT], d_s[ATT_QT];
    const int kbk = (int)blockIdx.x;  // key block; low blocks (most work) first
    const int b = blockIdx.y / heads, head = blockIdx.y % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const uint16_t* dOg = dout + (int64_t)b * S * H + (int64_t)head * HD;
    const int64_t rowbase = ((int64_t)b * heads + head) * S;
    const int kw0 = kbk * ATT_BK;             // first key of the workgroup
    const int k0 = kw0 + wave * 32;           // first key of this wave
    const int kj = k0 + (lane & 31);          // key owned by this lane

    uint4 kf[HD / 16], vf[HD / 16];
#pragma unroll
    for (int ds = 0; ds < HD / 16; ++ds) {
        kf[ds] = make_uint4(0, 0, 0, 0);
        vf[ds] = make_uint4(0, 0, 0, 0);
        if (kj < S) {
            kf[ds] = *(const uint4*)(Kg + (int64_t)kj * ld + ds * 16 + 8 * half);
            vf[ds] = *(const uint4*)(Vg + (int64_t)kj * ld + ds * 16 + 8 * half);
        }
    }
    f32x16 dk[HD / 32], dv[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dk[dt][r] = 0.f;
            dv[dt][r] = 0.f;
        }

    const int qstart = (kw0 / ATT_QT) * ATT_QT;
    for (int q0 = qstart; q0 < S; q0 += ATT_QT) {
        __syncthreads();
        load_rows<ATT_QT, HD>(Qg, ld, q0, S, Qs);
        load_rows<ATT_QT, HD>(dOg, H, q0, S, dOs);
        load_rows_t<ATT_QT, HD>(Qg, ld, q0, S, Qt);
        load_rows_t<ATT_QT, HD>(dOg, H, q0, S, dOt);
        if (threadIdx.x < ATT_QT) {
            const int q = q0 + threadIdx.x;
            lse_s[threadIdx.x] = q < S ? lse[rowbase + q] * LOG2E : 0.f;
            d_s[threadIdx.x] = q < S ? dvec[rowbase + q] : 0.f;
        }
        __syncthreads();
        if (q0 + ATT_QT - 1 < k0) continue;  // every query of this tile precedes this wave's keys
#pragma unroll
        for (int qt = 0; qt < ATT_QT / 32; ++qt) {
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds) {
                const bf16x8 qa = as_bf16x8(*(const uint4*)&Qs[qt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, as_bf16x8(kf[ds]), s, 0, 0, 0);
                const bf16x8 da = as_bf16x8(*(const uint4*)&dOs[qt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, as_bf16x8(vf[ds]), dp, 0, 0, 0);
            }
            f32x16 p;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = qt * 32 + acc_row(r, half);
                const int q = q0 + ql;
                const bool ok = kj <= q && q < S && kj < S;
                const float pv = ok ? exp2f(s[r] * sl2 - lse_s[ql]) : 0.f;
                p[r] = pv;
                s[r] = pv * (dp[r] - d_s[ql]);  // dS
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pb = frag_acc(p, ks * 8);
                const bf16x8 sb = frag_acc(s, ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt) {
                    const bf16x8 oa = frag_t<ATT_QT + TPAD>(dOt, dt * 32 + (lane & 31), qt * 32 + ks * 16, half);
                    dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb, dv[dt], 0, 0, 0);
                    const bf16x8 qa = frag_t<ATT_QT + TPAD>(Qt, dt * 32 + (lane & 31), qt * 32 + ks * 16, half);
                    dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb, dk[dt], 0, 0, 0);
                }
            }
        }
    }
    if (kj < S) {
        uint16_t* krow = dqkv + ((int64_t)b * S + kj) * ld + H + (int64_t)head * HD;
        uint16_t* vrow = krow + H;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                *(uint2*)(krow + d) = make_uint2(pack_bf2(dk[dt][4 * g] * scale, dk[dt][4 * g + 1] * scale),
                                                 pack_bf2(dk[dt][4 * g + 2] * scale, dk[dt][4 * g + 3] * scale));
                *(uint2*)(vrow + d) = make_uint2(pack_bf2(dv[dt][4 * g], dv[dt][4 * g + 1]),
                                                 pack_bf2(dv[dt][4 * g + 2], dv[dt][4 * g + 3]));
            }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static void check_attn(int B, int S, int heads, int hd) {
    if (hd != 64 && hd != 128) MT_FAIL(MT_E_SHAPE, "attention: head_dim %d not in {64, 128}", hd);
    if (B < 1 || S < 1 || heads < 1) MT_FAIL(MT_E_SHAPE, "attention: empty shape");
    if ((int64_t)B * heads > 65535) MT_FAIL(MT_E_SHAPE, "attention: batch*heads too large");
}

void attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int B, int S, int heads, int hd, hipStream_t s) {
    check_attn(B, S, heads, hd);
    const float sl2 = LOG2E / sqrtf((float)hd);
    const dim3 grid((S + ATT_BQ - 1) / ATT_BQ, B * heads);
    // causal: S(S+1)/2 score entries, each 2*hd flops for QK^T and 2*hd for PV
    ProfScope prof(PROF_ATTN_FWD, 4.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    if (hd == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(ATT_THREADS), 0, s, qkv, o, lse, S, heads, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(ATT_THREADS), 0, s, qkv, o, lse, S, heads, sl2);
    launch_check("attention_fwd", s);
}

void attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout, uint16_t* dqkv,
                   float* dvec, int B, int S, int heads, int hd, hipStream_t s) {
    check_attn(B, S, heads, hd);
    const float scale = 1.0f / sqrtf((float)hd);
    const float sl2 = LOG2E * scale;
    const int64_t T = (int64_t)B * S;
    const int64_t n = T * heads;
    const dim3 gq((S + ATT_BQ - 1) / ATT_BQ, B * heads), gk((S + ATT_BK - 1) / ATT_BK, B * heads);
    // causal entries x (QK^T recompute, dP, dV, dK, dQ) at 2*hd flops each
    ProfScope prof(PROF_ATTN_BWD, 10.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    if (hd == 128) {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<128>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o, dout, dvec,
                           T, S, heads);
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<64>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o, dout, dvec, T,
                           S, heads);
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
    }
    launch_check("attention_bwd", s);
}

}  // namespace mt
