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
// Operands read along their sequence index (V^T for P V, K^T for dQ, Q^T and
// dO^T for dK, dV) are first written to global memory transposed, [B, heads,
// hd, S], by a tiled transpose kernel, so every tile reaches LDS as plain
// coalesced row copies.  In LDS the transposed tiles ([hd][64 rows], 128 B per
// row, no padding) store each 16-row group in the order 0-3, 8-11, 4-7, 12-15
// (the rows one lane half contracts over are then one 16-byte chunk) and XOR
// the chunk index with (d >> 1) & 7, which makes both the 16-byte row writes
// and the fragment reads bank-conflict free.  Tiles are double buffered with
// register prefetch: one barrier per tile.
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
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// transposed copies in global memory: [B*S, ld] (head at column h*hd)
// -> [B, heads, hd, S]
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void transpose_heads_kernel(const uint16_t* __restrict__ src, int64_t ld, int S,
                                                              int heads, int hd, uint16_t* __restrict__ dst) {
    __shared__ uint16_t tile[64][64 + 2];
    const int s0 = blockIdx.x * 64, d0 = blockIdx.y * 64;
    const int bh = blockIdx.z;
    const int b = bh / heads, head = bh % heads;
    const uint16_t* in = src + (int64_t)b * S * ld + (int64_t)head * hd + d0;
    // read 64 rows (positions) x 64 columns (features): 8 lanes per row
    for (int u = threadIdx.x; u < 64 * 8; u += 256) {
        const int r = u / 8, c = (u % 8) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (s0 + r < S) v = *(const uint4*)(in + (int64_t)(s0 + r) * ld + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            tile[c + 2 * q][r] = (uint16_t)(w[q] & 0xffffu);
            tile[c + 2 * q + 1][r] = (uint16_t)(w[q] >> 16);
        }
    }
    __syncthreads();
    uint16_t* out = dst + ((int64_t)bh * hd + d0) * S + s0;
    for (int u = threadIdx.x; u < 64 * 32; u += 256) {
        const int d = u / 32, c = (u % 32) * 2;
        if (s0 + c + 1 < S && (S & 1) == 0) {
            *(uint32_t*)(out + (int64_t)d * S + c) = (uint32_t)tile[d][c] | ((uint32_t)tile[d][c + 1] << 16);
        } else {
            if (s0 + c < S) out[(int64_t)d * S + c] = tile[d][c];
            if (s0 + c + 1 < S) out[(int64_t)d * S + c + 1] = tile[d][c + 1];
        }
    }
}

static void transpose_heads(const uint16_t* src, int64_t ld, int B, int S, int heads, int hd, uint16_t* dst,
                            hipStream_t s) {
    const dim3 grid((S + 63) / 64, hd / 64, B * heads);
    hipLaunchKernelGGL(transpose_heads_kernel, grid, dim3(256), 0, s, src, ld, S, heads, hd, dst);
}

// ---------------------------------------------------------------------------
// LDS tiles
// ---------------------------------------------------------------------------
// [ROWS][HD + RPAD] tile of rows r0.. of a [S][ld] matrix; each thread owns
// PER 16-byte chunks (register prefetch, then store).
template <int ROWS, int HD>
struct RowTile {
    static constexpr int CH = ROWS * HD / 8;
    static constexpr int PER = CH / ATT_THREADS;
    static_assert(CH % ATT_THREADS == 0, "tile/threads");
    uint4 v[PER];
    __device__ __forceinline__ void load(const uint16_t* G, int64_t ld, int r0, int S) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * ATT_THREADS;
            const int row = u / (HD / 8), c = (u % (HD / 8)) * 8;
            v[i] = make_uint4(0, 0, 0, 0);
            if (r0 + row < S) v[i] = *(const uint4*)(G + (int64_t)(r0 + row) * ld + c);
        }
    }
    __device__ __forceinline__ void store(uint16_t (*T)[HD + RPAD]) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * ATT_THREADS;
            const int row = u / (HD / 8), c = (u % (HD / 8)) * 8;
            *(uint4*)&T[row][c] = v[i];
        }
    }
};

// Physical 16-byte chunk of logical chunk c in row d of a transposed tile.
__device__ __forceinline__ int swz(int c, int d) { return c ^ ((d >> 1) & 7); }

// [HD][64] transposed tile from a [hd][S] global matrix (rows r0 .. r0+63 of
// the sequence index), stored permuted and swizzled (see the file comment).
// Work unit: one feature row d and one 16-row group g (32 bytes).
template <int HD>
struct TTile {
    static constexpr int UNITS = HD * 4;
    static constexpr int PER = UNITS / ATT_THREADS;
    static_assert(UNITS % ATT_THREADS == 0, "tile/threads");
    uint4 a[PER], b[PER];
    __device__ __forceinline__ void load(const uint16_t* G, int64_t S, int r0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * ATT_THREADS;
            const int d = u / 4, g = u % 4;
            const int s = r0 + 16 * g;
            const uint16_t* p = G + (int64_t)d * S + s;
            a[i] = make_uint4(0, 0, 0, 0);
            b[i] = make_uint4(0, 0, 0, 0);
            if (s + 16 <= S && (S & 7) == 0) {
                a[i] = *(const uint4*)p;
                b[i] = *(const uint4*)(p + 8);
            } else if (s < S) {
                uint32_t w[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const uint32_t lo = s + 2 * q < S ? p[2 * q] : 0u;
                    const uint32_t hi = s + 2 * q + 1 < S ? p[2 * q + 1] : 0u;
                    w[q] = lo | (hi << 16);
                }
                a[i] = make_uint4(w[0], w[1], w[2], w[3]);
                b[i] = make_uint4(w[4], w[5], w[6], w[7]);
            }
        }
    }
    __device__ __forceinline__ void store(uint16_t (*T)[64]) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int u = threadIdx.x + i * ATT_THREADS;
            const int d = u / 4, g = u % 4;
            // rows 0-3 and 8-11 of the group -> chunk 2g, rows 4-7 and 12-15 -> chunk 2g+1
            *(uint4*)&T[d][8 * swz(2 * g, d)] = make_uint4(a[i].x, a[i].y, b[i].x, b[i].y);
            *(uint4*)&T[d][8 * swz(2 * g + 1, d)] = make_uint4(a[i].z, a[i].w, b[i].z, b[i].w);
        }
    }
};

// A-operand fragment from a transposed tile: feature row `row`, the 8
// contraction rows c0 + {4h..4h+3, 8+4h..8+4h+3} (c0 a multiple of 16).
__device__ __forceinline__ bf16x8 frag_t(const uint16_t (*T)[64], int row, int c0, int half) {
    return as_bf16x8(*(const uint4*)&T[row][8 * swz(c0 / 8 + half, row)]);
}

// B-operand fragment from 8 accumulator values (elements r0 .. r0+7 of a tile)
__device__ __forceinline__ bf16x8 frag_acc(const f32x16& a, int r0) {
    return as_bf16x8(make_uint4(pack_bf2(a[r0 + 0], a[r0 + 1]), pack_bf2(a[r0 + 2], a[r0 + 3]),
                                pack_bf2(a[r0 + 4], a[r0 + 5]), pack_bf2(a[r0 + 6], a[r0 + 7])));
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(ATT_THREADS) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                               const uint16_t* __restrict__ vt,
                                                               uint16_t* __restrict__ o, float* __restrict__ lse, int S,
                                                               int heads, float sl2) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[2][HD][64];
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    const int qb = nqb - 1 - (int)blockIdx.x;  // most work first
    const int bh = blockIdx.y;
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vtg = vt + (int64_t)bh * HD * S;
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
    for (int dt = 0; dt < HD / 32; ++dt) zero(oacc[dt]);
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_BKV - 1) / ATT_BKV;
    RowTile<ATT_BKV, HD> kt_;
    TTile<HD> vt_;
    kt_.load(Kg, ld, 0, S);
    vt_.load(Vtg, S, 0);
    kt_.store(Ks[0]);
    vt_.store(Vt[0]);
    __syncthreads();
    for (int kb = 0; kb < nkv; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * ATT_BKV;
        if (kb + 1 < nkv) {
            kt_.load(Kg, ld, k0 + ATT_BKV, S);
            vt_.load(Vtg, S, k0 + ATT_BKV);
        }
        if (k0 <= q0 + 31) {  // else every key of this tile is in this wave's future
            f32x16 st[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                zero(st[kt]);
#pragma unroll
                for (int ds = 0; ds < HD / 16; ++ds) {
                    const bf16x8 a = as_bf16x8(*(const uint4*)&Ks[cur][kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                    st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(qf[ds]), st[kt], 0, 0, 0);
                }
            }
            // masking only where the tile crosses this wave's diagonal or the end
            if (k0 + ATT_BKV - 1 > q0 || k0 + ATT_BKV > S) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kt * 32 + acc_row(r, half);
                        if (key > qi || key >= S) st[kt][r] = -INFINITY;
                    }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kt][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx * sl2);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float ps = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, -m_new));
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
                        const bf16x8 va = frag_t(Vt[cur], dt * 32 + (lane & 31), kt * 32 + ks * 16, half);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[dt], 0, 0, 0);
                    }
                }
        }
        if (kb + 1 < nkv) {
            kt_.store(Ks[cur ^ 1]);
            vt_.store(Vt[cur ^ 1]);
        }
        __syncthreads();
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
        if (half == 0) lse[(int64_t)bh * S + qi] = (m_run + log2f(l_run)) * LN2;
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
                                                                  const uint16_t* __restrict__ ktg,
                                                                  const float* __restrict__ lse,
                                                                  const uint16_t* __restrict__ dout,
                                                                  const float* __restrict__ dvec,
                                                                  uint16_t* __restrict__ dqkv, int S, int heads,
                                                                  float sl2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][ATT_BKV][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Kt[2][HD][64];
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    const int qb = nqb - 1 - (int)blockIdx.x;
    const int bh = blockIdx.y;
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const uint16_t* Ktg = ktg + (int64_t)bh * HD * S;
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
    const int64_t rowbase = (int64_t)bh * S;
    const float lse2 = qi < S ? lse[rowbase + qi] * LOG2E : 0.f;
    const float Dq = qi < S ? dvec[rowbase + qi] : 0.f;
    f32x16 dq[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) zero(dq[dt]);

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_BKV - 1) / ATT_BKV;
    RowTile<ATT_BKV, HD> k_, v_;
    TTile<HD> kt_;
    k_.load(Kg, ld, 0, S);
    v_.load(Vg, ld, 0, S);
    kt_.load(Ktg, S, 0);
    k_.store(Ks[0]);
    v_.store(Vs[0]);
    kt_.store(Kt[0]);
    __syncthreads();
    for (int kb = 0; kb < nkv; ++kb) {
        const int cur = kb & 1;
        const int k0 = kb * ATT_BKV;
        if (kb + 1 < nkv) {
            k_.load(Kg, ld, k0 + ATT_BKV, S);
            v_.load(Vg, ld, k0 + ATT_BKV, S);
            kt_.load(Ktg, S, k0 + ATT_BKV);
        }
        if (k0 <= q0 + 31) {
            f32x16 st[2], dp[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                zero(st[kt]);
                zero(dp[kt]);
#pragma unroll
                for (int ds = 0; ds < HD / 16; ++ds) {
                    const bf16x8 ka = as_bf16x8(*(const uint4*)&Ks[cur][kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                    st[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, as_bf16x8(qf[ds]), st[kt], 0, 0, 0);
                    const bf16x8 va = as_bf16x8(*(const uint4*)&Vs[cur][kt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                    dp[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, as_bf16x8(df[ds]), dp[kt], 0, 0, 0);
                }
                if (k0 + ATT_BKV - 1 > q0 || k0 + ATT_BKV > S || q0 + 32 > S) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kt * 32 + acc_row(r, half);
                        if (key > qi || key >= S || qi >= S) st[kt][r] = -INFINITY;
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, -lse2));
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
                        const bf16x8 ka = frag_t(Kt[cur], dt * 32 + (lane & 31), kt * 32 + ks * 16, half);
                        dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, sb, dq[dt], 0, 0, 0);
                    }
                }
        }
        if (kb + 1 < nkv) {
            k_.store(Ks[cur ^ 1]);
            v_.store(Vs[cur ^ 1]);
            kt_.store(Kt[cur ^ 1]);
        }
        __syncthreads();
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
__global__ __launch_bounds__(ATT_THREADS) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ qkv, const uint16_t* __restrict__ qtg, const uint16_t* __restrict__ dotg,
    const float* __restrict__ lse, const uint16_t* __restrict__ dout, const float* __restrict__ dvec,
    uint16_t* __restrict__ dqkv, int S, int heads, float sl2, float scale) {
    __shared__ __attribute__((aligned(16))) uint16_t Qs[2][ATT_QT][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t dOs[2][ATT_QT][HD + RPAD];
    __shared__ __attribute__((aligned(16))) uint16_t Qt[2][HD][64];
    __shared__ __attribute__((aligned(16))) uint16_t dOt[2][HD][64];
    __shared__ float lse_s[2][ATT_QT], d_s[2][ATT_QT];
    const int kbk = (int)blockIdx.x;  // key block; low blocks (most work) first
    const int bh = blockIdx.y;
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const uint16_t* Qtg = qtg + (int64_t)bh * HD * S;
    const uint16_t* dOtg = dotg + (int64_t)bh * HD * S;
    const uint16_t* dOg = dout + (int64_t)b * S * H + (int64_t)head * HD;
    const int64_t rowbase = (int64_t)bh * S;
    const int kw0 = kbk * ATT_BK;     // first key of the workgroup
    const int k0 = kw0 + wave * 32;   // first key of this wave
    const int kj = k0 + (lane & 31);  // key owned by this lane

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
    for (int dt = 0; dt < HD / 32; ++dt) {
        zero(dk[dt]);
        zero(dv[dt]);
    }

    const int qstart = (kw0 / ATT_QT) * ATT_QT;
    const int nqt = (S - qstart + ATT_QT - 1) / ATT_QT;
    RowTile<ATT_QT, HD> q_, o_;
    TTile<HD> qt_, ot_;
    float ls = 0.f, dd = 0.f;
    auto load_tile = [&](int q0) {
        q_.load(Qg, ld, q0, S);
        o_.load(dOg, H, q0, S);
        qt_.load(Qtg, S, q0);
        ot_.load(dOtg, S, q0);
        if (threadIdx.x < ATT_QT) {
            const int q = q0 + threadIdx.x;
            ls = q < S ? lse[rowbase + q] * LOG2E : 0.f;
            dd = q < S ? dvec[rowbase + q] : 0.f;
        }
    };
    auto store_tile = [&](int buf) {
        q_.store(Qs[buf]);
        o_.store(dOs[buf]);
        qt_.store(Qt[buf]);
        ot_.store(dOt[buf]);
        if (threadIdx.x < ATT_QT) {
            lse_s[buf][threadIdx.x] = ls;
            d_s[buf][threadIdx.x] = dd;
        }
    };
    load_tile(qstart);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < nqt; ++it) {
        const int cur = it & 1;
        const int q0 = qstart + it * ATT_QT;
        if (it + 1 < nqt) load_tile(q0 + ATT_QT);
        if (q0 + ATT_QT - 1 >= k0) {  // else every query of this tile precedes this wave's keys
#pragma unroll
            for (int qt = 0; qt < ATT_QT / 32; ++qt) {
                f32x16 s, dp;
                zero(s);
                zero(dp);
#pragma unroll
                for (int ds = 0; ds < HD / 16; ++ds) {
                    const bf16x8 qa = as_bf16x8(*(const uint4*)&Qs[cur][qt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, as_bf16x8(kf[ds]), s, 0, 0, 0);
                    const bf16x8 da = as_bf16x8(*(const uint4*)&dOs[cur][qt * 32 + (lane & 31)][ds * 16 + 8 * half]);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, as_bf16x8(vf[ds]), dp, 0, 0, 0);
                }
                // mask only where this 32-query sub-tile reaches below this wave's keys or past the end
                const bool edge = q0 + qt * 32 < k0 + 31 || q0 + qt * 32 + 32 > S || k0 + 32 > S;
                f32x16 p;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ql = qt * 32 + acc_row(r, half);
                    float sv = s[r];
                    if (edge) {
                        const int q = q0 + ql;
                        if (kj > q || q >= S || kj >= S) sv = -INFINITY;
                    }
                    const float pv = __builtin_amdgcn_exp2f(fmaf(sv, sl2, -lse_s[cur][ql]));
                    p[r] = pv;
                    s[r] = pv * (dp[r] - d_s[cur][ql]);  // dS
                }
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8 pb = frag_acc(p, ks * 8);
                    const bf16x8 sb = frag_acc(s, ks * 8);
#pragma unroll
                    for (int dt = 0; dt < HD / 32; ++dt) {
                        const bf16x8 oa = frag_t(dOt[cur], dt * 32 + (lane & 31), qt * 32 + ks * 16, half);
                        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb, dv[dt], 0, 0, 0);
                        const bf16x8 qa = frag_t(Qt[cur], dt * 32 + (lane & 31), qt * 32 + ks * 16, half);
                        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb, dk[dt], 0, 0, 0);
                    }
                }
            }
        }
        if (it + 1 < nqt) store_tile(cur ^ 1);
        __syncthreads();
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

size_t attention_fwd_ws_bytes(int B, int S, int heads, int hd) {
    return round_up((size_t)B * S * heads * hd * 2, 256);
}

size_t attention_bwd_ws_bytes(int B, int S, int heads, int hd) {
    return 3 * round_up((size_t)B * S * heads * hd * 2, 256) + round_up((size_t)B * heads * S * 4, 256);
}

void attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int B, int S, int heads, int hd, void* ws,
                   size_t ws_bytes, hipStream_t s) {
    check_attn(B, S, heads, hd);
    if (!ws || ws_bytes < attention_fwd_ws_bytes(B, S, heads, hd)) MT_FAIL(MT_E_ARG, "attention: workspace too small");
    const int64_t H = (int64_t)heads * hd;
    uint16_t* vt = (uint16_t*)ws;
    const float sl2 = LOG2E / sqrtf((float)hd);
    const dim3 grid((S + ATT_BQ - 1) / ATT_BQ, B * heads);
    // causal: S(S+1)/2 score entries, each 2*hd flops for QK^T and 2*hd for PV
    ProfScope prof(PROF_ATTN_FWD, 4.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    transpose_heads(qkv + 2 * H, 3 * H, B, S, heads, hd, vt, s);
    if (hd == 128)
        hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(ATT_THREADS), 0, s, qkv, vt, o, lse, S, heads, sl2);
    else
        hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(ATT_THREADS), 0, s, qkv, vt, o, lse, S, heads, sl2);
    launch_check("attention_fwd", s);
}

void attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout, uint16_t* dqkv,
                   int B, int S, int heads, int hd, void* ws, size_t ws_bytes, hipStream_t s) {
    check_attn(B, S, heads, hd);
    if (!ws || ws_bytes < attention_bwd_ws_bytes(B, S, heads, hd)) MT_FAIL(MT_E_ARG, "attention: workspace too small");
    const int64_t H = (int64_t)heads * hd;
    const size_t tb = round_up((size_t)B * S * H * 2, 256);
    uint16_t* qt = (uint16_t*)ws;
    uint16_t* kt = (uint16_t*)((char*)ws + tb);
    uint16_t* dot = (uint16_t*)((char*)ws + 2 * tb);
    float* dvec = (float*)((char*)ws + 3 * tb);
    const float scale = 1.0f / sqrtf((float)hd);
    const float sl2 = LOG2E * scale;
    const int64_t T = (int64_t)B * S;
    const int64_t n = T * heads;
    const dim3 gq((S + ATT_BQ - 1) / ATT_BQ, B * heads), gk((S + ATT_BK - 1) / ATT_BK, B * heads);
    // causal entries x (QK^T recompute, dP, dV, dK, dQ) at 2*hd flops each
    ProfScope prof(PROF_ATTN_BWD, 10.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    transpose_heads(qkv, 3 * H, B, S, heads, hd, qt, s);
    transpose_heads(qkv + H, 3 * H, B, S, heads, hd, kt, s);
    transpose_heads(dout, H, B, S, heads, hd, dot, s);
    if (hd == 128) {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<128>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o, dout, dvec,
                           T, S, heads);
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, gk, dim3(ATT_THREADS), 0, s, qkv, qt, dot, lse, dout, dvec, dqkv, S,
                           heads, sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(ATT_THREADS), 0, s, qkv, kt, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<64>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, o, dout, dvec, T,
                           S, heads);
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, gk, dim3(ATT_THREADS), 0, s, qkv, qt, dot, lse, dout, dvec, dqkv, S,
                           heads, sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(ATT_THREADS), 0, s, qkv, kt, lse, dout, dvec, dqkv, S, heads,
                           sl2, scale);
    }
    launch_check("attention_bwd", s);
}

}  // namespace mt
