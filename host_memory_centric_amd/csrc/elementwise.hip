// Memory-bound kernels of the layer template and the head: RMSNorm forward and
// backward (with a deterministic two-phase gain gradient), RoPE, SwiGLU,
// cross entropy, ordered sums and conversions.  All are coalesced 16-byte
// accesses with fp32 arithmetic; row reductions use wave shuffles plus one LDS
// exchange.  None uses atomics, so every result is independent of scheduling.
#include <cstdlib>

#include "common.h"
#include "device.h"
#include "kernels.h"

namespace mt {

void launch_check(const char* what, hipStream_t s) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) MT_FAIL(MT_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
    static const bool sync = getenv("MT_SYNC_CHECK") && atoi(getenv("MT_SYNC_CHECK")) != 0;
    if (sync) {
        e = hipStreamSynchronize(s);
        if (e != hipSuccess) MT_FAIL(MT_E_HIP, "%s: %s", what, hipGetErrorString(e));
    }
}

constexpr int NORM_THREADS = 256;
constexpr int NORM_MAXC = 8;  // supports h <= 8 * 256 * 8 = 16384; kernels are instantiated per chunk count
constexpr int NORM_ROWS = 16; // rows per workgroup in the backward

// RMSNorm forward, one wave per row (four rows per workgroup): each lane
// holds NV 16-byte chunks of the row (columns 8 * (lane + 64 i)), the sum of
// squares is one wave reduction, and the output goes to bf16 y and, when y16
// is given, to fp16 y16 as well (both rounded from the same fp32 value).
template <int NV>
__global__ __launch_bounds__(256) void rmsnorm_fwd_wave_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ g,
                                                               uint16_t* __restrict__ y, uint16_t* __restrict__ y16,
                                                               float* __restrict__ rstd, int64_t T, int h, float eps) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= T) return;  // whole waves
    const uint16_t* xr = x + row * h;
    uint4 xv[NV];
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int c = (lane + 64 * it) * 8;
        xv[it] = make_uint4(0, 0, 0, 0);
        if (c < h) {
            xv[it] = *(const uint4*)(xr + c);
            const uint32_t w[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float a = bf_lo(w[q]), b = bf_hi(w[q]);
                ss += a * a + b * b;
            }
        }
    }
    const float r = 1.0f / sqrtf(wave_sum(ss) / (float)h + eps);
    if (lane == 0 && rstd) rstd[row] = r;
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int c = (lane + 64 * it) * 8;
        if (c < h) {
            const uint4 gv = *(const uint4*)(g + c);
            const uint32_t w[4] = {xv[it].x, xv[it].y, xv[it].z, xv[it].w};
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
            float v[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                v[2 * q] = (bf_lo(w[q]) * r) * bf_lo(gw[q]);
                v[2 * q + 1] = (bf_hi(w[q]) * r) * bf_hi(gw[q]);
            }
            if (y)
                *(uint4*)(y + row * h + c) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                                        pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
            if (y16)
                *(uint4*)(y16 + row * h + c) = make_uint4(pack_h2(v[0], v[1]), pack_h2(v[2], v[3]),
                                                          pack_h2(v[4], v[5]), pack_h2(v[6], v[7]));
        }
    }
}

void rmsnorm_fwd2(const uint16_t* x, const uint16_t* g, uint16_t* y, uint16_t* y16, float* rstd, int64_t T, int h,
                  float eps, hipStream_t s) {
    if (h % 8 || h > 64 * 8 * 32) MT_FAIL(MT_E_SHAPE, "rmsnorm: unsupported h=%d", h);
    if (T <= 0) return;
    const int nv = (h + 511) / 512;
    const dim3 grid((unsigned)((T + 3) / 4));
#define MT_NORM_FWD2(NVV)                                                                                     \
    if (nv <= NVV) {                                                                                          \
        hipLaunchKernelGGL(rmsnorm_fwd_wave_kernel<NVV>, grid, dim3(256), 0, s, x, g, y, y16, rstd, T, h, eps); \
        launch_check("rmsnorm_fwd", s);                                                                       \
        return;                                                                                               \
    }
    MT_NORM_FWD2(1) MT_NORM_FWD2(2) MT_NORM_FWD2(4) MT_NORM_FWD2(8) MT_NORM_FWD2(10) MT_NORM_FWD2(12)
    MT_NORM_FWD2(16) MT_NORM_FWD2(20) MT_NORM_FWD2(24) MT_NORM_FWD2(32)
#undef MT_NORM_FWD2
}

template <int NC>
__global__ __launch_bounds__(NORM_THREADS) void rmsnorm_bwd_kernel(
    const float* __restrict__ dy, const uint16_t* __restrict__ x, const float* __restrict__ rstd,
    const uint16_t* __restrict__ g, const float* __restrict__ resid, float* __restrict__ dx,
    uint16_t* __restrict__ dxb, float* __restrict__ dg_part, int64_t T, int h) {
    __shared__ float red[NORM_THREADS / 64];
    float dga[NC][8];
    float gf[NC][8];
#pragma unroll
    for (int it = 0; it < NC; ++it) {
        const int c = (threadIdx.x + it * NORM_THREADS) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            dga[it][e] = 0.f;
            gf[it][e] = 0.f;
        }
        if (c < h) {
            const uint4 gv = *(const uint4*)(g + c);
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gf[it][2 * q] = bf_lo(gw[q]);
                gf[it][2 * q + 1] = bf_hi(gw[q]);
            }
        }
    }
    const float inv_h = 1.0f / (float)h;
    const int64_t r0 = (int64_t)blockIdx.x * NORM_ROWS;
    for (int rr = 0; rr < NORM_ROWS; ++rr) {
        const int64_t row = r0 + rr;
        if (row >= T) break;  // uniform across the block
        const float r = rstd[row];
        float xh[NC][8], gy[NC][8];
        float dot = 0.f;
#pragma unroll
        for (int it = 0; it < NC; ++it) {
            const int c = (threadIdx.x + it * NORM_THREADS) * 8;
            if (c < h) {
                const uint4 xv = *(const uint4*)(x + row * h + c);
                const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
                const float4 d0 = *(const float4*)(dy + row * h + c);
                const float4 d1 = *(const float4*)(dy + row * h + c + 4);
                const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    xh[it][2 * q] = bf_lo(w[q]) * r;
                    xh[it][2 * q + 1] = bf_hi(w[q]) * r;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    gy[it][e] = dv[e] * gf[it][e];
                    dot += gy[it][e] * xh[it][e];
                    dga[it][e] += dv[e] * xh[it][e];
                }
            }
        }
        const float mean = block_sum<NORM_THREADS>(dot, red) * inv_h;
#pragma unroll
        for (int it = 0; it < NC; ++it) {
            const int c = (threadIdx.x + it * NORM_THREADS) * 8;
            if (c < h) {
                float o[8];
                float4 rs0 = make_float4(0, 0, 0, 0), rs1 = rs0;
                if (resid) {
                    rs0 = *(const float4*)(resid + row * h + c);
                    rs1 = *(const float4*)(resid + row * h + c + 4);
                }
                const float rv[8] = {rs0.x, rs0.y, rs0.z, rs0.w, rs1.x, rs1.y, rs1.z, rs1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = r * (gy[it][e] - xh[it][e] * mean) + rv[e];
                if (dx) {
                    *(float4*)(dx + row * h + c) = make_float4(o[0], o[1], o[2], o[3]);
                    *(float4*)(dx + row * h + c + 4) = make_float4(o[4], o[5], o[6], o[7]);
                }
                if (dxb)
                    *(uint4*)(dxb + row * h + c) = make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]),
                                                              pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7]));
            }
        }
    }
#pragma unroll
    for (int it = 0; it < NC; ++it) {
        const int c = (threadIdx.x + it * NORM_THREADS) * 8;
        if (c < h) {
            float* out = dg_part + (int64_t)blockIdx.x * h + c;
            *(float4*)out = make_float4(dga[it][0], dga[it][1], dga[it][2], dga[it][3]);
            *(float4*)(out + 4) = make_float4(dga[it][4], dga[it][5], dga[it][6], dga[it][7]);
        }
    }
}

int64_t rmsnorm_bwd_blocks(int64_t T) { return (T + NORM_ROWS - 1) / NORM_ROWS; }

void rmsnorm_bwd(const float* dy, const uint16_t* x, const float* rstd, const uint16_t* g, const float* resid,
                 float* dx, uint16_t* dx_b, float* dg_part, int64_t T, int h, hipStream_t s) {
    if (h % 8 || h > NORM_THREADS * 8 * NORM_MAXC) MT_FAIL(MT_E_SHAPE, "rmsnorm: unsupported h=%d", h);
    if (T <= 0) return;
    const int nc = (h + NORM_THREADS * 8 - 1) / (NORM_THREADS * 8);
    const dim3 grid((unsigned)rmsnorm_bwd_blocks(T));
#define MT_NORM_BWD(NCV) \
    case NCV: hipLaunchKernelGGL(rmsnorm_bwd_kernel<NCV>, grid, dim3(NORM_THREADS), 0, s, dy, x, rstd, g, resid, dx, dx_b, dg_part, T, h); break;
    switch (nc) { MT_NORM_BWD(1) MT_NORM_BWD(2) MT_NORM_BWD(3) MT_NORM_BWD(4) MT_NORM_BWD(5) MT_NORM_BWD(6) MT_NORM_BWD(7) MT_NORM_BWD(8) }
#undef MT_NORM_BWD
    launch_check("rmsnorm_bwd", s);
}

// Column sums of the gain partials in a fixed order: 16 row groups per column
// (group g sums rows g, g+16, ... in ascending order), then the 16 group sums
// in ascending group order.
__global__ __launch_bounds__(1024) void colsum_kernel(const float* __restrict__ part, int64_t nblk, int h,
                                                      uint16_t* __restrict__ out) {
    __shared__ float red[16][64];
    const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + c;
    float v = 0.f;
    if (j < h)
        for (int64_t b = rg; b < nblk; b += 16) v += part[b * h + j];
    red[rg][c] = v;
    __syncthreads();
    if (rg == 0 && j < h) {
        float t = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) t += red[g][c];
        out[j] = f2bf(t);
    }
}

void colsum_to_bf16(const float* part, int64_t nblk, int h, uint16_t* out, hipStream_t s) {
    hipLaunchKernelGGL(colsum_kernel, dim3((h + 63) / 64), dim3(1024), 0, s, part, nblk, h, out);
    launch_check("colsum", s);
}

// RoPE: one thread rotates 8 consecutive pairs (i, i + hd/2) of q or k.
__global__ void rope_kernel(uint16_t* __restrict__ qkv, const float* __restrict__ cs, const float* __restrict__ sn,
                            int64_t T, int S, int heads, int hd, int inverse) {
    const int half = hd / 2, groups = half / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_tok = (int64_t)2 * heads * groups;
    if (idx >= T * per_tok) return;
    const int64_t t = idx / per_tok;
    int rem = (int)(idx % per_tok);
    const int which = rem / (heads * groups);  // 0: q, 1: k
    rem %= heads * groups;
    const int head = rem / groups, gi = rem % groups;
    const int s = (int)(t % S);
    const int64_t h3 = (int64_t)3 * heads * hd;
    uint16_t* base = qkv + t * h3 + (int64_t)which * heads * hd + (int64_t)head * hd + gi * 8;
    const uint4 a = *(const uint4*)base;
    const uint4 b = *(const uint4*)(base + half);
    const float* cp = cs + (int64_t)s * half + gi * 8;
    const float* sp = sn + (int64_t)s * half + gi * 8;
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t ao[4], bo[4];
    const float sg = inverse ? -1.f : 1.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float c0 = cp[2 * q], c1 = cp[2 * q + 1];
        const float s0 = sg * sp[2 * q], s1 = sg * sp[2 * q + 1];
        const float a0 = bf_lo(aw[q]), a1 = bf_hi(aw[q]), b0 = bf_lo(bw[q]), b1 = bf_hi(bw[q]);
        ao[q] = pack_bf2(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        bo[q] = pack_bf2(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
    }
    *(uint4*)base = make_uint4(ao[0], ao[1], ao[2], ao[3]);
    *(uint4*)(base + half) = make_uint4(bo[0], bo[1], bo[2], bo[3]);
}

// The fused projection's fp32 output, finished: rows t0 .. t0+rows-1 of
// qkv32 ([rows, 3h], fp32) hold tokens t0 ... of the batch; q and k are
// rotated by RoPE in fp32 and every value is rounded once, to bf16 into qkv
// and to fp16 into qkv16 (both [T, 3h]).  One thread: 8 pairs (i, i + hd/2)
// of one head of q, k or v (v is only converted).
__global__ void qkv_finish_kernel(const float* __restrict__ qkv32, uint16_t* __restrict__ qkv,
                                  uint16_t* __restrict__ qkv16, const float* __restrict__ cs,
                                  const float* __restrict__ sn, int64_t t0, int64_t rows, int S, int heads, int hd,
                                  int interleaved) {
    const int half = hd / 2, groups = half / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_tok = (int64_t)3 * heads * groups;
    if (idx >= rows * per_tok) return;
    const int64_t tr = idx / per_tok;
    int rem = (int)(idx % per_tok);
    const int which = rem / (heads * groups);  // 0: q, 1: k, 2: v
    rem %= heads * groups;
    const int head = rem / groups, gi = rem % groups;
    const int64_t t = t0 + tr;
    const int s = (int)(t % S);
    const int64_t h3 = (int64_t)3 * heads * hd;
    const int64_t col = (int64_t)which * heads * hd + (int64_t)head * hd + gi * 8;
    float a[8], b[8];
    if (interleaved && which < 2) {
        // features (p, p + hd/2) of pair p at columns 2p, 2p + 1 of the head
        const float* src = qkv32 + tr * h3 + (int64_t)which * heads * hd + (int64_t)head * hd + 2 * (gi * 8);
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float4 v = *(const float4*)(src + 2 * e);
            a[e] = v.x;
            b[e] = v.y;
            a[e + 1] = v.z;
            b[e + 1] = v.w;
        }
    } else {
        const float* src = qkv32 + tr * h3 + col;
        const float4 a0 = *(const float4*)src, a1 = *(const float4*)(src + 4);
        const float4 b0 = *(const float4*)(src + half), b1 = *(const float4*)(src + half + 4);
        a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w; a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
        b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
    }
    if (which < 2) {
        const float* cp = cs + (int64_t)s * half + gi * 8;
        const float* sp = sn + (int64_t)s * half + gi * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float c = cp[e], si = sp[e];
            const float ra = a[e] * c - b[e] * si, rb = b[e] * c + a[e] * si;
            a[e] = ra;
            b[e] = rb;
        }
    }
    if (qkv) {
        uint16_t* d = qkv + t * h3 + col;
        *(uint4*)d = make_uint4(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(a[4], a[5]), pack_bf2(a[6], a[7]));
        *(uint4*)(d + half) =
            make_uint4(pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3]), pack_bf2(b[4], b[5]), pack_bf2(b[6], b[7]));
    }
    uint16_t* d16 = qkv16 + t * h3 + col;
    *(uint4*)d16 = make_uint4(pack_h2(a[0], a[1]), pack_h2(a[2], a[3]), pack_h2(a[4], a[5]), pack_h2(a[6], a[7]));
    *(uint4*)(d16 + half) =
        make_uint4(pack_h2(b[0], b[1]), pack_h2(b[2], b[3]), pack_h2(b[4], b[5]), pack_h2(b[6], b[7]));
}

void qkv_finish(const float* qkv32, uint16_t* qkv, uint16_t* qkv16, const float* cos, const float* sin, int64_t t0,
                int64_t rows, int S, int heads, int hd, bool interleaved, hipStream_t s) {
    if (hd % 16) MT_FAIL(MT_E_SHAPE, "qkv_finish: head_dim %d must be a multiple of 16", hd);
    const int64_t n = rows * 3 * heads * (hd / 16);
    if (n == 0) return;
    hipLaunchKernelGGL(qkv_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, qkv32, qkv, qkv16, cos,
                       sin, t0, rows, S, heads, hd, interleaved ? 1 : 0);
    launch_check("qkv_finish", s);
}

void rope_apply(uint16_t* qkv, const float* cos, const float* sin, int64_t T, int S, int heads, int hd, bool inverse,
                hipStream_t s) {
    if (hd % 16) MT_FAIL(MT_E_SHAPE, "rope: head_dim %d must be a multiple of 16", hd);
    const int64_t n = T * 2 * heads * (hd / 16);
    if (n == 0) return;
    hipLaunchKernelGGL(rope_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, qkv, cos, sin, T, S, heads,
                       hd, inverse ? 1 : 0);
    launch_check("rope", s);
}


__global__ void swiglu_fwd_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ a, int64_t T, int f) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = f / 8;
    if (idx >= T * per) return;
    const int64_t t = idx / per;
    const int c = (int)(idx % per) * 8;
    const uint4 gv = *(const uint4*)(gu + t * 2 * f + c);
    const uint4 uv = *(const uint4*)(gu + t * 2 * f + f + c);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float g0 = bf_lo(gw[q]), g1 = bf_hi(gw[q]);
        o[q] = pack_bf2(g0 * sigmoidf_(g0) * bf_lo(uw[q]), g1 * sigmoidf_(g1) * bf_hi(uw[q]));
    }
    *(uint4*)(a + t * f + c) = make_uint4(o[0], o[1], o[2], o[3]);
}

__global__ void swiglu_bwd_kernel(const uint16_t* __restrict__ da, const uint16_t* __restrict__ gu,
                                  uint16_t* __restrict__ dgu, int64_t T, int f) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = f / 8;
    if (idx >= T * per) return;
    const int64_t t = idx / per;
    const int c = (int)(idx % per) * 8;
    const uint4 dv = *(const uint4*)(da + t * f + c);
    const uint4 gv = *(const uint4*)(gu + t * 2 * f + c);
    const uint4 uv = *(const uint4*)(gu + t * 2 * f + f + c);
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w},
                   uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t og[4], ou[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float dg[2], du[2];
        const float d2[2] = {bf_lo(dw[q]), bf_hi(dw[q])}, g2[2] = {bf_lo(gw[q]), bf_hi(gw[q])},
                    u2[2] = {bf_lo(uw[q]), bf_hi(uw[q])};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float sg = sigmoidf_(g2[e]);
            dg[e] = d2[e] * u2[e] * sg * (1.0f + g2[e] * (1.0f - sg));
            du[e] = d2[e] * (g2[e] * sg);
        }
        og[q] = pack_bf2(dg[0], dg[1]);
        ou[q] = pack_bf2(du[0], du[1]);
    }
    *(uint4*)(dgu + t * 2 * f + c) = make_uint4(og[0], og[1], og[2], og[3]);
    *(uint4*)(dgu + t * 2 * f + f + c) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
}

// SwiGLU from the gate/up projection's fp32 output gu32 [rows, 2f]:
// a = silu(gate) * up in fp32, rounded once to bf16 (a, [rows, f]) and to
// fp16 (a16, [rows, f]).
__global__ void swiglu_fwd32_kernel(const float* __restrict__ gu32, uint16_t* __restrict__ gu,
                                    uint16_t* __restrict__ a, uint16_t* __restrict__ a16, int64_t rows, int f,
                                    int interleaved) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per = f / 8;
    if (idx >= rows * per) return;
    const int64_t t = idx / per;
    const int c = (int)(idx % per) * 8;
    float gv[8], uv[8];
    if (interleaved) {
        const float* src = gu32 + t * 2 * f + 2 * c;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float4 v = *(const float4*)(src + 2 * e);
            gv[e] = v.x;
            uv[e] = v.y;
            gv[e + 1] = v.z;
            uv[e + 1] = v.w;
        }
    } else {
        const float* gr = gu32 + t * 2 * f + c;
        const float4 g0 = *(const float4*)gr, g1 = *(const float4*)(gr + 4);
        const float4 u0 = *(const float4*)(gr + f), u1 = *(const float4*)(gr + f + 4);
        gv[0] = g0.x; gv[1] = g0.y; gv[2] = g0.z; gv[3] = g0.w; gv[4] = g1.x; gv[5] = g1.y; gv[6] = g1.z; gv[7] = g1.w;
        uv[0] = u0.x; uv[1] = u0.y; uv[2] = u0.z; uv[3] = u0.w; uv[4] = u1.x; uv[5] = u1.y; uv[6] = u1.z; uv[7] = u1.w;
    }
    if (gu) {
        *(uint4*)(gu + t * 2 * f + c) = make_uint4(pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3]),
                                                   pack_bf2(gv[4], gv[5]), pack_bf2(gv[6], gv[7]));
        *(uint4*)(gu + t * 2 * f + f + c) = make_uint4(pack_bf2(uv[0], uv[1]), pack_bf2(uv[2], uv[3]),
                                                       pack_bf2(uv[4], uv[5]), pack_bf2(uv[6], uv[7]));
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = swiglu_f(gv[e], uv[e]);
    if (a)
        *(uint4*)(a + t * f + c) =
            make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
    if (a16)
        *(uint4*)(a16 + t * f + c) =
            make_uint4(pack_h2(v[0], v[1]), pack_h2(v[2], v[3]), pack_h2(v[4], v[5]), pack_h2(v[6], v[7]));
}

void swiglu_fwd32(const float* gu32, uint16_t* gu, uint16_t* a, uint16_t* a16, int64_t rows, int f, bool interleaved,
                  hipStream_t s) {
    const int64_t n = rows * (f / 8);
    if (n == 0) return;
    hipLaunchKernelGGL(swiglu_fwd32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu32, gu, a, a16, rows,
                       f, interleaved ? 1 : 0);
    launch_check("swiglu_fwd32", s);
}

// bf16 -> fp16 (exact for every bf16 value inside fp16's range; weights of
// the layer template, |w| << 65504), 8 values per thread.
__global__ void bf16_to_f16_kernel(const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const uint4 v = *(const uint4*)(x + 8 * i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_h2(bf_lo(w[q]), bf_hi(w[q]));
    *(uint4*)(y + 8 * i) = make_uint4(o[0], o[1], o[2], o[3]);
}

void bf16_to_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t s) {
    if (n % 8) MT_FAIL(MT_E_SHAPE, "bf16_to_f16: %lld elements, not a multiple of 8", (long long)n);
    const int64_t n8 = n / 8;
    if (n8 == 0) return;
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, y, n8);
    launch_check("bf16_to_f16", s);
}

// bf16 -> fp16 with a transpose: each lane moves one 8x8 block (eight
// 16-byte row loads, an in-register transpose, eight 16-byte stores); the 64
// lanes of a wave cover a 64x64 tile, so that every load and store
// instruction touches eight whole 128-byte rows.  Four waves per workgroup
// take four consecutive column tiles.
// Source row of output column c of the permuted transpose (see bf16_to_f16_t).
__device__ __forceinline__ int64_t perm_src(int64_t c, int perm, int64_t pa, int64_t pb, int64_t rows) {
    if (perm == 1 && c < pa) {
        const int64_t o = c % pb;
        return c - o + o / 2 + (o & 1) * (pb / 2);
    }
    if (perm == 2) return c / 2 + (c & 1) * (rows / 2);
    return c;
}

__global__ __launch_bounds__(256) void bf16_to_f16_t_kernel(const uint16_t* __restrict__ x,
                                                            uint16_t* __restrict__ y, int64_t rows,
                                                            int64_t cols, int perm, int64_t pa, int64_t pb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.y * 64 + 8 * (lane >> 3);
    const int64_t c0 = ((int64_t)blockIdx.x * 4 + wave) * 64 + 8 * (lane & 7);
    if (r0 >= rows || c0 >= cols) return;
    uint32_t in[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint4 v = *(const uint4*)(x + perm_src(r0 + i, perm, pa, pb, rows) * cols + c0);
        in[i][0] = v.x;
        in[i][1] = v.y;
        in[i][2] = v.z;
        in[i][3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (j & 1) ? bf_hi(in[i][j >> 1]) : bf_lo(in[i][j >> 1]);
        *(uint4*)(y + (c0 + j) * rows + r0) =
            make_uint4(pack_h2(f[0], f[1]), pack_h2(f[2], f[3]), pack_h2(f[4], f[5]), pack_h2(f[6], f[7]));
    }
}

void bf16_to_f16_t(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols, int perm, int64_t pa, int64_t pb,
                   hipStream_t s) {
    if (rows % 8 || cols % 8)
        MT_FAIL(MT_E_SHAPE, "bf16_to_f16_t: %lld x %lld, not multiples of 8", (long long)rows, (long long)cols);
    if ((perm == 1 && (pb < 2 || pb % 2 || pa % pb || pa > rows)) || (perm == 2 && rows % 2) || perm < 0 || perm > 2)
        MT_FAIL(MT_E_ARG, "bf16_to_f16_t: bad permutation %d (%lld, %lld)", perm, (long long)pa, (long long)pb);
    if (rows == 0 || cols == 0) return;
    const dim3 grid((unsigned)((cols + 255) / 256), (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(bf16_to_f16_t_kernel, grid, dim3(256), 0, s, x, y, rows, cols, perm, pa, pb);
    launch_check("bf16_to_f16_t", s);
}

void swiglu_fwd(const uint16_t* gu, uint16_t* a, int64_t T, int f, hipStream_t s) {
    const int64_t n = T * (f / 8);
    if (n == 0) return;
    hipLaunchKernelGGL(swiglu_fwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, gu, a, T, f);
    launch_check("swiglu_fwd", s);
}

void swiglu_bwd(const uint16_t* da, const uint16_t* gu, uint16_t* dgu, int64_t T, int f, hipStream_t s) {
    const int64_t n = T * (f / 8);
    if (n == 0) return;
    hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, da, gu, dgu, T, f);
    launch_check("swiglu_bwd", s);
}

constexpr int CE_THREADS = 256;

// One workgroup per row: online max/sum over the vocabulary, then
// dz = (exp(z - lse) - onehot) / N for labelled rows, 0 for the last position
// of each sequence.
__global__ __launch_bounds__(CE_THREADS) void ce_kernel(const float* __restrict__ z, const int32_t* __restrict__ tok,
                                                        int64_t t0, int S, int V, float inv_n,
                                                        float* __restrict__ row_loss, uint16_t* __restrict__ dz) {
    __shared__ float red[CE_THREADS / 64];
    const int64_t r = blockIdx.x;
    const int64_t t = t0 + r;
    const float* zr = z + r * V;
    const bool labelled = (t % S) != (S - 1);
    const int label = labelled ? tok[t + 1] : -1;
    float m = -INFINITY, sum = 0.f;
    for (int c = threadIdx.x * 4; c < V; c += CE_THREADS * 4) {
        const float4 v = *(const float4*)(zr + c);
        const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        if (mx > m) {
            sum *= __expf(m - mx);
            m = mx;
        }
        sum += __expf(v.x - m) + __expf(v.y - m) + __expf(v.z - m) + __expf(v.w - m);
    }
    const float M = block_max<CE_THREADS>(m, red);
    const float tot = block_sum<CE_THREADS>(m == -INFINITY ? 0.f : sum * __expf(m - M), red);
    const float lse = M + __logf(tot);
    if (threadIdx.x == 0) row_loss[r] = labelled ? lse - zr[label] : 0.f;
    uint16_t* dr = dz + r * V;
    for (int c = threadIdx.x * 4; c < V; c += CE_THREADS * 4) {
        const float4 v = *(const float4*)(zr + c);
        float o[4] = {0.f, 0.f, 0.f, 0.f};
        if (labelled) {
            o[0] = __expf(v.x - lse) * inv_n - (c + 0 == label ? inv_n : 0.f);
            o[1] = __expf(v.y - lse) * inv_n - (c + 1 == label ? inv_n : 0.f);
            o[2] = __expf(v.z - lse) * inv_n - (c + 2 == label ? inv_n : 0.f);
            o[3] = __expf(v.w - lse) * inv_n - (c + 3 == label ? inv_n : 0.f);
        }
        *(uint2*)(dr + c) = make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    }
}

void cross_entropy(const float* z, const int32_t* tokens, int64_t t0, int64_t rows, int S, int V, float inv_n,
                   float* row_loss, uint16_t* dz, hipStream_t s) {
    if (V % 4) MT_FAIL(MT_E_SHAPE, "cross entropy: vocab %d must be a multiple of 4", V);
    if (rows <= 0) return;
    hipLaunchKernelGGL(ce_kernel, dim3((unsigned)rows), dim3(CE_THREADS), 0, s, z, tokens, t0, S, V, inv_n, row_loss,
                       dz);
    launch_check("cross_entropy", s);
}

__global__ __launch_bounds__(1024) void sum_kernel(const float* __restrict__ v, int64_t n, float scale,
                                                   float* __restrict__ out) {
    __shared__ float red[1024];
    float s = 0.f;
    for (int64_t i = threadIdx.x; i < n; i += 1024) s += v[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0] * scale;
}

void sum_scaled(const float* v, int64_t n, float scale, float* out, hipStream_t s) {
    hipLaunchKernelGGL(sum_kernel, dim3(1), dim3(1024), 0, s, v, n, scale, out);
    launch_check("sum", s);
}

__global__ void f2bf_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= n) return;
    if (i + 8 <= n) {
        const float4 a = *(const float4*)(x + i), b = *(const float4*)(x + i + 4);
        *(uint4*)(y + i) = make_uint4(pack_bf2(a.x, a.y), pack_bf2(a.z, a.w), pack_bf2(b.x, b.y), pack_bf2(b.z, b.w));
    } else {
        for (int64_t k = i; k < n; ++k) y[k] = f2bf(x[k]);
    }
}

void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s) {
    if (n <= 0) return;
    const int64_t th = (n + 7) / 8;
    hipLaunchKernelGGL(f2bf_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, s, x, y, n);
    launch_check("f32_to_bf16", s);
}

}  // namespace mt
