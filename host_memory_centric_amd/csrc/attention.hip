// Causal attention on gfx950 matrix cores: tiled online-softmax forward and a
// backward in three kernels (dV and dK over key tiles, dQ over query tiles),
// so no gradient is ever accumulated with atomics.  The forward runs the
// 8-wave ping-pong kernel (attn_fwd_pp_kernel: the two waves of a SIMD take
// turns at the MFMAs and the softmax); the 4-wave software-pipelined kernel
// (attn_fwd_kernel, MT_ATTN_FWD=pipe) gives the same bits 7-9 % slower.
//
// Scores are computed transposed where that keeps each query's softmax state
// inside one lane: with S^T = K Q^T on v_mfma_f32_32x32x16_bf16 a lane owns
// one query column and 16 key rows of each 32x32 tile, so the row max / row
// sum need one cross-half shuffle, the running rescale of O^T = V^T P^T is a
// per-lane multiply, and the probabilities are already laid out as the B
// operand of the next MFMA.  The dK and dV kernels use the untransposed
// S = Q K^T so that each lane owns one key column.
//
// Streamed operands (K and V in the forward and dQ kernels, Q and dO in the
// dK and dV kernels) are 64-row tiles copied straight from global memory into LDS
// (global_load_lds_dwordx4, double buffered, one barrier per tile) in their
// natural [row][feature] layout.  Each tile is read two ways: along the
// feature index as an ordinary MFMA fragment (Q K^T, dO V^T), and along the
// row index through the transposing LDS read ds_read_b64_tr_b16 as the A
// operand of the products that contract over rows (V^T P^T, dO^T P, Q^T dS,
// K^T dS^T).  No operand is ever transposed in global memory or in registers.
// The 16-byte chunks of row r are XOR-swizzled with 2(r mod 4) xor (r/4 mod 2),
// which keeps both read patterns free of bank conflicts.
//
// The contraction order of a transposed-read fragment follows the accumulator
// layout of the probabilities it meets: accumulator element e of lane half h
// holds row 8(e/4) + 4h + e%4 of a 16-row step, so the transposing reads fetch
// rows 4h..4h+3 and 8+4h..8+4h+3.
//
// Every kernel has a bf16 and an fp16 instantiation (F16: v_mfma_f32_32x32x16_f16,
// same rate).  The layer runs the fp16 ones on the forward's fp16 q, k, v, so
// that the backward recomputes exactly the forward's scores: the forward's
// probabilities enter P V as fp16 scaled by 2^14 (the running maximum offset
// by 14 in the exponent, the log-sum-exp corrected back), and the backward
// takes dO and dS as fp16 under per-(batch, head) powers of two chosen from
// bounds of their magnitudes, folded exactly into the exponent of P and
// divided out in fp32 at the end.  The bf16 instantiations serve the
// mt_op_attention_* entry points.
//
// Layout: qkv is the fused projection output [B*S, 3*H] (q | k | v, head h at
// columns h*hd .. h*hd + hd - 1 of each third), o is [B*S, H], lse is
// [B, heads, S] natural-log row logsumexp of the scaled scores.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "device.h"
#include "kernels.h"

namespace mt {

constexpr int ATT_WAVES = 4;
constexpr int ATT_THREADS = ATT_WAVES * 64;
constexpr int ATT_BQ = ATT_WAVES * 32;  // queries per workgroup (fwd, dQ)
constexpr int ATT_BK = ATT_WAVES * 32;  // keys per workgroup (dK/dV)
constexpr int ATT_T = 64;               // rows per streamed tile
constexpr float LOG2E = 1.4426950408889634f;
// fp16 attention: the probabilities enter the fp16 products multiplied by
// 2^P16_EXP (they are at most 1, so at most 16384: far below fp16's 65504,
// and a probability of 1/2^19 becomes 2^-5, a normal fp16 number)
constexpr float P16_EXP = 14.f;
constexpr float P16_SCALE = 16384.f;  // 2^P16_EXP
// fp16 backward: dO is scaled per (batch, head) so that its largest element
// lies in [2^11, 2^12), and dS so that its bound 2 |dO_q|_1 max|v| lies in
// [2^12, 2^13) (fp16 holds up to 65504); both scales are powers of two.
constexpr int DO16_TOP = 11;
constexpr int DS16_TOP = 12;
constexpr float LN2 = 0.6931471805599453f;

typedef short att_v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void att_lds_void;
typedef __attribute__((address_space(3))) att_v4s att_lds_v4s;

// ---------------------------------------------------------------------------
// streamed tile: ATT_T rows x HD features, bf16, swizzled 16-byte chunks
// ---------------------------------------------------------------------------
template <int HD>
struct ATile {
    static constexpr int CPR = HD / 8;                   // chunks per row
    static constexpr int ELEMS = ATT_T * HD;
    static constexpr int INSTR = ATT_T * HD * 2 / 1024;  // 1 KB direct-load instructions per tile
    static constexpr int RPI = 1024 / (2 * HD);          // rows per instruction
    static_assert(INSTR % ATT_WAVES == 0, "instructions per wave");

    __device__ __forceinline__ static int fz(int row) { return (2 * (row & 3)) ^ ((row >> 2) & 1); }
    __device__ __forceinline__ static int phys(int row, int c) { return c ^ fz(row); }

    // rows r0 .. r0+ATT_T-1 of a [*, ld] matrix, all of them below the end
    __device__ __forceinline__ static void dma(const uint16_t* G, int64_t ld, int r0, uint16_t* T, int wave,
                                               int lane) {
#pragma unroll
        for (int jj = 0; jj < INSTR / ATT_WAVES; ++jj) {
            const int j = wave + jj * ATT_WAVES;
            const int row = j * RPI + lane / CPR, p = lane % CPR;
            const uint16_t* g = G + (int64_t)(r0 + row) * ld + 8 * (p ^ fz(row));
            __builtin_amdgcn_global_load_lds((const void*)g, (att_lds_void*)(T + j * 512), 16, 0, 0);
        }
    }
    // the last, partial tile: register path, rows at or past S are zero
    __device__ __forceinline__ static void sync(const uint16_t* G, int64_t ld, int r0, int S, uint16_t* T, int t) {
        for (int u = t; u < ATT_T * CPR; u += ATT_THREADS) {
            const int row = u / CPR, c = u % CPR;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r0 + row < S) v = *(const uint4*)(G + (int64_t)(r0 + row) * ld + 8 * c);
            *(uint4*)(T + row * HD + 8 * phys(row, c)) = v;
        }
    }
    __device__ __forceinline__ static void load(const uint16_t* G, int64_t ld, int r0, int S, uint16_t* T, int wave,
                                                int lane) {
        if (r0 + ATT_T <= S)
            dma(G, ld, r0, T, wave, lane);
        else
            sync(G, ld, r0, S, T, threadIdx.x);
    }
    // fragment along the features: row `row`, features 16*ds + 8*half .. +7
    __device__ __forceinline__ static bf16x8 frag_row(const uint16_t* T, int row, int ds, int half) {
        return as_bf16x8(*(const uint4*)(T + row * HD + 8 * phys(row, 2 * ds + half)));
    }
    // A fragment of the transposed tile: feature dbase + lane%32, contraction
    // over the tile rows of 16-row step ks in the accumulator order
    __device__ __forceinline__ static bf16x8 frag_tr(const uint16_t* T, int dbase, int ks, int lane) {
        const int g = lane >> 4, j = lane & 15;
        const int r = j >> 2, q = j & 3;
        const int m = dbase + 16 * (g & 1) + 4 * q;  // the 4 features this lane supplies
        const int kb1 = 16 * ks + 4 * (g >> 1) + r, kb2 = kb1 + 8;
        const int c = m >> 3, sub = m & 7;
        const uint16_t* a0 = T + kb1 * HD + 8 * phys(kb1, c) + sub;
        const uint16_t* a1 = T + kb2 * HD + 8 * phys(kb2, c) + sub;
        const att_v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((att_lds_v4s*)a0);
        const att_v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((att_lds_v4s*)a1);
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
};

// Work order of the causal kernels.  The blocks of a (batch, head) differ in
// length (the causal prefix), so the launch takes the (batch, head) pairs in
// groups of G and dispatches each group's blocks longest first: the short
// blocks fill the end of each group, and at the end of the launch nothing
// long starts last.  G is chosen so that a group spans about WGS workgroups
// (several rounds of the machine): at long sequences a group is one or two
// heads, whose concurrent blocks then share their K/V (or Q/dO) tiles in the
// L2; at short sequences a group spans many heads.  blockIdx.x + gridDim.x *
// blockIdx.y is the dispatch order; gridDim.x is the number of (batch, head)
// pairs and gridDim.y the number of blocks per pair.  rank 0 is the longest
// block.
template <int WGS>
__device__ __forceinline__ void attn_work(int& bh, int& rank) {
    const int nbh = (int)gridDim.x, nblk = (int)gridDim.y;
    const int lin = (int)blockIdx.x + nbh * (int)blockIdx.y;
    const int G = min(nbh, max(1, (WGS + nblk - 1) / nblk));
    const int per = G * nblk;
    const int g = lin / per, r = lin - g * per;
    const int gsz = min(G, nbh - g * G);  // the last group may hold fewer pairs
    rank = r / gsz;
    bh = g * G + (r - rank * gsz);
}

// B-operand fragment from 8 accumulator values (elements r0 .. r0+7 of a
// tile), rounded to bf16 (F16 = false) or fp16
template <bool F16 = false>
__device__ __forceinline__ bf16x8 frag_acc(const f32x16& a, int r0) {
    if constexpr (F16)
        return as_bf16x8(make_uint4(pack_h2(a[r0 + 0], a[r0 + 1]), pack_h2(a[r0 + 2], a[r0 + 3]),
                                    pack_h2(a[r0 + 4], a[r0 + 5]), pack_h2(a[r0 + 6], a[r0 + 7])));
    else
        return as_bf16x8(make_uint4(pack_bf2(a[r0 + 0], a[r0 + 1]), pack_bf2(a[r0 + 2], a[r0 + 3]),
                                    pack_bf2(a[r0 + 4], a[r0 + 5]), pack_bf2(a[r0 + 6], a[r0 + 7])));
}

// The forward's output rows: bf16 o and, when o16 is given, fp16 o16 (both
// rounded from the same normalised fp32 accumulators).
template <int HD>
__device__ __forceinline__ void store_o(const f32x16* oacc, float inv_l, uint16_t* orow, uint16_t* orow16, int half) {
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = dt * 32 + 8 * g + 4 * half;
            const float v0 = oacc[dt][4 * g] * inv_l, v1 = oacc[dt][4 * g + 1] * inv_l;
            const float v2 = oacc[dt][4 * g + 2] * inv_l, v3 = oacc[dt][4 * g + 3] * inv_l;
            *(uint2*)(orow + d) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
            if (orow16) *(uint2*)(orow16 + d) = make_uint2(pack_h2(v0, v1), pack_h2(v2, v3));
        }
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ void zero(f32x16& a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// ---------------------------------------------------------------------------
// forward, 4 waves (128 queries) per workgroup
// ---------------------------------------------------------------------------
// Software-pipelined over key tiles: while the softmax of tile j runs on the
// vector ALUs, the MFMAs of tile j+1's scores are already in flight.  K and V
// have separate double buffers with staggered loads: during step j the LDS
// holds K_{j+1} and V_j (read) while K_{j+2} and V_{j+1} arrive.
template <int HD, bool F16 = false>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(const uint16_t* __restrict__ qkv,
                                                               uint16_t* __restrict__ o, uint16_t* __restrict__ o16,
                                                               float* __restrict__ lse, int S, int heads, float sl2) {
    using TL = ATile<HD>;
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf[2][TL::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t vbuf[2][TL::ELEMS];
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    int bh, rank;
    attn_work<4096>(bh, rank);
    const int qb = nqb - 1 - rank;  // the last query block has the most keys
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    // the wave index is uniform: conditions on it become scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    for (int dt = 0; dt < HD / 32; ++dt) zero(oacc[dt]);
    float m_run = -INFINITY, l_run = 0.f;

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_T - 1) / ATT_T;
    // key tiles this wave needs: k0 <= q0 + 31
    const int nk_wave = min(nkv, (q0 + 31) / ATT_T + 1);

    auto scores = [&](const uint16_t* Ks, f32x16* st) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            zero(st[kt]);
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds)
                st[kt] = mfma32x16<F16>(TL::frag_row(Ks, kt * 32 + (lane & 31), ds, half), as_bf16x8(qf[ds]),
                                        st[kt]);
        }
    };
    auto softmax_pv = [&](f32x16* st, const uint16_t* Vs, int k0) {
        // masking only where the tile crosses this wave's diagonal or the end
        if (k0 + ATT_T - 1 > q0 || k0 + ATT_T > S) {
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
        // fp16 path: probabilities scaled by 2^P16_EXP (exact), so that the
        // small ones of long rows stay normal fp16 numbers
        const float m_sub = F16 ? m_new - P16_EXP : m_new;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, -m_sub));
                st[kt][r] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        // once the running maxima settle, most tiles leave every one of them
        // unchanged (alpha == 1 exactly): skip the rescale then
        if (__any(m_new != m_run)) {
#pragma unroll
            for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        }
        m_run = m_new;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 pb = frag_acc<F16>(st[kt], ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt)
                    oacc[dt] = mfma32x16<F16>(TL::frag_tr(Vs, dt * 32, kt * 2 + ks, lane), pb, oacc[dt]);
            }
    };

    f32x16 st_cur[2], st_nxt[2];
    // Step j: loads into the buffers not read in this step (restrict: the
    // compiler need not wait for them before the reads), the scores of tile
    // j+1, then the softmax and PV of tile j.
    auto step = [&](const uint16_t* __restrict__ kread, const uint16_t* __restrict__ vread,
                    uint16_t* __restrict__ kwrite, uint16_t* __restrict__ vwrite, int j) {
        if (j + 2 < nkv) TL::load(Kg, ld, (j + 2) * ATT_T, S, kwrite, wave, lane);
        if (j + 1 < nkv) TL::load(Vg, ld, (j + 1) * ATT_T, S, vwrite, wave, lane);
        if (j + 1 < nk_wave) scores(kread, st_nxt);
        if (j < nk_wave) softmax_pv(st_cur, vread, j * ATT_T);
    };

    TL::load(Kg, ld, 0, S, kbuf[0], wave, lane);
    TL::load(Vg, ld, 0, S, vbuf[0], wave, lane);
    if (nkv > 1) TL::load(Kg, ld, ATT_T, S, kbuf[1], wave, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    scores(kbuf[0], st_cur);
    __syncthreads();  // every wave has read K_0 before step 0 loads K_2 over it
    for (int j = 0; j < nkv; ++j) {
        const int c = j & 1;
        step(kbuf[c ^ 1], vbuf[c], kbuf[c], vbuf[c ^ 1], j);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) st_cur[kt] = st_nxt[kt];
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (qi < S) {
        const int64_t ro = ((int64_t)b * S + qi) * H + (int64_t)head * HD;
        store_o<HD>(oacc, 1.0f / l_run, o + ro, o16 ? o16 + ro : nullptr, half);
        if (half == 0) lse[(int64_t)bh * S + qi] = (m_run + log2f(l_run) - (F16 ? P16_EXP : 0.f)) * LN2;
    }
}

// ---------------------------------------------------------------------------
// forward, ping-pong: 8 waves (256 queries) per workgroup, two per SIMD.
// ---------------------------------------------------------------------------
// Each wave alternates an MFMA cluster M(j) (the scores of key tile j+1 and
// O += V_j^T P_j^T) with a vector cluster V(j+1) (the softmax of tile j+1: max,
// exp2, sum, the running rescale of O, P to bf16).  Group 1 (waves 4-7) runs
// one phase behind group 0, with one workgroup barrier between phases, so in
// every phase one wave of each SIMD feeds the matrix core while the other runs
// the softmax.  Wave (g, w) owns queries 64w + 32g .. +31 of the block, so
// both groups need about the same key tiles.
//
// LDS: two slots, slot t % 2 holding K_t and V_{t-1} (the operands of M(t-1)).
// M(t-1) runs in phases 2t (group 0) and 2t+1 (group 1); the loads of slot
// t+2 are issued by all waves at phase 2t+2 (after both groups read slot t)
// and waited for at the end of phase 2t+3, before the first read at 2t+4.
// Every wave runs the same loop of 2*NT+2 phases with one barrier each, so
// the barrier sequence is the same for all waves whatever their work.
constexpr int ATT_PP_WAVES = 8;
constexpr int ATT_PP_THREADS = ATT_PP_WAVES * 64;
constexpr int ATT_PP_BQ = ATT_PP_WAVES * 32;

template <int HD, bool F16 = false>
__global__ __launch_bounds__(ATT_PP_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_pp_kernel(
    const uint16_t* __restrict__ qkv, uint16_t* __restrict__ o, uint16_t* __restrict__ o16, float* __restrict__ lse,
    int S, int heads, float sl2) {
    using TL = ATile<HD>;
    __shared__ __attribute__((aligned(1024))) uint16_t kbuf[2][TL::ELEMS];
    __shared__ __attribute__((aligned(1024))) uint16_t vbuf[2][TL::ELEMS];
    const int nqb = (S + ATT_PP_BQ - 1) / ATT_PP_BQ;
    int bh, rank;
    attn_work<2048>(bh, rank);
    const int qb = nqb - 1 - rank;  // the last query block has the most keys
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    // the wave index is uniform: conditions on it become scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave >> 2, w4 = wave & 3;
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const int q0 = qb * ATT_PP_BQ + w4 * 64 + grp * 32;
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

    const int kv_end = min(S, qb * ATT_PP_BQ + ATT_PP_BQ);
    const int NT = (kv_end + ATT_T - 1) / ATT_T;  // key tiles of the workgroup
    const int nk_wave = min(NT, (q0 + 31) / ATT_T + 1);  // key tiles this wave needs

    // Loads of one 64-row tile (K or V) by all 8 waves: 2 (hd 128) or 1 (hd
    // 64) direct 1 KB instructions per wave, or the register path for the
    // last, partial tile.
    auto load_tile = [&](const uint16_t* G, int r0, uint16_t* __restrict__ T) __attribute__((always_inline)) {
        if (r0 + ATT_T <= S) {
#pragma unroll
            for (int jj = 0; jj < TL::INSTR / ATT_PP_WAVES; ++jj) {
                const int j = wave + jj * ATT_PP_WAVES;
                const int row = j * TL::RPI + lane / TL::CPR, pc = lane % TL::CPR;
                const uint16_t* g = G + (int64_t)(r0 + row) * ld + 8 * (pc ^ TL::fz(row));
                __builtin_amdgcn_global_load_lds((const void*)g, (att_lds_void*)(T + j * 512), 16, 0, 0);
            }
        } else {
            for (int u = threadIdx.x; u < ATT_T * TL::CPR; u += ATT_PP_THREADS) {
                const int row = u / TL::CPR, c = u % TL::CPR;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (r0 + row < S) v = *(const uint4*)(G + (int64_t)(r0 + row) * ld + 8 * c);
                *(uint4*)(T + row * HD + 8 * TL::phys(row, c)) = v;
            }
        }
    };
    // slot t: K_t (t < NT) and V_{t-1} (t >= 1)
    auto load_slot = [&](int t, uint16_t* __restrict__ kdst, uint16_t* __restrict__ vdst) __attribute__((always_inline)) {
        if (t < NT) load_tile(Kg, t * ATT_T, kdst);
        if (t >= 1) load_tile(Vg, (t - 1) * ATT_T, vdst);
    };

    f32x16 st[2];   // scores of the next tile (written in M, read in V)
    bf16x8 pb[4];   // probabilities of the current tile as MFMA operands
    // M(j): O += V_j^T P_j^T (j < nk_wave), then the scores of tile j+1
    // (j+1 < nk_wave); in this order the probabilities are dead before the
    // scores are written (registers)
    auto mcluster = [&](const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs, int j) __attribute__((always_inline)) {
        if (j >= 0 && j < nk_wave) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int dt = 0; dt < HD / 32; ++dt)
                        oacc[dt] = mfma32x16<F16>(TL::frag_tr(Vs, dt * 32, kt * 2 + ks, lane), pb[kt * 2 + ks],
                                                  oacc[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < nk_wave) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                zero(st[kt]);
#pragma unroll
                for (int ds = 0; ds < HD / 16; ++ds)
                    st[kt] = mfma32x16<F16>(TL::frag_row(Ks, kt * 32 + (lane & 31), ds, half), as_bf16x8(qf[ds]),
                                            st[kt]);
            }
        }
    };
    // V(j): softmax of tile j (j < nk_wave), the same arithmetic as attn_fwd_kernel
    auto vcluster = [&](int j) __attribute__((always_inline)) {
        if (j >= nk_wave) return;
        const int k0 = j * ATT_T;
        if (k0 + ATT_T - 1 > q0 || k0 + ATT_T > S) {
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
        // fp16 path: probabilities scaled by 2^P16_EXP (exact), so that the
        // small ones of long rows stay normal fp16 numbers
        const float m_sub = F16 ? m_new - P16_EXP : m_new;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, -m_sub));
                st[kt][r] = p;
                ps += p;
            }
        ps += __shfl_xor(ps, 32);
        l_run = l_run * alpha + ps;
        if (__any(m_new != m_run)) {
#pragma unroll
            for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
        }
        m_run = m_new;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) pb[kt * 2 + ks] = frag_acc<F16>(st[kt], ks * 8);
    };

    load_slot(0, kbuf[0], vbuf[0]);
    if (NT >= 1) load_slot(1, kbuf[1], vbuf[1]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Group 0 runs M(j) in phase 2j+2 and V(j) in phase 2j+1, group 1 one
    // phase later (its extra barrier comes first, group 0's last).  The loads
    // of slot j+2 go out in phase 2j+2 (group 0 after its M(j) cluster, group
    // 1 at the start of V(j)) and are waited for at the end of phase 2j+3.
    auto fence = [&](bool wait) __attribute__((always_inline)) {
        if (wait) __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    auto vstep = [&](int j) __attribute__((always_inline)) {
        if (grp == 1 && j + 2 <= NT) load_slot(j + 2, kbuf[j & 1], vbuf[j & 1]);  // slot j+2 has j's parity
        vcluster(j);
        fence(grp == 0);
    };
    auto mstep = [&](const uint16_t* __restrict__ Ks, const uint16_t* __restrict__ Vs, uint16_t* __restrict__ kl,
                     uint16_t* __restrict__ vl, int j) __attribute__((always_inline)) {
        mcluster(Ks, Vs, j);
        // after the cluster: the compiler makes every LDS read wait for the
        // wave's outstanding direct loads, so loads issued before the reads
        // would be waited for at once
        if (grp == 0 && j + 2 <= NT) load_slot(j + 2, kl, vl);
        fence(grp == 1);
    };
    if (grp == 1) fence(false);
    mcluster(kbuf[0], vbuf[0], -1);
    fence(false);
    for (int j = 0; j < NT; j += 2) {
        vstep(j);
        mstep(kbuf[1], vbuf[1], kbuf[0], vbuf[0], j);  // M(j) reads slot j+1 (odd), loads slot j+2 (even)
        if (j + 1 < NT) {
            vstep(j + 1);
            mstep(kbuf[0], vbuf[0], kbuf[1], vbuf[1], j + 1);
        }
    }
    if (grp == 0) fence(false);
    if (qi < S) {
        const int64_t ro = ((int64_t)b * S + qi) * H + (int64_t)head * HD;
        store_o<HD>(oacc, 1.0f / l_run, o + ro, o16 ? o16 + ro : nullptr, half);
        if (half == 0) lse[(int64_t)bh * S + qi] = (m_run + log2f(l_run) - (F16 ? P16_EXP : 0.f)) * LN2;
    }
}

// ---------------------------------------------------------------------------
// backward: D = rowsum(dO * O)
// ---------------------------------------------------------------------------
// Backward pre-passes: LG = HD / 8 lanes per (token, head) row, each lane 8
// features (16 bytes of every operand), so one load instruction of a wave
// reads 64 / LG whole rows; the row's sums and maxima are combined over its
// lanes with shuffles.
template <int LG>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = LG / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
template <int LG>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int o = LG / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// D = rowsum(dO * O) per (token, head), stored [batch, head, seq].
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                    float* __restrict__ dvec, int64_t T, int S, int heads) {
    constexpr int LG = HD / 8;
    const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LG;
    const int sub = threadIdx.x % LG;
    if (idx >= T * heads) return;  // whole groups
    const int64_t t = idx / heads;
    const int head = (int)(idx % heads);
    const int64_t off = t * (int64_t)heads * HD + (int64_t)head * HD + 8 * sub;
    const uint4 x = *(const uint4*)(o + off), y = *(const uint4*)(dout + off);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) s += bf_lo(xw[q]) * bf_lo(yw[q]) + bf_hi(xw[q]) * bf_hi(yw[q]);
    s = group_sum<LG>(s);
    if (sub == 0) dvec[((t / S) * heads + head) * S + t % S] = s;
}

// fp16 backward, first pass, per (token, head): D = rowsum(dO * O) and the
// row statistics that bound the scaled operands: |dO_row|_1, max |dO_row|,
// max |v_row| (v: the saved fp16 projection).
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_stats_kernel(const uint16_t* __restrict__ qkv16,
                                                             const uint16_t* __restrict__ o,
                                                             const uint16_t* __restrict__ dout,
                                                             float* __restrict__ stats, int64_t T, int S, int heads) {
    constexpr int LG = HD / 8;
    const int64_t idx = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LG;
    const int sub = threadIdx.x % LG;
    if (idx >= T * heads) return;  // whole groups
    const int64_t t = idx / heads;
    const int head = (int)(idx % heads);
    const int64_t H = (int64_t)heads * HD;
    const int64_t off = t * H + (int64_t)head * HD + 8 * sub;
    const uint4 x = *(const uint4*)(o + off), y = *(const uint4*)(dout + off);
    const uint4 z = *(const uint4*)(qkv16 + t * 3 * H + 2 * H + (int64_t)head * HD + 8 * sub);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w}, zw[4] = {z.x, z.y, z.z, z.w};
    float d = 0.f, l1 = 0.f, mdo = 0.f, mv = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float y0 = bf_lo(yw[q]), y1 = bf_hi(yw[q]);
        d += bf_lo(xw[q]) * y0 + bf_hi(xw[q]) * y1;
        l1 += fabsf(y0) + fabsf(y1);
        mdo = fmaxf(mdo, fmaxf(fabsf(y0), fabsf(y1)));
        mv = fmaxf(mv, fmaxf(fabsf(h2f((uint16_t)(zw[q] & 0xffff))), fabsf(h2f((uint16_t)(zw[q] >> 16)))));
    }
    d = group_sum<LG>(d);
    l1 = group_sum<LG>(l1);
    mdo = group_max<LG>(mdo);
    mv = group_max<LG>(mv);
    if (sub == 0) {
        const int64_t r = ((t / S) * heads + head) * S + t % S;
        const int64_t n = T * heads;
        stats[r] = d;
        stats[n + r] = l1;
        stats[2 * n + r] = mdo;
        stats[3 * n + r] = mv;
    }
}

// 2^k with k an integer such that x * 2^k lies in [2^top, 2^(top+1)); 1 for x == 0.
__device__ __forceinline__ float pow2_scale(float x, int top) {
    if (!(x > 0.f)) return 1.f;
    const int e = __builtin_amdgcn_frexp_expf(x) - 1;  // floor(log2 x)
    return ldexpf(1.f, max(-120, min(120, top - e)));
}

// fp16 backward, second pass, one workgroup per (batch, head): the maxima of
// the row statistics over the sequence and the two scales (dO, dS).
__global__ __launch_bounds__(256) void attn_bwd_scale_kernel(const float* __restrict__ stats, float* __restrict__ sc,
                                                             int64_t n, int S) {
    __shared__ float red[3][4];
    const int bh = blockIdx.x;
    const float* l1 = stats + n + (int64_t)bh * S;
    const float* mdo = stats + 2 * n + (int64_t)bh * S;
    const float* mv = stats + 3 * n + (int64_t)bh * S;
    float a = 0.f, b = 0.f, c = 0.f;
    for (int i = threadIdx.x; i < S; i += 256) {
        a = fmaxf(a, l1[i]);
        b = fmaxf(b, mdo[i]);
        c = fmaxf(c, mv[i]);
    }
    a = wave_max(a);
    b = wave_max(b);
    c = wave_max(c);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][w] = a;
        red[1][w] = b;
        red[2][w] = c;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float l1m = 0.f, dom = 0.f, vm = 0.f;
        for (int i = 0; i < 4; ++i) {
            l1m = fmaxf(l1m, red[0][i]);
            dom = fmaxf(dom, red[1][i]);
            vm = fmaxf(vm, red[2][i]);
        }
        const float so = pow2_scale(dom, DO16_TOP);
        const float ss = pow2_scale(2.f * l1m * so * vm, DS16_TOP);
        sc[4 * bh] = so;
        sc[4 * bh + 1] = ss;
        sc[4 * bh + 2] = (float)(__builtin_amdgcn_frexp_expf(ss) - 1);  // log2 ss, exact
        sc[4 * bh + 3] = 0.f;
    }
}

// fp16 backward, third pass: dO16 = dO * so(batch, head), exact (a power of
// two times a bf16 value inside fp16's range).
__global__ void attn_bwd_do16_kernel(const uint16_t* __restrict__ dout, const float* __restrict__ sc,
                                     uint16_t* __restrict__ do16, int64_t T, int S, int heads, int hd) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t H = (int64_t)heads * hd;
    if (idx >= T * H / 8) return;
    const int64_t e = idx * 8;
    const int64_t t = e / H;
    const int head = (int)((e % H) / hd);
    const float so = sc[4 * ((t / S) * heads + head)];
    const uint4 v = *(const uint4*)(dout + e);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = pack_h2(bf_lo(w[q]) * so, bf_hi(w[q]) * so);
    *(uint4*)(do16 + e) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// backward: dQ, one workgroup per 128 queries, loop over key tiles
// ---------------------------------------------------------------------------
// Two workgroups per CU (the LDS allows it; 256 registers per lane suffice).
// F16: q, k, v, dO (scaled by so) and dS (scaled by so * ss) are fp16 (sc:
// [batch*heads][so, ss, log2 ss, 0]); else all bf16 and sc unused.
template <int HD, bool F16 = false>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq_kernel(const uint16_t* __restrict__ qkv,
                                                                  const float* __restrict__ lse,
                                                                  const uint16_t* __restrict__ dout,
                                                                  const float* __restrict__ dvec,
                                                                  const float* __restrict__ sc,
                                                                  uint16_t* __restrict__ dqkv, int S, int heads,
                                                                  float sl2, float scale) {
    using TL = ATile<HD>;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2][2 * TL::ELEMS];  // [buffer][K | V]
    const int nqb = (S + ATT_BQ - 1) / ATT_BQ;
    int bh, rank;
    attn_work<4096>(bh, rank);
    const int qb = nqb - 1 - rank;  // the last query block has the most keys
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    // the wave index is uniform: conditions on it become scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int64_t rowbase = (int64_t)bh * S;
    const float so = F16 ? sc[4 * bh] : 1.f, ss = F16 ? sc[4 * bh + 1] : 1.f;
    // (fp16: the scale of dS folded into the exponent of P, exactly)
    const float lse2 = qi < S ? lse[rowbase + qi] * LOG2E - (F16 ? sc[4 * bh + 2] : 0.f) : 0.f;
    const float Dq = qi < S ? dvec[rowbase + qi] * so : 0.f;
    f32x16 dq[HD / 32];
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) zero(dq[dt]);

    const int kv_end = min(S, qb * ATT_BQ + ATT_BQ);
    const int nkv = (kv_end + ATT_T - 1) / ATT_T;
    auto load = [&](int t, uint16_t* __restrict__ buf) {
        TL::load(Kg, ld, t * ATT_T, S, buf, wave, lane);
        TL::load(Vg, ld, t * ATT_T, S, buf + TL::ELEMS, wave, lane);
    };
    auto step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ nxt, int kb) {
        if (kb + 1 < nkv) load(kb + 1, nxt);
        const int k0 = kb * ATT_T;
        if (k0 > q0 + 31) return;
        const uint16_t* Ks = cur;
        const uint16_t* Vs = cur + TL::ELEMS;
        f32x16 st[2], dp[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            zero(st[kt]);
            zero(dp[kt]);
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds) {
                const int row = kt * 32 + (lane & 31);
                st[kt] = mfma32x16<F16>(TL::frag_row(Ks, row, ds, half), as_bf16x8(qf[ds]), st[kt]);
                dp[kt] = mfma32x16<F16>(TL::frag_row(Vs, row, ds, half), as_bf16x8(df[ds]), dp[kt]);
            }
            if (k0 + ATT_T - 1 > q0 || k0 + ATT_T > S || q0 + 32 > S) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kt * 32 + acc_row(r, half);
                    if (key > qi || key >= S || qi >= S) st[kt][r] = -INFINITY;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(st[kt][r], sl2, -lse2));
                st[kt][r] = p * (dp[kt][r] - Dq);  // dS^T
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 sb = frag_acc<F16>(st[kt], ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt)
                    dq[dt] = mfma32x16<F16>(TL::frag_tr(Ks, dt * 32, kt * 2 + ks, lane), sb, dq[dt]);
            }
    };

    load(0, smem[0]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int kb = 0; kb < nkv; ++kb) {
        const int cur = kb & 1;
        step(smem[cur], smem[cur ^ 1], kb);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (qi < S) {
        uint16_t* row = dqkv + ((int64_t)b * S + qi) * ld + (int64_t)head * HD;
        const float sq = F16 ? scale / (so * ss) : scale;
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                *(uint2*)(row + d) = make_uint2(pack_bf2(dq[dt][4 * g] * sq, dq[dt][4 * g + 1] * sq),
                                                pack_bf2(dq[dt][4 * g + 2] * sq, dq[dt][4 * g + 3] * sq));
            }
    }
}

// ---------------------------------------------------------------------------
// backward: dV (GRAD_K = false) or dK (GRAD_K = true), one workgroup per 128
// keys, loop over query tiles.  The two gradients are separate launches: one
// kernel holding K, V, dK and dV for its keys needs about 300 registers per
// lane (one wave per SIMD); apart, each runs two workgroups per CU, which more
// than pays for recomputing Q K^T once more.
// ---------------------------------------------------------------------------
template <int HD, bool GRAD_K, bool F16 = false>
__global__ __launch_bounds__(ATT_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_kv_kernel(
    const uint16_t* __restrict__ qkv, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    const float* __restrict__ dvec, const float* __restrict__ sc, uint16_t* __restrict__ dqkv, int S, int heads,
    float sl2, float scale) {
    using TL = ATile<HD>;
    __shared__ __attribute__((aligned(1024))) uint16_t smem[2][2 * TL::ELEMS];  // [buffer][Q | dO]
    __shared__ float rs[2][2][ATT_T];  // [buffer][lse*log2(e) | D] of the tile's queries
    int bh, kbk;
    attn_work<4096>(bh, kbk);  // key block: the first has the most queries
    const int b = bh / heads, head = bh % heads;
    const int lane = threadIdx.x & 63, half = lane >> 5;
    // the wave index is uniform: conditions on it become scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t H = (int64_t)heads * HD, ld = 3 * H;
    const uint16_t* Qg = qkv + (int64_t)b * S * ld + (int64_t)head * HD;
    const uint16_t* Kg = Qg + H;
    const uint16_t* Vg = Qg + 2 * H;
    const uint16_t* dOg = dout + (int64_t)b * S * H + (int64_t)head * HD;
    const int64_t rowbase = (int64_t)bh * S;
    const float so = F16 ? sc[4 * bh] : 1.f, ss = F16 ? sc[4 * bh + 1] : 1.f;
    // fp16: the scale of the fp16 operand (dS for dK, P for dV) folded into
    // the exponent of P, exactly
    const float pexp = F16 ? (GRAD_K ? sc[4 * bh + 2] : P16_EXP) : 0.f;
    const int kw0 = kbk * ATT_BK;     // first key of the workgroup
    const int k0 = kw0 + wave * 32;   // first key of this wave
    const int kj = k0 + (lane & 31);  // key owned by this lane

    uint4 kf[HD / 16], vf[GRAD_K ? HD / 16 : 1];
#pragma unroll
    for (int ds = 0; ds < HD / 16; ++ds) {
        kf[ds] = make_uint4(0, 0, 0, 0);
        if (kj < S) kf[ds] = *(const uint4*)(Kg + (int64_t)kj * ld + ds * 16 + 8 * half);
        if constexpr (GRAD_K) {
            vf[ds] = make_uint4(0, 0, 0, 0);
            if (kj < S) vf[ds] = *(const uint4*)(Vg + (int64_t)kj * ld + ds * 16 + 8 * half);
        }
    }
    f32x16 acc[HD / 32];  // dK or dV of this lane's key
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt) zero(acc[dt]);

    const int qstart = (kw0 / ATT_T) * ATT_T;
    const int nqt = (S - qstart + ATT_T - 1) / ATT_T;
    // lse and D of a tile's queries; indices past the end are clamped (finite
    // values for rows that the mask removes)
    float rl = 0.f, rd = 0.f;
    auto fetch_rows = [&](int q0) {
        if (threadIdx.x < ATT_T) {
            const int q = min(q0 + (int)threadIdx.x, S - 1);
            rl = lse[rowbase + q] * LOG2E - pexp;
            rd = dvec[rowbase + q] * so;
        }
    };
    auto load = [&](int t, uint16_t* __restrict__ buf) {
        TL::load(Qg, ld, qstart + t * ATT_T, S, buf, wave, lane);
        TL::load(dOg, H, qstart + t * ATT_T, S, buf + TL::ELEMS, wave, lane);
    };
    auto step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ nxt, const float* __restrict__ ls,
                    const float* __restrict__ dd, int it) {
        if (it + 1 < nqt) load(it + 1, nxt);
        const int q0 = qstart + it * ATT_T;
        if (q0 + ATT_T - 1 < k0) return;  // every query of this tile precedes this wave's keys
        const uint16_t* Qs = cur;
        const uint16_t* dOs = cur + TL::ELEMS;
#pragma unroll
        for (int qt = 0; qt < ATT_T / 32; ++qt) {
            const int row = qt * 32 + (lane & 31);
            f32x16 s, dp;
            zero(s);
#pragma unroll
            for (int ds = 0; ds < HD / 16; ++ds)
                s = mfma32x16<F16>(TL::frag_row(Qs, row, ds, half), as_bf16x8(kf[ds]), s);
            if constexpr (GRAD_K) {
                zero(dp);
#pragma unroll
                for (int ds = 0; ds < HD / 16; ++ds)
                    dp = mfma32x16<F16>(TL::frag_row(dOs, row, ds, half), as_bf16x8(vf[ds]), dp);
            }
            // mask only where this 32-query sub-tile reaches below this wave's keys or past the end
            // (a uniform condition: one branch around the whole mask)
            if (q0 + qt * 32 < k0 + 31 || q0 + qt * 32 + 32 > S || k0 + 32 > S) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int q = q0 + qt * 32 + acc_row(r, half);
                    if (kj > q || q >= S || kj >= S) s[r] = -INFINITY;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int ql = qt * 32 + acc_row(r, half);
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -ls[ql]));
                if constexpr (GRAD_K)
                    s[r] = pv * (dp[r] - dd[ql]);  // dS
                else
                    s[r] = pv;  // P
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 sb = frag_acc<F16>(s, ks * 8);
#pragma unroll
                for (int dt = 0; dt < HD / 32; ++dt)
                    acc[dt] = mfma32x16<F16>(TL::frag_tr(GRAD_K ? Qs : dOs, dt * 32, qt * 2 + ks, lane), sb, acc[dt]);
            }
        }
    };

    load(0, smem[0]);
    fetch_rows(qstart);
    if (threadIdx.x < ATT_T) {
        rs[0][0][threadIdx.x] = rl;
        rs[0][1][threadIdx.x] = rd;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int it = 0; it < nqt; ++it) {
        const int cur = it & 1;
        if (it + 1 < nqt) fetch_rows(qstart + (it + 1) * ATT_T);
        step(smem[cur], smem[cur ^ 1], rs[cur][0], rs[cur][1], it);
        if (it + 1 < nqt && threadIdx.x < ATT_T) {
            rs[cur ^ 1][0][threadIdx.x] = rl;
            rs[cur ^ 1][1][threadIdx.x] = rd;
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }
    if (kj < S) {
        uint16_t* orow = dqkv + ((int64_t)b * S + kj) * ld + (GRAD_K ? H : 2 * H) + (int64_t)head * HD;
        // undo the operand scales: dK carries so * ss, dV carries so * 2^P16_EXP
        const float fs = GRAD_K ? (F16 ? scale / (so * ss) : scale) : (F16 ? 1.0f / (so * P16_SCALE) : 1.0f);
#pragma unroll
        for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = dt * 32 + 8 * g + 4 * half;
                *(uint2*)(orow + d) = make_uint2(pack_bf2(acc[dt][4 * g] * fs, acc[dt][4 * g + 1] * fs),
                                                 pack_bf2(acc[dt][4 * g + 2] * fs, acc[dt][4 * g + 3] * fs));
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
    if ((S + 127) / 128 > 65535 || (int64_t)B * heads * ((S + 127) / 128) >= (int64_t)1 << 31)
        MT_FAIL(MT_E_SHAPE, "attention: sequence too long");
}

size_t attention_fwd_ws_bytes(int, int, int, int) { return 0; }

size_t attention_bwd_ws_bytes(int B, int S, int heads, int) { return round_up((size_t)B * heads * S * 4, 256); }

// fp16 backward: row statistics [4][B*heads*S] fp32, scales [B*heads][4]
// fp32, scaled dO [B*S, heads*hd] fp16.
size_t attention_bwd16_ws_bytes(int B, int S, int heads, int hd) {
    const size_t n = (size_t)B * heads * S;
    return round_up(4 * n * 4, 256) + round_up((size_t)B * heads * 16, 256) + round_up(n * hd * 2, 256);
}

template <bool F16>
static void launch_attn_fwd(const uint16_t* qkv, uint16_t* o, uint16_t* o16, float* lse, int B, int S, int heads,
                            int hd, bool pipe, float sl2, hipStream_t s) {
    if (pipe) {
        const dim3 grid(B * heads, (S + ATT_BQ - 1) / ATT_BQ);
        if (hd == 128)
            hipLaunchKernelGGL((attn_fwd_kernel<128, F16>), grid, dim3(ATT_THREADS), 0, s, qkv, o, o16, lse, S, heads,
                               sl2);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<64, F16>), grid, dim3(ATT_THREADS), 0, s, qkv, o, o16, lse, S, heads,
                               sl2);
    } else {
        const dim3 grid(B * heads, (S + ATT_PP_BQ - 1) / ATT_PP_BQ);
        if (hd == 128)
            hipLaunchKernelGGL((attn_fwd_pp_kernel<128, F16>), grid, dim3(ATT_PP_THREADS), 0, s, qkv, o, o16, lse, S,
                               heads, sl2);
        else
            hipLaunchKernelGGL((attn_fwd_pp_kernel<64, F16>), grid, dim3(ATT_PP_THREADS), 0, s, qkv, o, o16, lse, S,
                               heads, sl2);
    }
}

void attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int B, int S, int heads, int hd, void* ws,
                   size_t ws_bytes, hipStream_t s) {
    attention_fwd_ex(qkv, false, o, nullptr, lse, B, S, heads, hd, s);
}

void attention_fwd_ex(const uint16_t* qkv, bool f16, uint16_t* o, uint16_t* o16, float* lse, int B, int S, int heads,
                      int hd, hipStream_t s) {
    check_attn(B, S, heads, hd);
    const float sl2 = LOG2E / sqrtf((float)hd);
    // causal: S(S+1)/2 score entries, each 2*hd flops for QK^T and 2*hd for PV
    ProfScope prof(PROF_ATTN_FWD, 4.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    // MT_ATTN_FWD=pipe: the 4-wave software-pipelined kernel; otherwise the
    // 8-wave ping-pong kernel (same arithmetic, bit-identical results)
    static const bool pipe = [] {
        const char* e = getenv("MT_ATTN_FWD");
        return e && strcmp(e, "pipe") == 0;
    }();
    if (f16)
        launch_attn_fwd<true>(qkv, o, o16, lse, B, S, heads, hd, pipe, sl2, s);
    else
        launch_attn_fwd<false>(qkv, o, o16, lse, B, S, heads, hd, pipe, sl2, s);
    launch_check("attention_fwd", s);
}

void attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout, uint16_t* dqkv,
                   int B, int S, int heads, int hd, void* ws, size_t ws_bytes, hipStream_t s) {
    check_attn(B, S, heads, hd);
    if (!ws || ws_bytes < attention_bwd_ws_bytes(B, S, heads, hd)) MT_FAIL(MT_E_ARG, "attention: workspace too small");
    float* dvec = (float*)ws;
    const float scale = 1.0f / sqrtf((float)hd);
    const float sl2 = LOG2E * scale;
    const int64_t T = (int64_t)B * S;
    const int64_t n = T * heads;
    const dim3 gq(B * heads, (S + ATT_BQ - 1) / ATT_BQ), gk(B * heads, (S + ATT_BK - 1) / ATT_BK);
    // causal entries x (QK^T recompute, dP, dV, dK, dQ) at 2*hd flops each (the
    // kernels execute 16*hd: Q K^T three times and dO V^T twice)
    ProfScope prof(PROF_ATTN_BWD, 10.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    if (hd == 128) {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<128>, dim3((unsigned)((n * 16 + 255) / 256)), dim3(256), 0, s, o, dout,
                           dvec, T, S, heads);
        hipLaunchKernelGGL((attn_bwd_kv_kernel<128, false>), gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr,
                           dqkv, S, heads, sl2, scale);
        hipLaunchKernelGGL((attn_bwd_kv_kernel<128, true>), gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr,
                           dqkv, S, heads, sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, gq, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr, dqkv, S,
                           heads, sl2, scale);
    } else {
        hipLaunchKernelGGL(attn_bwd_pre_kernel<64>, dim3((unsigned)((n * 8 + 255) / 256)), dim3(256), 0, s, o, dout, dvec,
                           T, S, heads);
        hipLaunchKernelGGL((attn_bwd_kv_kernel<64, false>), gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr,
                           dqkv, S, heads, sl2, scale);
        hipLaunchKernelGGL((attn_bwd_kv_kernel<64, true>), gk, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr,
                           dqkv, S, heads, sl2, scale);
        hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, gq, dim3(ATT_THREADS), 0, s, qkv, lse, dout, dvec, nullptr, dqkv, S,
                           heads, sl2, scale);
    }
    launch_check("attention_bwd", s);
}

template <int HD>
static void launch_attn_bwd16(const uint16_t* qkv16, const uint16_t* o, const float* lse, const uint16_t* dout,
                              uint16_t* dqkv, int B, int S, int heads, char* ws, float sl2, float scale, hipStream_t s) {
    const int64_t T = (int64_t)B * S, n = T * heads;
    float* stats = (float*)ws;
    float* sc = (float*)(ws + round_up(4 * (size_t)n * 4, 256));
    uint16_t* do16 = (uint16_t*)((char*)sc + round_up((size_t)B * heads * 16, 256));
    const dim3 gq(B * heads, (S + ATT_BQ - 1) / ATT_BQ), gk(B * heads, (S + ATT_BK - 1) / ATT_BK);
    hipLaunchKernelGGL(attn_bwd_stats_kernel<HD>, dim3((unsigned)((n * (HD / 8) + 255) / 256)), dim3(256), 0, s, qkv16,
                       o, dout, stats, T, S, heads);
    hipLaunchKernelGGL(attn_bwd_scale_kernel, dim3((unsigned)(B * heads)), dim3(256), 0, s, stats, sc, n, S);
    const int64_t n8 = n * HD / 8;
    hipLaunchKernelGGL(attn_bwd_do16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, dout, sc, do16, T, S,
                       heads, HD);
    hipLaunchKernelGGL((attn_bwd_kv_kernel<HD, false, true>), gk, dim3(ATT_THREADS), 0, s, qkv16, lse, do16, stats, sc,
                       dqkv, S, heads, sl2, scale);
    hipLaunchKernelGGL((attn_bwd_kv_kernel<HD, true, true>), gk, dim3(ATT_THREADS), 0, s, qkv16, lse, do16, stats, sc,
                       dqkv, S, heads, sl2, scale);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<HD, true>), gq, dim3(ATT_THREADS), 0, s, qkv16, lse, do16, stats, sc, dqkv,
                       S, heads, sl2, scale);
}

void attention_bwd16(const uint16_t* qkv16, const uint16_t* o, const float* lse, const uint16_t* dout,
                     uint16_t* dqkv, int B, int S, int heads, int hd, void* ws, size_t ws_bytes, hipStream_t s) {
    check_attn(B, S, heads, hd);
    if (!ws || ws_bytes < attention_bwd16_ws_bytes(B, S, heads, hd))
        MT_FAIL(MT_E_ARG, "attention (fp16): workspace too small");
    const float scale = 1.0f / sqrtf((float)hd);
    const float sl2 = LOG2E * scale;
    ProfScope prof(PROF_ATTN_BWD, 10.0 * hd * (double)B * heads * ((double)S * (S + 1) / 2), s);
    if (hd == 128)
        launch_attn_bwd16<128>(qkv16, o, lse, dout, dqkv, B, S, heads, (char*)ws, sl2, scale, s);
    else
        launch_attn_bwd16<64>(qkv16, o, lse, dout, dqkv, B, S, heads, (char*)ws, sl2, scale, s);
    launch_check("attention_bwd16", s);
}

// ---------------------------------------------------------------------------
// Allocation-free attention backward: the same kernels with the row dot
// products D = rowsum(dO * O) in a file-scope device array instead of a
// caller workspace, for callers that cannot allocate device memory.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_SCRATCH_BYTES];

// Device address of `scratch` on the stream's device.  The array's name in
// host code is only a handle for the runtime; its address on a device comes
// from hipGetSymbolAddress, taken once per device with that device current.
static void* static_scratch(hipStream_t s) {
    constexpr int MAX_DEV = 64;
    static std::mutex mu;
    static void* addr[MAX_DEV] = {};
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) MT_FAIL(MT_E_HIP, "attention (no-alloc): device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEV) MT_FAIL(MT_E_ARG, "attention (no-alloc): device %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) MT_FAIL(MT_E_HIP, "attention (no-alloc): hipGetDevice: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            MT_FAIL(MT_E_HIP, "attention (no-alloc): hipSetDevice(%d): %s", dev, hipGetErrorString(e));
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || p == nullptr)
            MT_FAIL(MT_E_HIP, "attention (no-alloc): hipGetSymbolAddress: %s", hipGetErrorString(e));
        if (e2 != hipSuccess) MT_FAIL(MT_E_HIP, "attention (no-alloc): hipSetDevice(%d): %s", cur, hipGetErrorString(e2));
        addr[dev] = p;
    }
    return addr[dev];
}

void attention_bwd_noalloc(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout,
                           uint16_t* dqkv, int B, int S, int heads, int hd, hipStream_t s) {
    check_attn(B, S, heads, hd);
    const size_t need = attention_bwd_ws_bytes(B, S, heads, hd);
    if (need > ATTN_STATIC_SCRATCH_BYTES)
        MT_FAIL(MT_E_ARG,
                "attention (no-alloc): batch*heads*seq = %lld rows need %zu bytes of scratch, above the %zu-byte "
                "static buffer (at most %zu rows)",
                (long long)B * heads * S, need, (size_t)ATTN_STATIC_SCRATCH_BYTES, (size_t)ATTN_STATIC_SCRATCH_BYTES / 4);
    // every element of D is written by the first kernel before it is read,
    // so the buffer needs no clearing between calls
    attention_bwd(qkv, o, lse, dout, dqkv, B, S, heads, hd, static_scratch(s), ATTN_STATIC_SCRATCH_BYTES, s);
}

}  // namespace mt
