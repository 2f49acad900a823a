// Host-side launchers of the gfx950 kernels used by the layer template.
#pragma once
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"

namespace mt {

// Check the last launch (and, with MT_SYNC_CHECK=1, synchronise the stream).
void launch_check(const char* what, hipStream_t s = nullptr);

// Kernel timing (see mt_prof_enable): a scope that records a start event on
// construction and an end event on destruction, when timing is on.
enum ProfClass { PROF_GEMM_NT = 0, PROF_GEMM_NN, PROF_GEMM_TN, PROF_ATTN_FWD, PROF_ATTN_BWD, PROF_GEMM_FWD16, PROF_N };
struct ProfScope {
    ProfScope(ProfClass c, double flops, hipStream_t s);
    ~ProfScope();
    int idx = -1;
    hipStream_t s;
};

struct GemmDesc {
    int64_t M = 0, N = 0, K = 0;
    const void* A = nullptr;
    int64_t lda = 0;
    bool a_kmajor = true;
    const void* B = nullptr;
    int64_t ldb = 0;
    bool b_kmajor = true;
    float* Cf = nullptr;        // fp32 output (optional)
    void* Cb = nullptr;         // bf16 output (optional)
    const void* R = nullptr;    // bf16 residual added before storing (optional)
    int64_t ldc = 0;
    int accumulate = 0;         // Cf += result
    void* ws = nullptr;         // split-K scratch (fp32)
    size_t ws_bytes = 0;
    bool f16 = false;           // A and B hold fp16 (not bf16) values; A K-major only
    // Fused epilogue (fp16 operands, gemm_epi_ok shapes; no Cf, R, accumulation):
    //  epi 1: RoPE on interleaved q/k pairs (columns below rope_cols), every column
    //    stored de-interleaved as fp16 into Cb;
    //  epi 2: SwiGLU on interleaved gate/up pairs: Cb = gate | up (bf16, optional),
    //    Ca = silu(gate) * up (bf16, optional), Ca16 the same as fp16 (optional),
    //    both [M, N/2].
    int epi = 0;
    const float* rope_cos = nullptr;
    const float* rope_sin = nullptr;
    int rope_S = 0, rope_hd = 0;
    int64_t rope_t0 = 0, rope_cols = 0;
    void* Ca = nullptr;
    void* Ca16 = nullptr;
};
void gemm(const GemmDesc& d, hipStream_t s);
// Whether an M x N x K GEMM (A K-major) can take a fused epilogue.
bool gemm_epi_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb);
int gemm_pick_splits(int64_t M, int64_t N, int64_t K);
size_t gemm_splitk_bytes(int64_t M, int64_t N, int64_t K);

// Backward: dx = resid + rstd * (dy*g - xh * mean(dy*g*xh)); writes fp32 and
// bf16 dx (either may be NULL), and per-row-block partials of dg.
int64_t rmsnorm_bwd_blocks(int64_t T);
void rmsnorm_bwd(const float* dy, const uint16_t* x, const float* rstd, const uint16_t* g, const float* resid,
                 float* dx, uint16_t* dx_b, float* dg_part, int64_t T, int h, hipStream_t s);
// dg[j] = sum over blocks (in order) of part[b][j], stored bf16.
void colsum_to_bf16(const float* part, int64_t nblk, int h, uint16_t* out, hipStream_t s);

// RoPE on the q and k parts of a fused [T, 3h] buffer (in place); inverse
// rotation when `inverse`.
void rope_apply(uint16_t* qkv, const float* cos, const float* sin, int64_t T, int S, int heads, int hd,
                bool inverse, hipStream_t s);

// RMSNorm forward, one wave per row: bf16 y and fp16 y16 from the same fp32
// values, and rstd fp32 [T] (each output skipped when NULL).
void rmsnorm_fwd2(const uint16_t* x, const uint16_t* g, uint16_t* y, uint16_t* y16, float* rstd, int64_t T, int h,
                  float eps, hipStream_t s);
// The fused projection's fp32 output of tokens t0 .. t0+rows-1 ([rows, 3h];
// with `interleaved`, the q and k pairs of each head interleaved as the
// epilogue of gemm epi 1 takes them): RoPE on q and k in fp32, then bf16 into
// qkv (skipped when NULL) and fp16 into qkv16 ([T, 3h], features in order).
void qkv_finish(const float* qkv32, uint16_t* qkv, uint16_t* qkv16, const float* cos, const float* sin, int64_t t0,
                int64_t rows, int S, int heads, int hd, bool interleaved, hipStream_t s);
// SwiGLU from an fp32 gate/up [rows, 2f] (with `interleaved`, gate and up of
// feature j in columns 2j and 2j + 1): gu = gate | up (bf16 [rows, 2f]), a
// (bf16) and a16 (fp16), [rows, f] (each skipped when NULL).
void swiglu_fwd32(const float* gu32, uint16_t* gu, uint16_t* a, uint16_t* a16, int64_t rows, int f, bool interleaved,
                  hipStream_t s);
// bf16 -> fp16 elementwise (n a multiple of 8).
void bf16_to_f16(const uint16_t* x, uint16_t* y, int64_t n, hipStream_t s);
// bf16 x [rows, cols] -> fp16 y = x^T [cols, rows] (rows, cols multiples of 8),
// with the columns of y optionally permuted: y[k][c] = x[src(c)][k] where
//  perm 0: src(c) = c;
//  perm 1 (RoPE pairs): for c < pa, c = g*pb + 2j + e -> g*pb + j + e*pb/2 (pb = head
//    dim; pairs of a head interleaved), src(c) = c above pa;
//  perm 2 (gate/up pairs): c = 2j + e -> j + e*rows/2.
void bf16_to_f16_t(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols, int perm, int64_t pa, int64_t pb,
                   hipStream_t s);

// SwiGLU: a = silu(gate) * up from gu [T, 2f]; and its backward.
void swiglu_fwd(const uint16_t* gu, uint16_t* a, int64_t T, int f, hipStream_t s);
void swiglu_bwd(const uint16_t* da, const uint16_t* gu, uint16_t* dgu, int64_t T, int f, hipStream_t s);

// Causal flash attention on a fused qkv buffer (scratch: the backward's row
// dot products D = rowsum(dO * O); the forward needs none).
size_t attention_fwd_ws_bytes(int B, int S, int heads, int hd);
size_t attention_bwd_ws_bytes(int B, int S, int heads, int hd);
void attention_fwd(const uint16_t* qkv, uint16_t* o, float* lse, int B, int S, int heads, int hd, void* ws,
                   size_t ws_bytes, hipStream_t s);
// The forward on q, k, v held as fp16 (f16 = true; the probabilities enter
// P V as fp16 too) or bf16, writing bf16 o and, when o16 != NULL, fp16 o16.
void attention_fwd_ex(const uint16_t* qkv, bool f16, uint16_t* o, uint16_t* o16, float* lse, int B, int S, int heads,
                      int hd, hipStream_t s);
void attention_bwd(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout, uint16_t* dqkv,
                   int B, int S, int heads, int hd, void* ws, size_t ws_bytes, hipStream_t s);
// The backward on the forward's fp16 q, k, v (qkv16, as attention_fwd_ex with
// f16 = true read them, so that the recomputed scores equal the forward's):
// dO and dS enter the products as fp16 under per-(batch, head) power-of-two
// scales taken from bounds of their magnitudes; o and dout bf16, dqkv bf16.
size_t attention_bwd16_ws_bytes(int B, int S, int heads, int hd);
void attention_bwd16(const uint16_t* qkv16, const uint16_t* o, const float* lse, const uint16_t* dout,
                     uint16_t* dqkv, int B, int S, int heads, int hd, void* ws, size_t ws_bytes, hipStream_t s);
// The same backward with its scratch in a file-scope device array of
// ATTN_STATIC_SCRATCH_BYTES per device (no workspace argument, no allocation).
constexpr size_t ATTN_STATIC_SCRATCH_BYTES = 64ull << 20;
void attention_bwd_noalloc(const uint16_t* qkv, const uint16_t* o, const float* lse, const uint16_t* dout,
                           uint16_t* dqkv, int B, int S, int heads, int hd, hipStream_t s);

// Cross entropy over a chunk of logits z [rows, V] (fp32) for tokens
// t0..t0+rows-1 of the batch: per-row loss and dz (bf16) = (softmax - onehot)/N.
void cross_entropy(const float* z, const int32_t* tokens, int64_t t0, int64_t rows, int S, int V, float inv_n,
                   float* row_loss, uint16_t* dz, hipStream_t s);
// loss = sum(row_loss[0..n)) * scale, summed in a fixed order.
void sum_scaled(const float* v, int64_t n, float scale, float* out, hipStream_t s);
void f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t s);

}  // namespace mt
