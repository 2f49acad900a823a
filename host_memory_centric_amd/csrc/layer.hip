// The stateless layer template (MegaTrain paper page, appendix A.4: templates
// hold the attention and MLP kernels but no weight pointers; weights are bound
// right before execution) and the head.  Every entry point here only enqueues
// kernels on the caller's stream; all device memory (weight slot, gradient
// slot, activations, saved internals, workspace) is the caller's.
#include <cstdlib>
#include <cstring>

#include "common.h"
#include "kernels.h"

namespace mt {

namespace {

// Bump allocator over a caller buffer (256-byte aligned pieces).
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* b) : base((char*)b) {}
    template <class T>
    T* take(size_t count) {
        T* p = base ? (T*)(base + off) : nullptr;
        off = round_up(off + count * sizeof(T), 256);
        return p;
    }
};

// Token chunk of the per-token phases: the whole batch up to 32768 tokens,
// else chunks of 32768 (a function of the shape only, so every run of a
// configuration computes identically; a multiple of the RMSNorm backward's
// row blocks, so the gain partials of the chunks are those of the whole).
int64_t fwd_chunk(int64_t T) { return std::min<int64_t>(T, 32768); }
// Above one chunk the MLP runs chunked in the backward too: its [T, 2f] and
// [T, f] internals are not kept but recomputed per chunk from the saved
// residual stream, and its weight gradients accumulate in fp32 over the
// chunks in order.
bool mlp_chunked(int64_t T) { return T > fwd_chunk(T); }

// Internals of one layer's forward that its backward reads.
struct Saved {
    uint16_t* n1;    // RMSNorm output before attention [T, h]
    float* rstd1;    // [T]
    uint16_t* qkv;   // fused projection as fp16, q and k rotated [T, 3h]
    uint16_t* o;     // attention output [T, h]
    float* lse;      // [B, heads, S]
    uint16_t* xm;    // residual stream after attention [T, h]
    uint16_t* n2;    // RMSNorm output before the MLP [T, h] (NULL when the MLP is chunked)
    float* rstd2;    // [T]
    uint16_t* gu;    // gate | up [T, 2f] (NULL when the MLP is chunked)
    uint16_t* a;     // silu(gate) * up [T, f] (NULL when the MLP is chunked)
};

Saved carve_saved(Carve& c, const mt_model_cfg* cfg, int64_t B, int64_t S) {
    const int64_t T = B * S, h = cfg->hidden, f = cfg->ffn;
    Saved s;
    s.n1 = c.take<uint16_t>(T * h);
    s.rstd1 = c.take<float>(T);
    s.qkv = c.take<uint16_t>(T * 3 * h);
    s.o = c.take<uint16_t>(T * h);
    s.lse = c.take<float>(B * cfg->heads * S);
    s.xm = c.take<uint16_t>(T * h);
    s.rstd2 = c.take<float>(T);
    s.n2 = s.gu = s.a = nullptr;
    if (!mlp_chunked(T)) {
        s.n2 = c.take<uint16_t>(T * h);
        s.gu = c.take<uint16_t>(T * 2 * f);
        s.a = c.take<uint16_t>(T * f);
    }
    return s;
}

// Forward transients (fp16 GEMM operands and fp32 GEMM outputs); they share
// memory with the backward temporaries below, which are dead during a forward.
struct FwdWs {
    uint16_t* w16;    // the layer's four matrices as fp16, transposed to [in, out]: [h*3h | h*h | h*2f | f*h]
                      // (q/k pairs and gate/up pairs interleaved, see qkv_project and gate_up_project)
    uint16_t* n16;    // RMSNorm output of a token chunk, fp16 [Tc, h]
    float* qkv32;     // fused projection of a token chunk, fp32 [Tc, 3h]
    uint16_t* o16;    // attention output as fp16, whole batch [T, h]
    float* gu32;      // gate | up of a token chunk, fp32 [Tc, 2f]
    uint16_t* a16;    // SwiGLU output of a token chunk, fp16 [Tc, f]
    void* splitk;     // split-K partials (the backward's buffer, idle during a forward), or NULL
    size_t splitk_bytes;
};

FwdWs carve_fwd(Carve& c, const mt_model_cfg* cfg, int64_t T) {
    const int64_t h = cfg->hidden, f = cfg->ffn, Tc = fwd_chunk(T);
    FwdWs w;
    w.w16 = c.take<uint16_t>(4 * h * h + 3 * h * f);
    w.n16 = c.take<uint16_t>(Tc * h);
    w.qkv32 = c.take<float>(Tc * 3 * h);
    w.o16 = c.take<uint16_t>(T * h);
    w.gu32 = c.take<float>(Tc * 2 * f);
    w.a16 = c.take<uint16_t>(Tc * f);
    w.splitk = nullptr;
    w.splitk_bytes = 0;
    return w;
}

struct BwdWs {
    FwdWs fw;         // forward transients, overlapping the backward temporaries after xtmp
    uint16_t* xtmp;   // forward output during recompute [T, h]
    uint16_t* da;     // [T, f]
    uint16_t* dgu;    // [T, 2f]
    float* dn;        // gradient at a RMSNorm output [T, h]
    float* dxm;       // gradient of the mid residual stream [T, h]
    uint16_t* dxm_b;  // its bf16 copy
    uint16_t* dout;   // gradient of the attention output [T, h]
    uint16_t* dqkv;   // [T, 3h]
    void* attn;       // attention scratch (the backward's row statistics, scales, scaled dO)
    size_t attn_bytes;
    float* dg_part;   // RMSNorm gain partials [blocks, h]
    void* splitk;     // split-K partials
    size_t splitk_bytes;
    // chunked MLP only (else NULL): one chunk's recomputed internals, the
    // fp16 gate/up weight transposed to [h, 2f], the fp32 weight-gradient sums
    uint16_t* mc_n2;  // [Tc, h] bf16
    uint16_t* mc_n16; // [Tc, h] fp16
    float* mc_rstd;   // [Tc]
    float* mc_gu32;   // [Tc, 2f]
    uint16_t* mc_gu;  // [Tc, 2f] bf16
    uint16_t* mc_a;   // [Tc, f] bf16
    uint16_t* mc_wgu; // [h, 2f] fp16
    float* mc_dwd;    // [h, f]
    float* mc_dwgu;   // [2f, h]
};

size_t splitk_need(const mt_model_cfg* cfg, int64_t T) {
    const int64_t h = cfg->hidden, f = cfg->ffn, Tm = mlp_chunked(T) ? fwd_chunk(T) : T;
    size_t m = 0;
    m = std::max(m, gemm_splitk_bytes(h, f, Tm));
    m = std::max(m, gemm_splitk_bytes(2 * f, h, Tm));
    m = std::max(m, gemm_splitk_bytes(h, h, T));
    m = std::max(m, gemm_splitk_bytes(3 * h, h, T));
    return m;
}

// Workspace of a layer call that is given a saved-internals buffer; a call
// without one carves the internals right after these pieces.
BwdWs carve_ws(Carve& c, const mt_model_cfg* cfg, int64_t B, int64_t S) {
    const int64_t T = B * S, h = cfg->hidden, f = cfg->ffn;
    size_t fwd_bytes = 0;
    BwdWs w;
    w.xtmp = c.take<uint16_t>(T * h);
    const size_t union_off = c.off;
    {
        Carve cf(c.base ? c.base + union_off : nullptr);
        w.fw = carve_fwd(cf, cfg, T);
        fwd_bytes = cf.off;
    }
    const int64_t Tm = mlp_chunked(T) ? fwd_chunk(T) : T;  // rows of the MLP's backward temporaries
    w.da = c.take<uint16_t>(Tm * f);
    w.dgu = c.take<uint16_t>(Tm * 2 * f);
    w.dn = c.take<float>(T * h);
    w.dxm = c.take<float>(T * h);
    w.dxm_b = c.take<uint16_t>(T * h);
    w.dout = c.take<uint16_t>(T * h);
    w.dqkv = c.take<uint16_t>(T * 3 * h);
    w.attn_bytes = std::max(attention_fwd_ws_bytes((int)B, (int)S, cfg->heads, cfg->head_dim),
                            attention_bwd16_ws_bytes((int)B, (int)S, cfg->heads, cfg->head_dim));
    w.attn = c.take<char>(w.attn_bytes);
    w.dg_part = c.take<float>(rmsnorm_bwd_blocks(T) * h);
    w.splitk_bytes = splitk_need(cfg, T);
    w.splitk = c.take<char>(w.splitk_bytes);
    w.fw.splitk = w.splitk;  // outside the forward's transients
    w.fw.splitk_bytes = w.splitk_bytes;
    w.mc_n2 = w.mc_n16 = w.mc_gu = w.mc_a = w.mc_wgu = nullptr;
    w.mc_rstd = w.mc_gu32 = w.mc_dwd = w.mc_dwgu = nullptr;
    if (mlp_chunked(T)) {
        w.mc_n2 = c.take<uint16_t>(Tm * h);
        w.mc_n16 = c.take<uint16_t>(Tm * h);
        w.mc_rstd = c.take<float>(Tm);
        w.mc_gu32 = c.take<float>(Tm * 2 * f);
        w.mc_gu = c.take<uint16_t>(Tm * 2 * f);
        w.mc_a = c.take<uint16_t>(Tm * f);
        w.mc_wgu = c.take<uint16_t>(h * 2 * f);
        w.mc_dwd = c.take<float>(h * f);
        w.mc_dwgu = c.take<float>(2 * f * h);
    }
    if (c.off < union_off + fwd_bytes) c.off = union_off + fwd_bytes;  // the union's larger part
    return w;
}

void check_act_shape(const mt_model_cfg* cfg, int32_t B, int32_t S) {
    check_cfg(cfg);
    if (B < 1 || S < 1) MT_FAIL(MT_E_SHAPE, "batch and seq must be positive");
    if ((int64_t)B * S % 8) MT_FAIL(MT_E_SHAPE, "batch*seq must be a multiple of 8");
    if (cfg->head_dim != 64 && cfg->head_dim != 128) MT_FAIL(MT_E_SHAPE, "head_dim must be 64 or 128");
}

template <class T>
void need(const T* p, const char* what) {
    if (!p) MT_FAIL(MT_E_ARG, "%s is NULL", what);
    if ((uintptr_t)p & 15) MT_FAIL(MT_E_ALIGN, "%s must be 16-byte aligned", what);
}

GemmDesc gd(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, bool ak, const void* Bm, int64_t ldb,
            bool bk, int64_t ldc) {
    GemmDesc d;
    d.M = M;
    d.N = N;
    d.K = K;
    d.A = A;
    d.lda = lda;
    d.a_kmajor = ak;
    d.B = Bm;
    d.ldb = ldb;
    d.b_kmajor = bk;
    d.ldc = ldc;
    return d;
}

// QKV projection of tokens t0 .. t0 + rows - 1 from their fp16 RMSNorm output:
// q and k rotated, then q, k, v as fp16 into qkv16 ([T, 3h]).  wqkv16 is the
// fp16 weight transposed to [h, 3h] with the (p, p + hd/2) feature pairs of
// every q and k head interleaved, so that the GEMM's epilogue rotates each pair
// inside one lane; shapes that the fused epilogue does not take go through
// fp32 (qkv32, [rows, 3h]) and a separate kernel with the same arithmetic.
void qkv_project(const mt_model_cfg* cfg, const uint16_t* n16, const uint16_t* wqkv16, int64_t rows, int64_t t0, int S,
                 const float* cs, const float* sn, uint16_t* qkv16, float* qkv32, hipStream_t s) {
    const int64_t h = cfg->hidden;
    GemmDesc d = gd(rows, 3 * h, h, n16, h, true, wqkv16, 3 * h, false, 3 * h);
    d.f16 = true;
    if (gemm_epi_ok(rows, 3 * h, h, h, 3 * h)) {
        d.epi = 1;
        d.Cb = qkv16 + t0 * 3 * h;
        d.rope_cos = cs;
        d.rope_sin = sn;
        d.rope_S = S;
        d.rope_hd = cfg->head_dim;
        d.rope_t0 = t0;
        d.rope_cols = 2 * h;
        gemm(d, s);
    } else {
        d.Cf = qkv32;
        gemm(d, s);
        qkv_finish(qkv32, nullptr, qkv16, cs, sn, t0, rows, S, cfg->heads, cfg->head_dim, true, s);
    }
}

// Gate/up projection and SwiGLU of rows tokens from their fp16 RMSNorm output:
// gu = gate | up (bf16 [rows, 2f]), a = silu(gate) * up (bf16) and a16 (fp16)
// [rows, f], each skipped when NULL.  wgu16 is the fp16 weight transposed to
// [h, 2f] with gate and up of every feature interleaved; shapes that the fused
// epilogue does not take go through fp32 (gu32, [rows, 2f]).
void gate_up_project(const mt_model_cfg* cfg, const uint16_t* n16, const uint16_t* wgu16, int64_t rows, uint16_t* gu,
                     uint16_t* a, uint16_t* a16, float* gu32, hipStream_t s) {
    const int64_t h = cfg->hidden, f = cfg->ffn;
    GemmDesc d = gd(rows, 2 * f, h, n16, h, true, wgu16, 2 * f, false, 2 * f);
    d.f16 = true;
    if (gemm_epi_ok(rows, 2 * f, h, h, 2 * f)) {
        d.epi = 2;
        d.Cb = gu;
        d.Ca = a;
        d.Ca16 = a16;
        gemm(d, s);
    } else {
        d.Cf = gu32;
        gemm(d, s);
        swiglu_fwd32(gu32, gu, a, a16, rows, (int)f, true, s);
    }
}

// Forward of one layer: x -> y, internals into sv.  The GEMM operands of the
// forward are fp16 (the weights converted exactly and transposed to [in, out],
// the activations rounded once from fp32: three more significand bits than
// bf16).  The backward reads q, k, v as the same fp16 values, so that its
// recomputed attention scores are the forward's; its other internals are
// stored bf16, from the same fp32 values.  Per-token work runs over token
// chunks (fwd_chunk), attention over the whole batch.
void layer_forward(const mt_layer_view* v, const mt_model_cfg* cfg, int B, int S, const uint16_t* x, uint16_t* y,
                   const float* cs, const float* sn, const Saved& sv, const FwdWs& fw, hipStream_t s) {
    const int64_t T = (int64_t)B * S, h = cfg->hidden, f = cfg->ffn, Tc = fwd_chunk(T);
    const uint16_t* g_attn = (const uint16_t*)v->w[0];
    const uint16_t* g_mlp = (const uint16_t*)v->w[3];
    uint16_t* wqkv = fw.w16;
    uint16_t* wo = wqkv + 3 * h * h;
    uint16_t* wgu = wo + h * h;
    uint16_t* wd = wgu + 2 * f * h;
    bf16_to_f16_t((const uint16_t*)v->w[1], wqkv, 3 * h, h, 1, 2 * h, cfg->head_dim, s);
    bf16_to_f16_t((const uint16_t*)v->w[2], wo, h, h, 0, 0, 0, s);
    bf16_to_f16_t((const uint16_t*)v->w[4], wgu, 2 * f, h, 2, 0, 0, s);
    bf16_to_f16_t((const uint16_t*)v->w[5], wd, h, f, 0, 0, 0, s);

    // attention RMSNorm, QKV projection, RoPE: per token chunk
    for (int64_t t0 = 0; t0 < T; t0 += Tc) {
        const int64_t rows = std::min(Tc, T - t0);
        rmsnorm_fwd2(x + t0 * h, g_attn, sv.n1 + t0 * h, fw.n16, sv.rstd1 + t0, rows, (int)h, cfg->eps, s);
        qkv_project(cfg, fw.n16, wqkv, rows, t0, S, cs, sn, sv.qkv, fw.qkv32, s);
    }
    attention_fwd_ex(sv.qkv, true, sv.o, fw.o16, sv.lse, B, S, cfg->heads, cfg->head_dim, s);
    // output projection + residual, MLP RMSNorm, gate/up, SwiGLU, down + residual: per token chunk
    for (int64_t t0 = 0; t0 < T; t0 += Tc) {
        const int64_t rows = std::min(Tc, T - t0);
        GemmDesc d = gd(rows, h, h, fw.o16 + t0 * h, h, true, wo, h, false, h);
        d.f16 = true;
        d.R = x + t0 * h;
        d.Cb = sv.xm + t0 * h;
        gemm(d, s);
        rmsnorm_fwd2(sv.xm + t0 * h, g_mlp, sv.n2 ? sv.n2 + t0 * h : nullptr, fw.n16, sv.rstd2 + t0, rows, (int)h,
                     cfg->eps, s);
        gate_up_project(cfg, fw.n16, wgu, rows, sv.gu ? sv.gu + t0 * 2 * f : nullptr, sv.a ? sv.a + t0 * f : nullptr,
                        fw.a16, fw.gu32, s);
        d = gd(rows, h, f, fw.a16, f, true, wd, h, false, h);
        d.f16 = true;
        d.R = sv.xm + t0 * h;
        d.Cb = y + t0 * h;
        d.ws = fw.splitk;  // (a ragged last round of tiles may run with K split)
        d.ws_bytes = fw.splitk_bytes;
        gemm(d, s);
    }
}

void layer_backward(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_act* io, const Saved& sv, BwdWs& w,
                    hipStream_t s) {
    const int B = io->batch, S = io->seq;
    const int64_t T = (int64_t)B * S, h = cfg->hidden, f = cfg->ffn;
    const uint16_t* wqkv = (const uint16_t*)v->w[1];
    const uint16_t* wo = (const uint16_t*)v->w[2];
    const uint16_t* wgu = (const uint16_t*)v->w[4];
    const uint16_t* wd = (const uint16_t*)v->w[5];
    const uint16_t* dyb = (const uint16_t*)io->dy_bf16;

    const uint16_t* g_mlp = (const uint16_t*)v->w[3];
    GemmDesc d;
    if (!mlp_chunked(T)) {
        // down projection
        d = gd(h, f, T, dyb, h, false, sv.a, f, false, f);
        d.Cb = v->g[5];
        d.ws = w.splitk;
        d.ws_bytes = w.splitk_bytes;
        gemm(d, s);
        d = gd(T, f, h, dyb, h, true, wd, f, false, f);
        d.Cb = w.da;
        gemm(d, s);
        swiglu_bwd(w.da, sv.gu, w.dgu, T, (int)f, s);
        // gate/up projection
        d = gd(2 * f, h, T, w.dgu, 2 * f, false, sv.n2, h, false, h);
        d.Cb = v->g[4];
        d.ws = w.splitk;
        d.ws_bytes = w.splitk_bytes;
        gemm(d, s);
        d = gd(T, h, 2 * f, w.dgu, 2 * f, true, wgu, h, false, h);
        d.Cf = w.dn;
        d.ws = w.splitk;
        d.ws_bytes = w.splitk_bytes;
        gemm(d, s);
        // MLP RMSNorm (+ residual)
        rmsnorm_bwd(w.dn, sv.xm, sv.rstd2, g_mlp, io->dy, w.dxm, w.dxm_b, w.dg_part, T, (int)h, s);
    } else {
        // Per token chunk: recompute the chunk's MLP input (RMSNorm), gate/up
        // (the forward's fp16 GEMM) and SwiGLU exactly as the forward computed
        // them, then its backward; the weight gradients are summed over the
        // chunks in order in fp32 and rounded once.
        const int64_t Tc = fwd_chunk(T);
        bf16_to_f16_t(wgu, w.mc_wgu, 2 * f, h, 2, 0, 0, s);
        for (int64_t t0 = 0; t0 < T; t0 += Tc) {
            const int64_t rows = std::min(Tc, T - t0);
            const int acc = t0 > 0;
            rmsnorm_fwd2(sv.xm + t0 * h, g_mlp, w.mc_n2, w.mc_n16, w.mc_rstd, rows, (int)h, cfg->eps, s);
            gate_up_project(cfg, w.mc_n16, w.mc_wgu, rows, w.mc_gu, w.mc_a, nullptr, w.mc_gu32, s);
            // down projection
            d = gd(h, f, rows, dyb + t0 * h, h, false, w.mc_a, f, false, f);
            d.Cf = w.mc_dwd;
            d.accumulate = acc;
            d.ws = w.splitk;
            d.ws_bytes = w.splitk_bytes;
            gemm(d, s);
            d = gd(rows, f, h, dyb + t0 * h, h, true, wd, f, false, f);
            d.Cb = w.da;
            gemm(d, s);
            swiglu_bwd(w.da, w.mc_gu, w.dgu, rows, (int)f, s);
            // gate/up projection
            d = gd(2 * f, h, rows, w.dgu, 2 * f, false, w.mc_n2, h, false, h);
            d.Cf = w.mc_dwgu;
            d.accumulate = acc;
            d.ws = w.splitk;
            d.ws_bytes = w.splitk_bytes;
            gemm(d, s);
            d = gd(rows, h, 2 * f, w.dgu, 2 * f, true, wgu, h, false, h);
            d.Cf = w.dn + t0 * h;
            d.ws = w.splitk;
            d.ws_bytes = w.splitk_bytes;
            gemm(d, s);
            // MLP RMSNorm (+ residual); the chunk's gain partials are row
            // blocks t0 / 16 .. of the whole
            rmsnorm_bwd(w.dn + t0 * h, sv.xm + t0 * h, sv.rstd2 + t0, g_mlp, io->dy + t0 * h, w.dxm + t0 * h,
                        w.dxm_b + t0 * h, w.dg_part + rmsnorm_bwd_blocks(t0) * h, rows, (int)h, s);
        }
        f32_to_bf16(w.mc_dwd, (uint16_t*)v->g[5], h * f, s);
        f32_to_bf16(w.mc_dwgu, (uint16_t*)v->g[4], 2 * f * h, s);
    }
    colsum_to_bf16(w.dg_part, rmsnorm_bwd_blocks(T), (int)h, (uint16_t*)v->g[3], s);
    // output projection
    d = gd(h, h, T, w.dxm_b, h, false, sv.o, h, false, h);
    d.Cb = v->g[2];
    d.ws = w.splitk;
    d.ws_bytes = w.splitk_bytes;
    gemm(d, s);
    d = gd(T, h, h, w.dxm_b, h, true, wo, h, false, h);
    d.Cb = w.dout;
    gemm(d, s);
    // attention and RoPE
    attention_bwd16(sv.qkv, sv.o, sv.lse, w.dout, w.dqkv, B, S, cfg->heads, cfg->head_dim, w.attn, w.attn_bytes, s);
    rope_apply(w.dqkv, io->rope_cos, io->rope_sin, T, S, cfg->heads, cfg->head_dim, true, s);
    // QKV projection
    d = gd(3 * h, h, T, w.dqkv, 3 * h, false, sv.n1, h, false, h);
    d.Cb = v->g[1];
    d.ws = w.splitk;
    d.ws_bytes = w.splitk_bytes;
    gemm(d, s);
    d = gd(T, h, 3 * h, w.dqkv, 3 * h, true, wqkv, h, false, h);
    d.Cf = w.dn;
    d.ws = w.splitk;
    d.ws_bytes = w.splitk_bytes;
    gemm(d, s);
    // attention RMSNorm (+ residual)
    rmsnorm_bwd(w.dn, (const uint16_t*)io->x_in, sv.rstd1, (const uint16_t*)v->w[0], w.dxm, io->dx,
                (uint16_t*)io->dx_bf16, w.dg_part, T, (int)h, s);
    colsum_to_bf16(w.dg_part, rmsnorm_bwd_blocks(T), (int)h, (uint16_t*)v->g[0], s);
}

struct HeadWs {
    uint16_t* xf;
    float* rstd;
    float* z;
    uint16_t* dz;
    float* dxf;
    float* row_loss;
    float* dwh;
    float* dg_part;
    void* splitk;
    size_t splitk_bytes;
};

constexpr int64_t HEAD_CHUNK = 8192;

HeadWs carve_head(Carve& c, const mt_model_cfg* cfg, int64_t B, int64_t S) {
    const int64_t T = B * S, h = cfg->hidden, V = cfg->vocab;
    const int64_t Tc = std::min(T, HEAD_CHUNK);
    HeadWs w;
    w.xf = c.take<uint16_t>(Tc * h);
    w.rstd = c.take<float>(Tc);
    w.z = c.take<float>(Tc * V);
    w.dz = c.take<uint16_t>(Tc * V);
    w.dxf = c.take<float>(Tc * h);
    w.row_loss = c.take<float>(T);
    w.dwh = c.take<float>(V * h);
    w.dg_part = c.take<float>(((T + HEAD_CHUNK - 1) / HEAD_CHUNK) * rmsnorm_bwd_blocks(Tc) * h);
    w.splitk_bytes = gemm_splitk_bytes(V, h, Tc);
    w.splitk = c.take<char>(w.splitk_bytes);
    return w;
}

hipStream_t as_stream(void* s) { return (hipStream_t)s; }

// Workspace pieces and the internals of a layer call: from io->saved when
// given, else carved in the workspace after the backward temporaries.
void carve_call(const mt_model_cfg* cfg, const mt_act* io, BwdWs& w, Saved& sv) {
    size_t wb, sb;
    mt_layer_workspace_bytes(cfg, io->batch, io->seq, &wb);
    mt_layer_saved_bytes(cfg, io->batch, io->seq, &sb);
    const size_t need_ws = io->saved ? wb : wb + sb;
    if (io->workspace_bytes < need_ws)
        MT_FAIL(MT_E_ARG, "workspace holds %zu bytes, needs %zu%s", io->workspace_bytes, need_ws,
                io->saved ? "" : " (no saved buffer: workspace + saved bytes)");
    need(io->workspace, "workspace");
    Carve c(io->workspace);
    w = carve_ws(c, cfg, io->batch, io->seq);
    if (io->saved) {
        if (io->saved_bytes < sb) MT_FAIL(MT_E_ARG, "saved buffer holds %zu bytes, needs %zu", io->saved_bytes, sb);
        need(io->saved, "saved");
        Carve cs(io->saved);
        sv = carve_saved(cs, cfg, io->batch, io->seq);
    } else {
        sv = carve_saved(c, cfg, io->batch, io->seq);
    }
}

}  // namespace

}  // namespace mt

using namespace mt;

extern "C" {

int mt_bind(const mt_model_cfg* cfg, int unit, const void* dev_w_slot, void* dev_g_slot, mt_layer_view* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr && dev_w_slot != nullptr, "NULL argument");
        if (((uintptr_t)dev_w_slot | (uintptr_t)dev_g_slot) & 255)
            MT_FAIL(MT_E_ALIGN, "device slots must be 256-byte aligned");
        // the head's device slot has the untied layout even for tied weights
        mt_model_cfg c = *cfg;
        if (unit == MT_UNIT_HEAD) c.tied = 0;
        const mt_unit_layout L = layout_of(&c, unit);
        memset(out, 0, sizeof(*out));
        for (int j = 0; j < L.n_tensors; ++j) {
            out->w[j] = (const char*)dev_w_slot + L.tensor_off[j];
            out->g[j] = dev_g_slot ? (char*)dev_g_slot + L.tensor_off[j] : nullptr;
        }
    });
}

int mt_layer_saved_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        check_act_shape(cfg, batch, seq);
        Carve c(nullptr);
        carve_saved(c, cfg, batch, seq);
        *out = c.off;
    });
}

int mt_layer_workspace_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        check_act_shape(cfg, batch, seq);
        Carve c(nullptr);
        carve_ws(c, cfg, batch, seq);
        *out = c.off;
    });
}

int mt_layer_fwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_act* io, void* stream) {
    return guard([&] {
        MT_CHECK_ARG(v && io, "NULL argument");
        check_act_shape(cfg, io->batch, io->seq);
        need(io->x_in, "x_in");
        need(io->x_out, "x_out");
        need(io->rope_cos, "rope_cos");
        need(io->rope_sin, "rope_sin");
        for (int j = 0; j < 6; ++j) need(v->w[j], "weight view");
        BwdWs w;
        Saved sv;
        carve_call(cfg, io, w, sv);
        layer_forward(v, cfg, io->batch, io->seq, (const uint16_t*)io->x_in, (uint16_t*)io->x_out, io->rope_cos,
                      io->rope_sin, sv, w.fw, as_stream(stream));
    });
}

int mt_layer_recompute_bwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_act* io, void* stream) {
    return guard([&] {
        MT_CHECK_ARG(v && io, "NULL argument");
        check_act_shape(cfg, io->batch, io->seq);
        need(io->x_in, "x_in");
        need(io->dy, "dy");
        need(io->dy_bf16, "dy_bf16");
        need(io->dx, "dx");
        need(io->dx_bf16, "dx_bf16");
        need(io->rope_cos, "rope_cos");
        need(io->rope_sin, "rope_sin");
        for (int j = 0; j < 6; ++j) {
            need(v->w[j], "weight view");
            need(v->g[j], "gradient view");
        }
        BwdWs w;
        Saved sv;
        carve_call(cfg, io, w, sv);
        const hipStream_t s = as_stream(stream);
        if (!io->saved) {
            layer_forward(v, cfg, io->batch, io->seq, (const uint16_t*)io->x_in, w.xtmp, io->rope_cos, io->rope_sin, sv,
                          w.fw, s);
        }
        layer_backward(v, cfg, io, sv, w, s);
    });
}

int mt_head_workspace_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        check_act_shape(cfg, batch, seq);
        Carve c(nullptr);
        carve_head(c, cfg, batch, seq);
        *out = c.off;
    });
}

int mt_head_fwd_bwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_head_io* io, void* stream) {
    return guard([&] {
        MT_CHECK_ARG(v && io, "NULL argument");
        check_act_shape(cfg, io->batch, io->seq);
        if (io->seq < 2) MT_FAIL(MT_E_SHAPE, "seq must be >= 2 for next-token loss");
        need(io->x, "x");
        need(io->dx, "dx");
        need(io->dx_bf16, "dx_bf16");
        need(io->loss, "loss");
        MT_CHECK_ARG(io->tokens != nullptr, "tokens is NULL");
        for (int j = 0; j < 2; ++j) {
            need(v->w[j], "head weight view");
            need(v->g[j], "head gradient view");
        }
        size_t nb;
        mt_head_workspace_bytes(cfg, io->batch, io->seq, &nb);
        if (io->workspace_bytes < nb) MT_FAIL(MT_E_ARG, "workspace holds %zu bytes, needs %zu", io->workspace_bytes, nb);
        need(io->workspace, "workspace");
        Carve c(io->workspace);
        HeadWs w = carve_head(c, cfg, io->batch, io->seq);
        const hipStream_t s = as_stream(stream);
        const int64_t T = (int64_t)io->batch * io->seq, h = cfg->hidden, V = cfg->vocab;
        const float inv_n = 1.0f / (float)((int64_t)io->batch * (io->seq - 1));
        const uint16_t* gf = (const uint16_t*)v->w[0];
        const uint16_t* wh = (const uint16_t*)v->w[1];
        const uint16_t* x = (const uint16_t*)io->x;
        const int64_t Tc = std::min(T, HEAD_CHUNK);
        const int64_t bpc = rmsnorm_bwd_blocks(Tc);
        int64_t nblk = 0;
        for (int64_t t0 = 0, ci = 0; t0 < T; t0 += Tc, ++ci) {
            const int64_t rows = std::min(Tc, T - t0);
            rmsnorm_fwd2(x + t0 * h, gf, w.xf, nullptr, w.rstd, rows, (int)h, cfg->eps, s);
            GemmDesc d = gd(rows, V, h, w.xf, h, true, wh, h, true, V);
            d.Cf = w.z;
            gemm(d, s);
            cross_entropy(w.z, io->tokens, t0, rows, io->seq, (int)V, inv_n, w.row_loss + t0, w.dz, s);
            d = gd(V, h, rows, w.dz, V, false, w.xf, h, false, h);
            d.Cf = w.dwh;
            d.accumulate = ci > 0;
            d.ws = w.splitk;
            d.ws_bytes = w.splitk_bytes;
            gemm(d, s);
            d = gd(rows, h, V, w.dz, V, true, wh, h, false, h);
            d.Cf = w.dxf;
            gemm(d, s);
            rmsnorm_bwd(w.dxf, x + t0 * h, w.rstd, gf, nullptr, io->dx + t0 * h, (uint16_t*)io->dx_bf16 + t0 * h,
                        w.dg_part + ci * bpc * h, rows, (int)h, s);
            nblk = ci * bpc + rmsnorm_bwd_blocks(rows);
        }
        colsum_to_bf16(w.dg_part, nblk, (int)h, (uint16_t*)v->g[0], s);
        f32_to_bf16(w.dwh, (uint16_t*)v->g[1], V * h, s);
        sum_scaled(w.row_loss, T, inv_n, io->loss, s);
    });
}

int mt_op_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int a_kmajor, const void* B, int64_t ldb,
               int b_kmajor, float* c_f32, void* c_bf16, const void* resid_bf16, int64_t ldc, int accumulate, void* ws,
               size_t ws_bytes, void* stream) {
    return guard([&] {
        GemmDesc d = gd(M, N, K, A, lda, a_kmajor != 0, B, ldb, b_kmajor != 0, ldc);
        d.Cf = c_f32;
        d.Cb = c_bf16;
        d.R = resid_bf16;
        d.accumulate = accumulate;
        d.ws = ws;
        d.ws_bytes = ws_bytes;
        gemm(d, as_stream(stream));
    });
}

int mt_op_attention_fwd(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv, void* o, float* lse,
                        void* ws, size_t ws_bytes, void* stream) {
    return guard([&] {
        need(qkv, "qkv");
        need(o, "o");
        need(ws, "ws");
        MT_CHECK_ARG(lse != nullptr, "lse is NULL");
        attention_fwd((const uint16_t*)qkv, (uint16_t*)o, lse, batch, seq, heads, hd, ws, ws_bytes, as_stream(stream));
    });
}

int mt_op_attention_bwd(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv, const void* o,
                        const float* lse, const void* d_o, void* dqkv, void* ws, size_t ws_bytes, void* stream) {
    return guard([&] {
        need(qkv, "qkv");
        need(o, "o");
        need(d_o, "d_o");
        need(dqkv, "dqkv");
        need(ws, "ws");
        MT_CHECK_ARG(lse != nullptr, "lse is NULL");
        attention_bwd((const uint16_t*)qkv, (const uint16_t*)o, lse, (const uint16_t*)d_o, (uint16_t*)dqkv, batch, seq,
                      heads, hd, ws, ws_bytes, as_stream(stream));
    });
}

int mt_op_attention_bwd_noalloc(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv,
                                const void* o, const float* lse, const void* d_o, void* dqkv, void* stream) {
    return guard([&] {
        need(qkv, "qkv");
        need(o, "o");
        need(d_o, "d_o");
        need(dqkv, "dqkv");
        MT_CHECK_ARG(lse != nullptr, "lse is NULL");
        attention_bwd_noalloc((const uint16_t*)qkv, (const uint16_t*)o, lse, (const uint16_t*)d_o, (uint16_t*)dqkv,
                              batch, seq, heads, hd, as_stream(stream));
    });
}

int mt_op_attention_ws_bytes(int32_t batch, int32_t seq, int32_t heads, int32_t hd, size_t* out) {
    return guard([&] {
        MT_CHECK_ARG(out != nullptr, "out is NULL");
        *out = std::max(attention_fwd_ws_bytes(batch, seq, heads, hd), attention_bwd_ws_bytes(batch, seq, heads, hd));
    });
}

}  // extern "C"
