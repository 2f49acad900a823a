/*
 * mt.h -- C ABI of the layer-streamed trainer (host-memory-centric training,
 * MI355X / gfx950).
 *
 * The method (MegaTrain paper page, section 3 "MegaTrain System" and appendix
 * A): host memory is the authoritative store of every layer's weights,
 * gradients and Adam moments; each layer streams through a bounded device
 * staging area, runs on a stateless layer template, is block-checkpointed and
 * recomputed in the backward pass; its gradients are offloaded and a host
 * Adam updates it.
 *
 * Conventions for every entry point
 *  - returns int: MT_OK (0) or a negative MT_E_* code; mt_last_error() gives a
 *    thread-local message for the last failure of the calling thread;
 *  - no C++ exception crosses this boundary;
 *  - device entry points validate arguments, enqueue work on the given HIP
 *    stream and return; faults surface at the caller's next synchronisation
 *    (set MT_SYNC_CHECK=1 in the environment to synchronise after every call);
 *  - the library never allocates or frees device memory on the training path
 *    and never creates streams or events: the caller owns device buffers,
 *    workspaces, streams and events.  The host store, pinned buffers from
 *    mt_pinned_alloc and the host worker threads belong to the library;
 *  - all bf16 data is stored as raw 16-bit patterns (uint16), row-major;
 *    floating-point roundings to bf16 are round-to-nearest-even.
 *
 * Environment switches (read once per process; results never depend on them):
 *  - MT_SYNC_CHECK=1: synchronise the stream after every device call;
 *  - MT_GEMM_IMPL=pipe: large GEMMs on the 4-wave pipelined kernel instead of
 *    the 8-wave ping-pong kernel (same bits);
 *  - MT_ATTN_FWD=pipe: attention forward on the 4-wave pipelined kernel
 *    instead of the 8-wave ping-pong kernel (same bits);
 *  - MT_NO_AVX512=1: the host Adam and accumulation on their scalar path
 *    (same bits).
 */
#ifndef MT_H
#define MT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MT_OK = 0,
    MT_E_ARG = -1,    /* bad pointer, size or enum value */
    MT_E_SHAPE = -2,  /* shape the kernels do not support (see each call) */
    MT_E_ALIGN = -3,  /* pointer not aligned as documented */
    MT_E_NOMEM = -4,  /* host allocation failed */
    MT_E_HIP = -5,    /* a HIP runtime call failed (message holds its error) */
    MT_E_STATE = -6,  /* call out of order */
    MT_E_IO = -7      /* file I/O failed (message holds the system error) */
};

/* Units of the host store: layers are 0..layers-1. */
enum { MT_UNIT_EMBED = -1, MT_UNIT_HEAD = -2 };

#define MT_BLOCK_ALIGN 4096 /* region alignment inside a block (4 KB pages) */
#define MT_TENSOR_ALIGN 256 /* tensor alignment inside a W/G region */

/* Model shape.  Llama-style decoder: per layer RMSNorm gain [h], fused QKV
 * weight [3h, h], output projection [h, h], RMSNorm gain [h], fused gate/up
 * weight [2f, h] (gate rows first), down projection [h, f]; embedding [V, h];
 * final RMSNorm gain [h] and LM head [V, h], which with `tied` is the
 * embedding matrix itself (paper page, appendix A.1: tied embedding and
 * head share one physical store).  Weights are [out, in]. */
typedef struct mt_model_cfg {
    int32_t layers, hidden, heads, head_dim, ffn, vocab;
    float eps;       /* RMSNorm epsilon (inside the square root) */
    float rope_base; /* RoPE base (rotate-half pairs (i, i + hd/2)) */
    int32_t tied;    /* 1: the LM head is the embedding matrix (weight tying), 0: untied */
} mt_model_cfg;

/* Layout of one unit's block.  Layer-contiguous tiling (paper page, appendix
 * A.1; hyper.ai summary, method): one block per unit holding, in order, the
 * bf16 weight region W, the bf16 gradient region G, and the fp32 Adam moment
 * regions M and V, each starting on a 4 KB boundary.  Tensors sit in W (and
 * at the same offsets in G and in the device staging slot) at 256-byte
 * aligned offsets; M and V use the same element indexing as W (4 bytes per
 * element).  Padding elements are zero and stay zero under Adam.
 * Two optional fp32 regions follow, with the same indexing, when the store
 * is created with the matching flag (0 bytes otherwise): P, a master copy of
 * the weights (MT_STORE_MASTER_FP32), and A, the gradient accumulator of
 * micro-batches (MT_STORE_GRAD_ACCUM). */
typedef struct mt_unit_layout {
    int32_t n_tensors;        /* 6 per layer; 1 for the embedding; 2 for the head (1 when tied) */
    int32_t pad_;
    uint64_t tensor_off[6];   /* byte offset of tensor j inside W */
    uint64_t tensor_numel[6]; /* element count of tensor j */
    uint64_t w_bytes;         /* bytes of W incl. inter-tensor padding (== G's) */
    uint64_t region_off[6];   /* W, G, M, V, P, A byte offsets inside the block */
    uint64_t region_bytes[6]; /* their 4 KB-padded sizes (P, A: 0 unless enabled) */
    uint64_t block_bytes;     /* total block size */
    uint64_t params;          /* real parameter count of the unit */
} mt_unit_layout;

/* Optional store regions (flags of mt_store_create_ex / mt_unit_layout_get_ex). */
/* (paper page, section 2: persistent state needs at least 12 bytes per
 * parameter -- bf16 weights and gradients, fp32 moments; the master copy
 * makes it 16 and keeps updates smaller than half a bf16 ulp of a weight.) */
enum {
    MT_STORE_MASTER_FP32 = 1, /* fp32 master weights P: Adam updates P, W = bf16(P) */
    MT_STORE_GRAD_ACCUM = 2,  /* fp32 accumulator A for gradient accumulation over micro-batches */
    /* Placement only (the layout is unchanged): each unit's W and G regions
     * are page-locked (hipHostMalloc), so weight loads can be copied to the
     * device straight from W and gradients straight into G, with no staging
     * copy through host memory; M, V, P and A stay pageable.  Needs a HIP
     * device; page-locked memory is a limited resource (MT_E_NOMEM when the
     * system refuses).  A layer of the method's format moves through host
     * DRAM once per transfer instead of three times (paper page, appendix
     * A.1 stages every load through pinned buffers). */
    MT_STORE_PINNED_DMA = 4
};

/* Pure function: the layout of `unit` in a store with the given flags
 * (mt_unit_layout_get: flags 0).  MT_E_SHAPE if hidden != heads * head_dim,
 * or a dimension is not a positive multiple of 8; MT_E_ARG for unknown flags. */
int mt_unit_layout_get(const mt_model_cfg* cfg, int unit, mt_unit_layout* out);
int mt_unit_layout_get_ex(const mt_model_cfg* cfg, uint32_t flags, int unit, mt_unit_layout* out);

/* ------------------------------------------------------------------------ */
/* Host store (the authoritative copy of all training state).               */
/* ------------------------------------------------------------------------ */
typedef struct mt_store mt_store;

/* Allocates one page-aligned, zero-filled block per unit (pageable memory;
 * 2 MB huge pages are requested).  Owned by the library; free with
 * mt_store_destroy.  mt_store_create_ex adds the optional regions of `flags`
 * (MT_STORE_*; mt_store_create: none); with MT_STORE_PINNED_DMA each block
 * is held as two allocations, [W | G] page-locked and [M | V | P | A]
 * pageable, and regions are addressed with mt_store_region. */
int mt_store_create(const mt_model_cfg* cfg, mt_store** out);
int mt_store_create_ex(const mt_model_cfg* cfg, uint32_t flags, mt_store** out);
void mt_store_destroy(mt_store* st);
/* Base address of a unit's block (layout as mt_unit_layout_get); MT_E_STATE
 * for a MT_STORE_PINNED_DMA store, whose blocks are not contiguous. */
int mt_store_block(mt_store* st, int unit, void** block);
/* Address of region `region` (0..5: W, G, M, V, P, A) of a unit, for every
 * kind of store; MT_E_STATE if the store does not hold that region. */
int mt_store_region(mt_store* st, int unit, int region, void** ptr);
/* Total bytes of all blocks. */
int mt_store_bytes(const mt_store* st, uint64_t* out);
/* Fills every W region from the seeded SplitMix64 generator: matrices
 * bf16(fp32(std * N(0,1))) via Box-Muller, RMSNorm gains = 1.  Streams:
 * embedding 1, final gain 2, LM head 3, layer l tensor j 16 + 8 l + j.
 * Multithreaded.  Zeroes G, M and V. */
int mt_store_fill_normal(mt_store* st, uint32_t seed, double std);
/* Master-weight stores: P = fp32(W) for every unit (exact), e.g. after the
 * caller wrote W through mt_store_region (mt_store_fill_normal does this
 * itself).  MT_E_STATE without MT_STORE_MASTER_FP32. */
int mt_store_sync_master(mt_store* st);

/* Checkpoint and resume of the host store (the store is the authoritative
 * copy of all training state -- paper page, section 3, execution workflow --
 * so a step counter and the blocks are a complete checkpoint; the pages list
 * an SSD tier below host memory as future work, section 6).  mt_store_save
 * writes a header (format tag, model config, store flags, t, block sizes),
 * every unit's whole block (embedding, head, layers 0..L-1: W, G, M, V and
 * the optional regions) and the per-unit micro-batch accumulation counts,
 * in parallel, then syncs the file.  mt_store_load reads such a file into a
 * store created with the same config and region flags (MT_E_ARG otherwise;
 * MT_STORE_PINNED_DMA is placement, not format, and may differ) and
 * returns t; a run resumed from it continues bit-identically.  MT_E_IO on
 * I/O errors.  Neither may overlap any other call on the store. */
int mt_store_save(const mt_store* st, const char* path, int64_t t);
int mt_store_load(mt_store* st, const char* path, int64_t* t_out);

/* Number of host worker threads used by pack, Adam, fill and embedding
 * (default: the process's CPU affinity count). */
int mt_set_threads(int n);
/* Threads of the optimizer calls alone (mt_step, mt_grad_accumulate); 0
 * (default) = as mt_set_threads.  Results do not depend on it.  Fewer
 * threads leave host memory bandwidth to the packer and the DMA engines
 * while an update overlaps them. */
int mt_set_optimizer_threads(int n);

/* ------------------------------------------------------------------------ */
/* Transfer engine                                                          */
/* ------------------------------------------------------------------------ */

/* Just-in-time packer (hyper.ai summary, method: a dedicated CPU worker
 * copies a layer from the pageable store into a pinned buffer from which DMA
 * runs at full bandwidth).  Copies the unit's W region (w_bytes) to dst,
 * which must hold at least w_bytes.  Multithreaded; safe to call for
 * distinct units concurrently; must not overlap mt_step on the same unit. */
int mt_pack_layer(mt_store* st, int unit, void* dst, size_t dst_bytes);

/* Tied weights (paper page, appendix A.1: structural aliasing of the
 * embedding and the LM head, one transfer of the shared matrix): packs the
 * head's device slot from the two units -- the head's final gain and the
 * embedding matrix E as the LM head -- in the untied head layout (dst holds
 * at least that layout's w_bytes).  MT_E_ARG unless cfg.tied. */
int mt_pack_head_tied(mt_store* st, void* dst, size_t dst_bytes);

/* Pinned (page-locked) host memory, hipHostMalloc-backed, owned by the
 * library.  Used for the two weight staging buffers and the gradient slabs
 * (paper page, appendix A.3: two pinned staging buffers sized to the largest
 * layer; K pinned gradient slabs). */
int mt_pinned_alloc(size_t bytes, void** out);
int mt_pinned_free(void* p);

/* Host memory copy with the library's threads and non-temporal stores (the
 * packer's copy), for staging between pageable buffers and pinned slabs.  Its
 * user is an extension of the pages' design: block checkpoints held in host
 * memory for long contexts at full depth (the pages keep activations on the
 * GPU and bound them per block: paper page, section 3 execution workflow;
 * 512K-token runs: section 4, long-context training).  dst and src must not
 * overlap (MT_E_ARG); NULL pointers are MT_E_ARG; 0 bytes is a no-op.
 * Synchronous. */
int mt_host_copy(void* dst, const void* src, size_t bytes);

/* Asynchronous copies on a caller stream (hipStream_t passed as void*):
 * host->device weight stream and device->host gradient evacuation (paper
 * page, appendix A.2: weight and gradient streams beside the compute stream).
 * src/dst on the host side should be pinned for asynchronous DMA. */
int mt_copy_h2d(void* dst_dev, const void* src_host, size_t bytes, void* stream);
int mt_copy_d2h(void* dst_host, const void* src_dev, size_t bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Host optimizer                                                           */
/* ------------------------------------------------------------------------ */
typedef struct mt_adam_cfg {
    double lr, beta1, beta2, eps, weight_decay;
} mt_adam_cfg;

/* CPU-side Adam over one unit (paper page, section 3: optimizer state never
 * leaves host memory; appendix A: SIMD-accelerated optimizer).  If grad_src
 * is non-NULL it holds the unit's bf16 gradient in W-region layout (w_bytes,
 * e.g. a pinned gradient slab) and is first landed into G; then for every
 * element, in fp32 with one rounding per operation:
 *   w = bf16 W (times (1 - lr*wd) if wd != 0); g = bf16 G;
 *   m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
 *   w' = w - (alpha*m) / (sqrt(v) + eps_hat);   W = bf16(w'),
 * with alpha = lr*sqrt(c2)/c1, eps_hat = eps*sqrt(c2), c1 = 1-b1^t,
 * c2 = 1-b2^t: the bias-corrected update lr*(m/c1)/(sqrt(v/c2)+eps) with
 * the corrections folded into two scalars (one division, one square root
 * per element).  Scalar constants are computed in fp64 and rounded once to
 * fp32.  t >= 1.
 * Master-weight stores read w from P instead of W and write P = w' (W is
 * still bf16(w')).  When k >= 1 micro-batch gradients were accumulated
 * (mt_grad_accumulate) since the unit's last step, the gradient landed is
 * the mean over the k + 1 micro-batches: G = bf16((A + bf16 src) / (k + 1))
 * (one fp32 addition, one fp32 division; src = grad_src, or G itself when
 * grad_src is NULL), and the unit's count restarts at 0.
 * If w_fp32_out is non-NULL it receives w' (w_bytes/2 floats, W indexing)
 * before rounding.  Multithreaded, deterministic. */
int mt_step(mt_store* st, int unit, const void* grad_src, const mt_adam_cfg* adam, int64_t t,
            float* w_fp32_out);

/* Gradient accumulation over micro-batches (paper page, section 3,
 * execution workflow: accumulated gradients live in host memory; appendix
 * A.3: a background CPU thread accumulates the offloaded gradients; the
 * author blog: larger batches amortise the per-step weight traffic):
 * adds one micro-batch's bf16 gradient (grad_src in W-region layout, or the
 * unit's G region when NULL) into the fp32 accumulator A, in call order:
 * A = bf16 src for the first micro-batch after a step, A = A + bf16 src
 * after that.  The unit's mt_step after the last micro-batch takes the mean.
 * MT_E_STATE without MT_STORE_GRAD_ACCUM.  Must not overlap mt_step or
 * mt_pack_layer on the same unit. */
int mt_grad_accumulate(mt_store* st, int unit, const void* grad_src);

/* Embedding on the host: dst[t, :] = E[tok[t], :] (bf16, [T, h]). */
int mt_embed_gather(mt_store* st, const int32_t* tok, int64_t T, void* dst);
/* Embedding gradient: dE[v] = sum over t with tok[t] == v of dx0[t]
 * (fp32, accumulated in ascending t), rounded once to bf16 into the
 * embedding unit's G region.  dx0: fp32 [T, h] on the host. */
int mt_embed_grad(mt_store* st, const int32_t* tok, int64_t T, const float* dx0);
/* Tied weights: the shared matrix's gradient is the LM head's plus the
 * embedding's.  head_grad: the head's bf16 gradient [V, h] (its slab, at the
 * LM head's offset); row v of the landed gradient is bf16 of the fp32 sum
 * head_grad[v] + dx0[t] over t with tok[t] == v, in ascending t (rows of
 * absent tokens: head_grad[v]).  MT_E_ARG unless cfg.tied. */
int mt_embed_grad_tied(mt_store* st, const int32_t* tok, int64_t T, const float* dx0, const void* head_grad);

/* RoPE tables computed on the host in fp64 (angle s * base^(-2i/hd)) and
 * rounded to fp32: cos_out, sin_out are [seq, head_dim/2]. */
int mt_rope_tables(const mt_model_cfg* cfg, int32_t seq, float* cos_out, float* sin_out);

/* ------------------------------------------------------------------------ */
/* Stateless layer template on the device                                   */
/* ------------------------------------------------------------------------ */

/* Views of one unit's tensors inside a device weight slot and gradient slot
 * (same offsets as the host W region). */
typedef struct mt_layer_view {
    const void* w[6];
    void* g[6];
} mt_layer_view;

/* Bind (paper page, appendix A.4; hyper.ai summary, method: a Bind primitive
 * maps views of the streaming buffer onto the template's input slots).  Pure
 * pointer arithmetic over the unit layout: no copy, no launch.  The head's
 * device slot always has the untied head layout (final gain, then the LM
 * head [V, h]); with tied weights mt_pack_head_tied fills it.  dev_g_slot may
 * be NULL (forward only).  MT_E_ALIGN unless both slots are 256-byte
 * aligned. */
int mt_bind(const mt_model_cfg* cfg, int unit, const void* dev_w_slot, void* dev_g_slot,
            mt_layer_view* out);

/* Activations of one layer call.  T = batch * seq tokens, row-major [T, h]
 * with token t = b * seq + s.  Positions restart at 0 in every batch row. */
typedef struct mt_act {
    int32_t batch, seq;
    const void* x_in;      /* bf16 [T, h]: layer input */
    void* x_out;           /* bf16 [T, h]: layer output (forward) */
    const float* dy;       /* fp32 [T, h]: gradient of the layer output */
    const void* dy_bf16;   /* bf16 copy of dy */
    float* dx;             /* fp32 [T, h]: gradient of the layer input */
    void* dx_bf16;         /* bf16 copy of dx */
    const float* rope_cos; /* fp32 [seq, head_dim/2] (device) */
    const float* rope_sin;
    void* saved;           /* layer internals (mt_layer_saved_bytes) or NULL */
    void* workspace;       /* scratch, 256-byte aligned (see below) */
    size_t saved_bytes, workspace_bytes;
} mt_act;

/* Bytes of a layer's saved internals (n1, rstd1, qkv, o, lse, x_mid, n2,
 * rstd2, gate|up, a; above 32768 tokens per call the MLP runs in token chunks
 * of 32768 and n2, gate|up and a are not kept: the backward recomputes them
 * chunk by chunk, as the pages' chunked MLP execution for long contexts
 * keeps the [tokens, ffn] buffers bounded).  Workspace of a layer call: mt_layer_workspace_bytes
 * when io->saved is given; a call without a saved buffer keeps the internals
 * in the workspace too and needs workspace + saved bytes.  MT_E_ARG when a
 * buffer is too small. */
int mt_layer_saved_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out);
int mt_layer_workspace_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out);

/* Layer forward (paper page, section 3, execution workflow: bind streamed
 * weights to a template and compute): RMSNorm, QKV GEMM, RoPE, causal
 * attention, output projection + residual, RMSNorm, gate/up GEMM, SwiGLU,
 * down projection + residual.  x_out = layer(x_in).  The projections take
 * fp16 operands (weights converted exactly, activations rounded once from
 * fp32) and q, k, v and the attention probabilities are kept in fp16; x_out
 * is bf16.  When io->saved is non-NULL the internals needed by the backward
 * are stored there; otherwise the workspace holds them as scratch.  Needs
 * x_in, x_out, rope tables, workspace.  MT_E_SHAPE unless head_dim is 64 or
 * 128. */
int mt_layer_fwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_act* io, void* stream);

/* Layer backward with recompute (paper page, section 3: block checkpoints,
 * activations recomputed in the backward, gradients offloaded right away):
 * if io->saved is NULL the layer's internals are first recomputed from x_in
 * into the workspace; otherwise they are read from io->saved (written by an
 * earlier mt_layer_fwd of the same x_in and weights).  The same kernels run in
 * both cases, so the results are bit-identical.  Writes dx, dx_bf16 and the
 * bf16 weight gradients into v->g (the device gradient slot). */
int mt_layer_recompute_bwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_act* io,
                           void* stream);

/* Head: final RMSNorm, LM head, mean next-token cross entropy over the
 * batch*(seq-1) labelled positions (label of token (b, s) is tok[b, s+1]),
 * and its backward, processed in token chunks of at most 8192. */
typedef struct mt_head_io {
    int32_t batch, seq;
    const void* x;         /* bf16 [T, h]: output of the last layer */
    const int32_t* tokens; /* device int32 [batch, seq] */
    float* dx;             /* fp32 [T, h]: gradient of x */
    void* dx_bf16;         /* bf16 copy of dx */
    float* loss;           /* device fp32 scalar */
    void* workspace;       /* mt_head_workspace_bytes */
    size_t workspace_bytes;
} mt_head_io;

int mt_head_workspace_bytes(const mt_model_cfg* cfg, int32_t batch, int32_t seq, size_t* out);
/* v binds the head unit: w[0] = final gain [h], w[1] = LM head [V, h];
 * g[0], g[1] receive their bf16 gradients. */
int mt_head_fwd_bwd(const mt_layer_view* v, const mt_model_cfg* cfg, const mt_head_io* io,
                    void* stream);

/* ------------------------------------------------------------------------ */
/* Single-operation entry points (the template's kernels, for tests)        */
/* ------------------------------------------------------------------------ */

/* C = op(A) * op(B), bf16 inputs, fp32 accumulation on MFMA.
 * a_kmajor: A is [M, K] (row stride lda) if nonzero, else [K, M].
 * b_kmajor: B is [N, K] (row stride ldb) if nonzero, else [K, N].
 * Outputs (any may be NULL, at least one not): c_f32 [M, N] fp32 (accumulated
 * into when accumulate != 0), c_bf16 [M, N] bf16, optional resid_bf16 [M, N]
 * added before rounding to c_bf16 / storing c_f32.  ldc is the row stride of
 * all of C's arrays.  M, N, K, lda, ldb, ldc must be positive multiples of 8
 * (MT_E_SHAPE otherwise); pointers 16-byte aligned.  ws/ws_bytes: fp32
 * scratch for deterministic split-K (may be NULL: no split). */
int mt_op_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, int a_kmajor,
               const void* B, int64_t ldb, int b_kmajor, float* c_f32, void* c_bf16,
               const void* resid_bf16, int64_t ldc, int accumulate, void* ws, size_t ws_bytes,
               void* stream);

/* Causal attention forward on a fused QKV buffer: qkv bf16 [batch*seq, 3*heads*hd]
 * (q | k | v, head-major inside each), o bf16 [batch*seq, heads*hd],
 * lse fp32 [batch, heads, seq] (natural-log row logsumexp of the scaled
 * scores).  Scale 1/sqrt(hd).  hd in {64, 128}.  ws: device scratch of at
 * least mt_op_attention_ws_bytes (the backward's per-row dot products
 * D = rowsum(dO * O), fp32 [batch, heads, seq]; the forward needs none). */
int mt_op_attention_fwd(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv, void* o,
                        float* lse, void* ws, size_t ws_bytes, void* stream);
/* Its backward: writes dq | dk | dv into dqkv (same layout as qkv). */
int mt_op_attention_bwd(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv,
                        const void* o, const float* lse, const void* d_o, void* dqkv, void* ws,
                        size_t ws_bytes, void* stream);
/* The same attention backward without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Its scratch (the row dot
 * products, 4 bytes per batch*heads*seq row) lives in a file-scope device
 * array of 64 MiB that every GPU the library runs on holds until the process
 * ends: MT_E_ARG when batch*heads*seq exceeds 16777216 rows (16M), and no
 * allocation of any kind is made.  Results are bit-identical to
 * mt_op_attention_bwd.  All calls on one GPU share that array: calls that
 * overlap in time on one GPU (e.g. on two streams) race and must be ordered
 * by the caller. */
int mt_op_attention_bwd_noalloc(int32_t batch, int32_t seq, int32_t heads, int32_t hd, const void* qkv,
                                const void* o, const float* lse, const void* d_o, void* dqkv, void* stream);
/* Scratch bytes either attention call needs. */
int mt_op_attention_ws_bytes(int32_t batch, int32_t seq, int32_t heads, int32_t hd, size_t* out);

/* ------------------------------------------------------------------------ */
/* Kernel timing                                                            */
/* ------------------------------------------------------------------------ */

/* One kernel class: GEMMs by operand orientation and type ("gemm_fwd16" the
 * layer forward's fp16 projections, "gemm_nt" the LM head's forward,
 * "gemm_nn" input gradient, "gemm_tn" weight gradient, each including its
 * split-K reduction) and attention ("attn_fwd", "attn_bwd").  flops are the
 * algorithmic flops of the recorded launches (2*M*N*K per GEMM; causal
 * attention counts the scores and products on and below the diagonal). */
typedef struct mt_prof_entry {
    char name[24];
    int64_t launches;
    double ms;
    double flops;
} mt_prof_entry;

/* Attainable bf16 MFMA rate of this GPU under sustained load (the denominator
 * of an MFMA utilisation that the clock under load cannot distort): launches,
 * on `stream`, a kernel of independent v_mfma_f32_32x32x16_bf16 chains on
 * register operands on every SIMD (no memory traffic) for iters / 5
 * iterations, then times one with `iters` iterations (1e5 takes about 50 ms)
 * and returns its rate in TFLOP/s in *tflops; synchronises the stream.
 * sink: device buffer of at least 2048 floats (written only by a result the
 * kernel cannot produce).  Not part of the training path. */
int mt_probe_mfma(int32_t iters, float* sink, void* stream, double* tflops);

/* on != 0: from now on every launch of a timed class is bracketed by two HIP
 * events recorded on the launch's own stream (events without the system-scope
 * fence, taken from a pool that switching on fills); on == 0 stops recording. */
int mt_prof_enable(int on);
/* Waits for the recorded events, adds their elapsed times into per-class
 * totals, and copies up to max entries (classes with launches) to out;
 * *n receives the number written.  reset != 0 clears the totals afterwards. */
int mt_prof_collect(mt_prof_entry* out, int max, int* n, int reset);

/* Thread-local message of the calling thread's last failure. */
const char* mt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MT_H */
