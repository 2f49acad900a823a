"""Plain CPU oracle of one layer-streamed training step (TEST INFRASTRUCTURE).

This module is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(the HIP library and its Python binding) never calls it and shares no code with
it; the only shared module is ``synth`` (seeded inputs, no training arithmetic).

What it computes.  The method -- host memory as the authoritative store,
per-layer streaming of weights, block checkpointing with recompute, gradient
offload, host-side Adam -- is a *schedule*: it reaches exactly the result of
one ordinary training step of the model (MegaTrain paper page, section 3
"MegaTrain System", execution workflow: block checkpoints only trade extra
forward compute for bounded memory; hyper.ai summary, experiments: no
numerical drift against the standard baselines).  So this oracle is the plain
definition: a forward pass, an analytic backward pass written out by hand (no
autodiff) and an Adam step in the method's storage format (bf16 weights, bf16
gradients, fp32 moments; paper page, section 2 "Preliminaries", the 12 bytes
per parameter accounting).  A second mode, ``streamed``, follows the method's
own order (keep only block-start activations, recompute a block, run its
backward top-down, update each layer as soon as its gradient exists) and exists
only to check that the schedule leaves the result unchanged.

Every function is generic over numpy float32 / float64 (``dt``); arithmetic is
done in that precision on weights that are exact bf16 values.

Readings taken where the pages are silent:
Llama-style pre-norm RMSNorm with eps inside the square root and the gain after
normalising; fused QKV; rotate-half RoPE with cos/sin tables computed in fp64
and rounded to fp32; causal softmax attention with scale 1/sqrt(hd); SwiGLU
silu(gate) * up; an LM head behind a final RMSNorm, untied unless the tied
form (head = embedding matrix) is asked for; mean next-token cross
entropy over the B*(S-1) labelled positions; PyTorch-form Adam with bias
correction, on the bf16 weights themselves unless an fp32 master copy is
kept; micro-batch gradients are rounded to bf16 each and averaged in fp32.
"""
import numpy as np

from synth import bf16_bits_to_f32, f32_to_bf16_bits, layer_tensor_shapes


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def bf16_round(x):
    """Round-to-nearest-even to bf16, returned widened to float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def to_float(bits_tree, dt):
    """Convert a (nested) dict/list of bf16 bit arrays into float arrays of
    dtype dt.  A model whose "head" is None ties its LM head to the
    embedding: the float tree's "head" is then the embedding array itself."""
    if isinstance(bits_tree, dict):
        out = {k: to_float(v, dt) for k, v in bits_tree.items() if v is not None}
        if "embed" in bits_tree and "head" in bits_tree and bits_tree["head"] is None:
            out["head"] = out["embed"]
        return out
    if isinstance(bits_tree, list):
        return [to_float(v, dt) for v in bits_tree]
    return bf16_bits_to_f32(bits_tree).astype(dt)


# ----------------------------------------------------------------------------
# building blocks of the layer template (paper page, appendix A.4: templates
# hold attention and MLP kernels; the pages leave their math to the model)
# ----------------------------------------------------------------------------

def rmsnorm_fwd(x, g, eps):
    """y = x * (mean_j x_j^2 + eps)^(-1/2) * g, row-wise over the last axis."""
    dt = x.dtype
    r = (1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + dt.type(eps))).astype(dt)
    xh = x * r
    return xh * g, xh, r


def rmsnorm_bwd(dy, xh, r, g):
    """Gradient of rmsnorm_fwd.  Returns (dx, dg)."""
    dg = np.sum(dy * xh, axis=tuple(range(dy.ndim - 1)))
    gy = dy * g
    dx = r * (gy - xh * np.mean(gy * xh, axis=-1, keepdims=True))
    return dx, dg


def rope_tables(S, hd, base):
    """cos/sin of the angle s * base^(-2i/hd), i < hd/2, in fp64 rounded to fp32."""
    i = np.arange(hd // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / hd)
    ang = np.arange(S, dtype=np.float64)[:, None] * theta[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_fwd(a, cos, sin):
    """Rotate pairs (i, i + hd/2) of the last axis by the position angle.

    ``a`` has shape [..., S, hd]; cos/sin have shape [S, hd/2]."""
    half = a.shape[-1] // 2
    c = cos.astype(a.dtype)
    s = sin.astype(a.dtype)
    a1, a2 = a[..., :half], a[..., half:]
    return np.concatenate([a1 * c - a2 * s, a2 * c + a1 * s], axis=-1)


def rope_bwd(da, cos, sin):
    """Gradient of rope_fwd: the rotation by the opposite angle."""
    half = da.shape[-1] // 2
    c = cos.astype(da.dtype)
    s = sin.astype(da.dtype)
    d1, d2 = da[..., :half], da[..., half:]
    return np.concatenate([d1 * c + d2 * s, d2 * c - d1 * s], axis=-1)


def attention_fwd(q, k, v):
    """Causal softmax attention per (batch, head).

    q, k, v: [B, nh, S, hd].  Returns o [B, nh, S, hd] and the row softmax
    P [B, nh, S, S] (zeros above the diagonal)."""
    dt = q.dtype
    B, nh, S, hd = q.shape
    scale = dt.type(1.0 / np.sqrt(hd))
    mask = np.triu(np.ones((S, S), dtype=bool), 1)
    o = np.empty_like(q)
    P = np.empty((B, nh, S, S), dtype=dt)
    for b in range(B):
        for hh in range(nh):
            A = (q[b, hh] @ k[b, hh].T) * scale
            A[mask] = -np.inf
            A = A - A.max(axis=-1, keepdims=True)
            E = np.exp(A)
            Pb = E / E.sum(axis=-1, keepdims=True)
            P[b, hh] = Pb
            o[b, hh] = Pb @ v[b, hh]
    return o, P


def attention_bwd(do, q, k, v, o, P):
    """Gradient of attention_fwd.  Returns (dq, dk, dv)."""
    dt = q.dtype
    hd = q.shape[-1]
    scale = dt.type(1.0 / np.sqrt(hd))
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    B, nh = q.shape[:2]
    for b in range(B):
        for hh in range(nh):
            Pb = P[b, hh]
            dv[b, hh] = Pb.T @ do[b, hh]
            dP = do[b, hh] @ v[b, hh].T
            Drow = np.sum(do[b, hh] * o[b, hh], axis=-1, keepdims=True)
            dA = Pb * (dP - Drow)
            dq[b, hh] = (dA @ k[b, hh]) * scale
            dk[b, hh] = (dA.T @ q[b, hh]) * scale
    return dq, dk, dv


def attention_suffix(q, k, v, do, r0, o_rows=None):
    """Causal attention of one head, evaluated only for the query rows s >= r0.

    q, k, v, do: [S, hd] of one (batch, head).  Every query s attends to keys
    0..s, so the outputs of the rows s >= r0 need only those rows' scores; and
    key j is attended only by queries s >= j, so for j >= r0 the suffix rows
    hold every term of dk_j and dv_j.  Returns, for rows / keys r0..S-1:
    o, lse (natural-log logsumexp of the scaled scores), dq, dk, dv.  Used to
    check long sequences where the full S x S probabilities do not fit.
    ``o_rows`` (optional) is the forward output at which the backward is
    evaluated (its rows enter rowsum(dO * O)); by default the rows' own o."""
    dt = q.dtype
    S, hd = q.shape
    scale = dt.type(1.0 / np.sqrt(hd))
    A = (q[r0:] @ k.T) * scale
    future = np.arange(S)[None, :] > np.arange(r0, S)[:, None]
    A[future] = -np.inf
    amax = A.max(axis=-1, keepdims=True)
    E = np.exp(A - amax)
    l = E.sum(axis=-1, keepdims=True)
    P = E / l
    lse = (amax + np.log(l))[:, 0]
    o = P @ v
    dP = do[r0:] @ v.T
    Drow = np.sum(do[r0:] * (o if o_rows is None else o_rows), axis=-1, keepdims=True)
    dA = P * (dP - Drow)
    dq = (dA @ k) * scale
    dk = (dA[:, r0:].T @ q[r0:]) * scale
    dv = P[:, r0:].T @ do[r0:]
    return o, lse, dq, dk, dv


def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_fwd(gate, up):
    return silu(gate) * up


def swiglu_bwd(da, gate, up):
    """Gradient of silu(gate) * up.  Returns (dgate, dup)."""
    sig = 1.0 / (1.0 + np.exp(-gate))
    dgate = da * up * sig * (1.0 + gate * (1.0 - sig))
    dup = da * (gate * sig)
    return dgate, dup


# ----------------------------------------------------------------------------
# one decoder layer (the stateless template applied to bound weights)
# ----------------------------------------------------------------------------

def _heads(t, B, S, nh, hd):
    return t.reshape(B, S, nh, hd).transpose(0, 2, 1, 3)


def _tokens(t, B, S, h):
    return t.transpose(0, 2, 1, 3).reshape(B * S, h)


def layer_fwd(x, W, cfg, cos, sin):
    """x [T, h] -> (y [T, h], cache).  W: dict of float arrays of one layer."""
    B, S, nh, hd, h, f = cfg.batch, cfg.seq, cfg.heads, cfg.head_dim, cfg.hidden, cfg.ffn
    n1, xh1, r1 = rmsnorm_fwd(x, W["g_attn"], cfg.eps)
    qkv = n1 @ W["wqkv"].T
    q = rope_fwd(_heads(qkv[:, :h], B, S, nh, hd), cos, sin)
    k = rope_fwd(_heads(qkv[:, h:2 * h], B, S, nh, hd), cos, sin)
    v = _heads(qkv[:, 2 * h:], B, S, nh, hd)
    oh, P = attention_fwd(q, k, v)
    o = _tokens(oh, B, S, h)
    xm = x + o @ W["wo"].T
    n2, xh2, r2 = rmsnorm_fwd(xm, W["g_mlp"], cfg.eps)
    gu = n2 @ W["wgu"].T
    gate, up = gu[:, :f], gu[:, f:]
    a = swiglu_fwd(gate, up)
    y = xm + a @ W["wd"].T
    cache = dict(x=x, n1=n1, xh1=xh1, r1=r1, q=q, k=k, v=v, oh=oh, P=P, o=o, xm=xm,
                 n2=n2, xh2=xh2, r2=r2, gate=gate, up=up, a=a)
    return y, cache


def layer_bwd(dy, c, W, cfg, cos, sin):
    """Analytic backward of layer_fwd.  Returns (dx, dW dict)."""
    B, S, nh, hd, h = cfg.batch, cfg.seq, cfg.heads, cfg.head_dim, cfg.hidden
    dW = {}
    # down projection and residual
    dW["wd"] = dy.T @ c["a"]
    da = dy @ W["wd"]
    dgate, dup = swiglu_bwd(da, c["gate"], c["up"])
    dgu = np.concatenate([dgate, dup], axis=1)
    dW["wgu"] = dgu.T @ c["n2"]
    dn2 = dgu @ W["wgu"]
    dxm_norm, dW["g_mlp"] = rmsnorm_bwd(dn2, c["xh2"], c["r2"], W["g_mlp"])
    dxm = dy + dxm_norm
    # attention block
    dW["wo"] = dxm.T @ c["o"]
    do = _heads(dxm @ W["wo"], B, S, nh, hd)
    dq, dk, dv = attention_bwd(do, c["q"], c["k"], c["v"], c["oh"], c["P"])
    dq = rope_bwd(dq, cos, sin)
    dk = rope_bwd(dk, cos, sin)
    dqkv = np.concatenate([_tokens(dq, B, S, h), _tokens(dk, B, S, h), _tokens(dv, B, S, h)], axis=1)
    dW["wqkv"] = dqkv.T @ c["n1"]
    dn1 = dqkv @ W["wqkv"]
    dx_norm, dW["g_attn"] = rmsnorm_bwd(dn1, c["xh1"], c["r1"], W["g_attn"])
    return dxm + dx_norm, dW


# ----------------------------------------------------------------------------
# one layer of a long sequence, for an output gradient that is zero outside a
# few row blocks (the long-context shapes: the plain layer's S x S
# probabilities and all-rows attention backward do not fit a CPU budget)
# ----------------------------------------------------------------------------

def _par(fn, items, workers=None):
    """fn over independent items on a thread pool (numpy and BLAS release the
    GIL inside array operations); returns the results in item order.  Only
    evaluation order changes: each item's arithmetic is the same as in a
    loop, and every sum across items is taken afterwards in item order."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    items = list(items)
    n = workers or max(1, min(len(items), len(os.sched_getaffinity(0))))
    if n == 1:
        return [fn(it) for it in items]
    with ThreadPoolExecutor(n) as ex:
        return list(ex.map(fn, items))


def _blas_one_thread():
    """Context in which BLAS calls run single-threaded (used around thread
    pools whose items each call BLAS, so the pools do not oversubscribe)."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1, user_api="blas")


def _rope_rows(a, cos, sin, nh, hd, inverse=False):
    """RoPE on token rows [n, nh*hd] whose positions are the rows of cos/sin
    ([n, hd/2]): the rotation of rope_fwd (rope_bwd when ``inverse``) applied
    to each head."""
    n = a.shape[0]
    ah = a.reshape(n, nh, hd).transpose(1, 0, 2)
    r = rope_bwd(ah, cos, sin) if inverse else rope_fwd(ah, cos, sin)
    return np.ascontiguousarray(r.transpose(1, 0, 2)).reshape(n, nh * hd)


def layer_rows(x, W, cfg, cos, sin, blocks, dy_blocks, dx_blocks=None, wqkv_rows=None, chunk=16384):
    """Forward and backward of one layer (layer_fwd / layer_bwd) on ONE
    sequence x [S, h] (positions 0..S-1) when the output gradient dy is zero
    outside the disjoint row ranges ``blocks`` = [(r0, r1), ...], with
    dy[r0:r1] = dy_blocks[i].

    Why this needs only those rows' queries: the layer is per token except
    for attention, and a query s attends to keys 0..s.  With dy zero outside
    the blocks, the MLP, the output projection and dO are zero outside them
    too, so the attention backward has terms only for the blocks' queries:
    dq lives on the block rows, while dk_j and dv_j collect, for every key
    j <= s, the terms of those queries.  So the exact result needs the
    softmax rows of the blocks' queries only (against all their keys), plus
    per-token work on every row: the attention RMSNorm, the keys and values
    with RoPE, the RoPE backward of dk, the QKV weight gradient (a reduction
    over all S tokens), dn1 and the RMSNorm backward.

    Per-token operations run in token chunks of ``chunk`` rows; attention
    runs exactly (full softmax over keys 0..s, no online rescaling) per
    (head, query block).  Sums over chunks, blocks and heads are taken in
    that order.

    dx_blocks: None for dx on all S rows (and the attention gain's
    gradient, a sum over all rows); or a list of (r0, r1) ranges where dx is
    wanted (the gain gradient is then not formed: None).  wqkv_rows: None for
    the whole QKV weight gradient; or output-row indices of Wqkv whose
    gradient rows are wanted (each still a sum over all S tokens).

    Returns dict(y=[y rows of each block], dx=[S, h] array or [dx rows of each
    dx block], dW={g_attn, wqkv (rows in wqkv_rows order if given), wo,
    g_mlp, wgu, wd})."""
    dt = x.dtype
    S, h = x.shape
    nh, hd, f = cfg.heads, cfg.head_dim, cfg.ffn
    assert nh * hd == h and cos.shape[0] >= S
    scale = dt.type(1.0 / np.sqrt(hd))
    chunks = [(a, min(S, a + chunk)) for a in range(0, S, chunk)]
    cos, sin = cos[:S], sin[:S]
    wq, wk, wv = W["wqkv"][:h], W["wqkv"][h:2 * h], W["wqkv"][2 * h:]

    # forward on every row: attention RMSNorm, keys (RoPE) and values
    n1, xh1 = np.empty_like(x), np.empty_like(x)
    r1 = np.empty((S, 1), dt)

    def norm1(c):
        a, b = c
        n1[a:b], xh1[a:b], r1[a:b] = rmsnorm_fwd(x[a:b], W["g_attn"], cfg.eps)
    _par(norm1, chunks)
    k = n1 @ wk.T
    v = n1 @ wv.T

    def rope_k(c):
        a, b = c
        k[a:b] = _rope_rows(k[a:b], cos[a:b], sin[a:b], nh, hd)
    _par(rope_k, chunks)

    dW = {"wo": np.zeros_like(W["wo"]), "wgu": np.zeros_like(W["wgu"]), "wd": np.zeros_like(W["wd"]),
          "g_mlp": np.zeros_like(W["g_mlp"])}
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    ys, dq_blocks, dxm_blocks = [], [], []
    for (r0, r1_), dy in zip(blocks, dy_blocks):
        # forward of the block's rows: queries, attention per head, the rest per token
        q = _rope_rows(n1[r0:r1_] @ wq.T, cos[r0:r1_], sin[r0:r1_], nh, hd)
        future = np.arange(r1_)[None, :] > np.arange(r0, r1_)[:, None]
        o = np.empty_like(q)
        probs = [None] * nh

        def attn(hh):
            cols = slice(hh * hd, (hh + 1) * hd)
            A = (q[:, cols] @ k[:r1_, cols].T) * scale
            A[future] = -np.inf
            A = A - A.max(axis=-1, keepdims=True)
            E = np.exp(A)
            P = E / E.sum(axis=-1, keepdims=True)
            probs[hh] = P
            o[:, cols] = P @ v[:r1_, cols]
        with _blas_one_thread():
            _par(attn, range(nh))
        xm = x[r0:r1_] + o @ W["wo"].T
        n2, xh2, r2 = rmsnorm_fwd(xm, W["g_mlp"], cfg.eps)
        gu = n2 @ W["wgu"].T
        gate, up = gu[:, :f], gu[:, f:]
        a = swiglu_fwd(gate, up)
        ys.append(xm + a @ W["wd"].T)
        # backward of the block's rows (layer_bwd restricted to them)
        dW["wd"] += dy.T @ a
        dgate, dup = swiglu_bwd(dy @ W["wd"], gate, up)
        dgu = np.concatenate([dgate, dup], axis=1)
        dW["wgu"] += dgu.T @ n2
        dxm_norm, dg = rmsnorm_bwd(dgu @ W["wgu"], xh2, r2, W["g_mlp"])
        dW["g_mlp"] += dg
        dxm = dy + dxm_norm
        dxm_blocks.append(dxm)
        dW["wo"] += dxm.T @ o
        do = dxm @ W["wo"]
        dq = np.empty_like(q)

        def attn_bwd(hh):
            cols = slice(hh * hd, (hh + 1) * hd)
            P = probs[hh]
            dv[:r1_, cols] += P.T @ do[:, cols]
            dP = do[:, cols] @ v[:r1_, cols].T
            D = np.sum(do[:, cols] * o[:, cols], axis=-1, keepdims=True)
            dA = P * (dP - D)
            dq[:, cols] = (dA @ k[:r1_, cols]) * scale
            dk[:r1_, cols] += (dA.T @ q[:, cols]) * scale
        with _blas_one_thread():
            _par(attn_bwd, range(nh))
        dq_blocks.append(_rope_rows(dq, cos[r0:r1_], sin[r0:r1_], nh, hd, inverse=True))
        del probs

    def rope_dk(c):
        a, b = c
        dk[a:b] = _rope_rows(dk[a:b], cos[a:b], sin[a:b], nh, hd, inverse=True)
    _par(rope_dk, chunks)

    def dqkv_rows(a, b):
        """[b - a, 3h] gradient of the fused QKV output on rows a..b-1."""
        d = np.concatenate([np.zeros((b - a, h), dt), dk[a:b], dv[a:b]], axis=1)
        for (r0, r1_), dq in zip(blocks, dq_blocks):
            lo, hi = max(a, r0), min(b, r1_)
            if lo < hi:
                d[lo - a:hi - a, :h] = dq[lo - r0:hi - r0]
        return d

    # QKV weight gradient: a reduction over all S tokens, chunk by chunk
    sel = None if wqkv_rows is None else np.asarray(wqkv_rows)
    dW["wqkv"] = np.zeros((3 * h if sel is None else len(sel), h), dt)
    for a, b in chunks:
        d = dqkv_rows(a, b)
        dW["wqkv"] += (d if sel is None else d[:, sel]).T @ n1[a:b]

    def dx_rows(a, b):
        dxn, dg = rmsnorm_bwd(dqkv_rows(a, b) @ W["wqkv"], xh1[a:b], r1[a:b], W["g_attn"])
        for (r0, r1_), dxm in zip(blocks, dxm_blocks):
            lo, hi = max(a, r0), min(b, r1_)
            if lo < hi:
                dxn[lo - a:hi - a] += dxm[lo - r0:hi - r0]
        return dxn, dg

    if dx_blocks is None:
        dx = np.empty_like(x)
        dW["g_attn"] = np.zeros_like(W["g_attn"])
        for a, b in chunks:
            dx[a:b], dg = dx_rows(a, b)
            dW["g_attn"] += dg
    else:
        dx = [dx_rows(a, b)[0] for a, b in dx_blocks]
        dW["g_attn"] = None
    return dict(y=ys, dx=dx, dW=dW)


# ----------------------------------------------------------------------------
# head: final RMSNorm, LM head, next-token cross entropy
# ----------------------------------------------------------------------------

def labels_of(tok):
    """label[b, s] = tok[b, s+1]; the last position of each row has no label."""
    return tok[:, 1:]


def head_fwd_bwd(x, g_final, w_head, tok, cfg):
    """Loss and gradients of the head.  Returns (loss, per_pos_loss, dx, dg_final, dw_head)."""
    B, S, V = cfg.batch, cfg.seq, cfg.vocab
    dt = x.dtype
    xf, xhf, rf = rmsnorm_fwd(x, g_final, cfg.eps)
    z = (xf @ w_head.T).reshape(B, S, V)
    zmax = z.max(axis=-1, keepdims=True)
    lse = (zmax + np.log(np.sum(np.exp(z - zmax), axis=-1, keepdims=True)))[..., 0]
    lab = labels_of(tok)
    N = B * (S - 1)
    zl = np.take_along_axis(z[:, :-1], lab[..., None].astype(np.int64), axis=-1)[..., 0]
    per_pos = lse[:, :-1] - zl
    loss = per_pos.sum() / dt.type(N)
    dz = np.exp(z - lse[..., None]) / dt.type(N)
    dz[:, -1, :] = 0
    bi, si = np.meshgrid(np.arange(B), np.arange(S - 1), indexing="ij")
    dz[bi, si, lab] -= dt.type(1.0) / dt.type(N)
    dz = dz.reshape(B * S, V)
    dw_head = dz.T @ xf
    dxf = dz @ w_head
    dx, dg = rmsnorm_bwd(dxf, xhf, rf, g_final)
    return loss, per_pos, dx, dg, dw_head


# ----------------------------------------------------------------------------
# Adam in the method's storage format (paper page, section 3: CPU-side Adam,
# moments never leave host memory; section 2: bf16 weights and grads, fp32
# moments)
# ----------------------------------------------------------------------------

def adam_consts(adam, t):
    """Scalar constants, each computed in fp64 and rounded once to fp32.

    The bias corrections c1 = 1 - beta1^t and c2 = 1 - beta2^t are folded into
    the step size and epsilon: alpha = lr * sqrt(c2) / c1 and
    eps_hat = eps * sqrt(c2).  In exact arithmetic
    lr * (m / c1) / (sqrt(v / c2) + eps) = alpha * m / (sqrt(v) + eps_hat),
    so this is the bias-corrected Adam update itself, in the form that needs
    one division and one square root per element."""
    f = np.float32
    c1 = 1.0 - adam.beta1 ** t
    c2 = 1.0 - adam.beta2 ** t
    return dict(b1=f(adam.beta1), b2=f(adam.beta2), omb1=f(1.0 - adam.beta1), omb2=f(1.0 - adam.beta2),
                alpha=f(adam.lr * np.sqrt(c2) / c1), eps_hat=f(adam.eps * np.sqrt(c2)),
                decay=f(1.0 - adam.lr * adam.weight_decay))


def adam_update(w_bits, g_fp32, m, v, adam, t, master=None):
    """One Adam step on one tensor, all in fp32, one IEEE rounding per operation.

    w_bits: bf16 weights (uint16); g_fp32: gradient as computed; m, v: fp32
    moments (updated in place).  The gradient is first stored as bf16, as the
    method keeps bf16 gradients on the host.  Operation order:
    m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*(g*g);
    w' = w - (alpha*m) / (sqrt(v) + eps_hat)   (constants of adam_consts).
    With ``master`` (fp32 master weights, updated in place) w is read from
    the master copy instead of the bf16 weights and receives w'.
    Returns (new bf16 bits, the fp32 weight before its bf16 rounding)."""
    k = adam_consts(adam, t)
    w = bf16_bits_to_f32(w_bits) if master is None else master.astype(np.float32)
    if adam.weight_decay != 0.0:
        w = w * k["decay"]
    gh = bf16_round(g_fp32)
    m[...] = k["b1"] * m + k["omb1"] * gh
    v[...] = k["b2"] * v + k["omb2"] * (gh * gh)
    denom = np.sqrt(v) + k["eps_hat"]
    step = k["alpha"] * m
    w_new = (w - step / denom).astype(np.float32)
    if master is not None:
        master[...] = w_new
    return f32_to_bf16_bits(w_new), w_new


def accumulate_micro(acc, g_fp32, first):
    """Gradient accumulation over micro-batches (paper page, section 3,
    execution workflow: accumulated gradients live in host memory; appendix
    A.3: a CPU thread accumulates the offloaded gradients).  Each
    micro-batch's gradient is stored as bf16, as the device produces it, and
    added in fp32 in micro-batch order.  Returns the new accumulator."""
    gh = bf16_round(np.asarray(g_fp32, dtype=np.float32))
    return gh.copy() if first else (acc + gh).astype(np.float32)


def accumulated_mean(acc, g_last_fp32, n):
    """The gradient Adam receives after n micro-batches: the mean
    (acc + bf16 g_last) / n, one fp32 addition and one fp32 division (acc
    holds the first n - 1)."""
    gh = bf16_round(np.asarray(g_last_fp32, dtype=np.float32))
    return ((acc + gh).astype(np.float32) / np.float32(n)).astype(np.float32)


# ----------------------------------------------------------------------------
# full step
# ----------------------------------------------------------------------------

def embed_fwd(embed, tok):
    return embed[tok.reshape(-1)]


def embed_bwd(dx0, tok, V, init=None):
    """dE[v] = init[v] (or 0) + sum over positions t with tok_t == v of
    dx0[t], accumulated in ascending t.  With a tied LM head ``init`` is the
    head's gradient as the device stores it (bf16): the shared matrix's
    gradient is the sum of both uses (paper page, appendix A.1: tied
    embedding and head share one physical store)."""
    dE = np.zeros((V, dx0.shape[1]), dtype=dx0.dtype) if init is None else np.array(init, dtype=dx0.dtype)
    np.add.at(dE, tok.reshape(-1), dx0)
    return dE


def forward_backward(Wf, tok, cfg, mode="resident", ckpt_every=None, on_layer_grad=None):
    """Loss and all gradients of one step.

    Wf: dict of float weights (embed, g_final, head, layers[list of dicts]).
    mode 'resident' keeps every layer's internals; mode 'streamed' keeps only
    the block-start activations (one every ``ckpt_every`` layers), recomputes a
    block's internals in the backward, and visits layers in the method's
    order.  ``on_layer_grad(l, dW)`` is called as soon as a layer's gradient
    exists (the hook where the method runs that layer's Adam)."""
    dt = Wf["embed"].dtype
    L = cfg.layers
    cos, sin = rope_tables(cfg.seq, cfg.head_dim, cfg.rope_base)
    x = embed_fwd(Wf["embed"], tok)
    K = ckpt_every or cfg.ckpt_every
    caches, ckpts = [], {}
    for l in range(L):
        if mode == "streamed" and l % K == 0:
            ckpts[l] = x
        x, c = layer_fwd(x, Wf["layers"][l], cfg, cos, sin)
        if mode == "resident":
            caches.append(c)
    loss, per_pos, dx, dg_final, dw_head = head_fwd_bwd(x, Wf["g_final"], Wf["head"], tok, cfg)
    grads = {"g_final": dg_final, "head": dw_head, "layers": [None] * L}
    if mode == "resident":
        for l in reversed(range(L)):
            dx, dW = layer_bwd(dx, caches[l], Wf["layers"][l], cfg, cos, sin)
            grads["layers"][l] = dW
            if on_layer_grad:
                on_layer_grad(l, dW)
    else:
        for b0 in reversed(range(0, L, K)):
            xb = ckpts[b0]
            block = []
            for l in range(b0, min(L, b0 + K)):
                xb, c = layer_fwd(xb, Wf["layers"][l], cfg, cos, sin)
                block.append(c)
            for l in reversed(range(b0, min(L, b0 + K))):
                dx, dW = layer_bwd(dx, block[l - b0], Wf["layers"][l], cfg, cos, sin)
                grads["layers"][l] = dW
                if on_layer_grad:
                    on_layer_grad(l, dW)
    grads["embed"] = embed_bwd(dx, tok, cfg.vocab)
    return loss, per_pos, grads, dx


class HostState:
    """Host-resident training state of the oracle: bf16 weights + fp32 moments
    (+ fp32 master weights with ``master``)."""

    def __init__(self, bits, master=False):
        self.tied = bits.get("head") is None
        self.bits = {"embed": bits["embed"].copy(), "g_final": bits["g_final"].copy(),
                     "head": None if self.tied else bits["head"].copy(),
                     "layers": [{k: v.copy() for k, v in lw.items()} for lw in bits["layers"]]}
        z = lambda a: np.zeros(a.shape, dtype=np.float32)
        top = ("embed", "g_final") if self.tied else ("embed", "g_final", "head")
        self.m = {k: z(self.bits[k]) for k in top}
        self.v = {k: z(self.bits[k]) for k in top}
        self.m["layers"] = [{k: z(a) for k, a in lw.items()} for lw in self.bits["layers"]]
        self.v["layers"] = [{k: z(a) for k, a in lw.items()} for lw in self.bits["layers"]]
        self.master = None
        if master:
            f = bf16_bits_to_f32
            self.master = {k: f(self.bits[k]).astype(np.float32) for k in top}
            self.master["layers"] = [{k: f(a).astype(np.float32) for k, a in lw.items()}
                                     for lw in self.bits["layers"]]
        self.t = 0


def train_step(state, tok, cfg, adam, mode="resident", dt=np.float32, ckpt_every=None):
    """One training step on ``state`` (updated in place).

    ``tok``: int tokens [B, S], or a list of n such micro-batches whose
    gradients are accumulated (``accumulate_micro``) before one Adam step on
    their mean (``accumulated_mean``); one micro-batch is the plain step.
    Returns dict(loss (mean over micro-batches), losses, grads (float, as
    computed; with several micro-batches their accumulated fp32 mean),
    w_fp32 (pre-rounding fp32 weights after Adam, same tree as the
    weights))."""
    micro = list(tok) if isinstance(tok, (list, tuple)) else [tok]
    n = len(micro)
    state.t += 1
    t = state.t
    Wf = to_float(state.bits, dt)
    w_fp32 = {"layers": [dict() for _ in range(cfg.layers)]}
    master = state.master

    def upd(bits_parent, key, g, m, v, ms):
        nb, wf = adam_update(bits_parent[key], g, m, v, adam, t, master=ms)
        bits_parent[key] = nb
        return wf

    def upd_layer(l, dW):
        for name in layer_tensor_shapes(cfg):
            ms = master["layers"][l][name] if master is not None else None
            w_fp32["layers"][l][name] = upd(state.bits["layers"][l], name, dW[name].astype(np.float32),
                                            state.m["layers"][l][name], state.v["layers"][l][name], ms)

    tied = state.tied
    top = ("g_final", "embed") if tied else ("head", "g_final", "embed")

    def top_grads(grads, dx0, tk):
        """Gradients of the non-layer units; tied: the embedding's is the sum
        of its two uses, the head's (stored bf16 by the device) first."""
        out = {k: grads[k] for k in ("head", "g_final", "embed")}
        if tied:
            out["embed"] = embed_bwd(dx0, tk, cfg.vocab, init=bf16_round(grads["head"].astype(np.float32)))
        return out

    acc = None
    losses = []
    for i, tk in enumerate(micro):
        last = i == n - 1
        if not last:
            loss, per_pos, grads, dx0 = forward_backward(Wf, tk, cfg, mode=mode, ckpt_every=ckpt_every)
            tg = top_grads(grads, dx0, tk)
            first = acc is None
            if first:
                acc = {"layers": [dict() for _ in range(cfg.layers)]}
            for l in range(cfg.layers):
                for name in layer_tensor_shapes(cfg):
                    acc["layers"][l][name] = accumulate_micro(acc["layers"][l].get(name), grads["layers"][l][name],
                                                              first)
            for name in top:
                acc[name] = accumulate_micro(acc.get(name), tg[name], first)
            losses.append(loss)
            continue

        def mean_of(g, a):
            return g.astype(np.float32) if a is None else accumulated_mean(a, g, n)

        gmean = {"layers": [None] * cfg.layers}

        def hook(l, dW):
            gmean["layers"][l] = {name: mean_of(dW[name], acc["layers"][l][name] if acc else None) for name in dW}
            upd_layer(l, gmean["layers"][l])

        loss, per_pos, grads, dx0 = forward_backward(Wf, tk, cfg, mode=mode, ckpt_every=ckpt_every,
                                                     on_layer_grad=hook if mode == "streamed" else None)
        losses.append(loss)
        if mode == "resident":
            for l in range(cfg.layers):
                hook(l, grads["layers"][l])
        tg = top_grads(grads, dx0, tk)
        for name in top:
            ms = master[name] if master is not None else None
            gmean[name] = mean_of(tg[name], acc[name] if acc else None)
            w_fp32[name] = upd(state.bits, name, gmean[name], state.m[name], state.v[name], ms)
    # grads: as computed for one micro-batch; with several, the fp32 mean
    # that Adam receives (before its bf16 storage rounding)
    if n == 1:
        gmean = dict(grads, embed=tg["embed"])
    return dict(loss=float(np.mean(np.asarray(losses, dtype=np.float64))), losses=losses, per_pos=per_pos,
                grads=gmean, w_fp32=w_fp32)
