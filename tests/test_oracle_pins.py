"""Pins of the CPU oracle against things other than itself (CPU only).

* fp64 central finite differences of the loss (random coordinates in every
  tensor, random directions);
* an independent fp64 model written with torch library routines
  (rms_norm, scaled_dot_product_attention, silu, cross_entropy, embedding,
  complex multiplication for the rotation) and torch autograd;
* closed forms and special cases (zero LM head gives ln V, zero queries give
  the causal running mean, RoPE identities, constant-row RMSNorm, silu at 0,
  Adam at t = 1);
* invariants of the method: streamed with block recompute equals resident,
  per-layer Adam equals end-of-step Adam, causality;
* golden values: SplitMix64 published outputs, the 12 bytes/parameter
  accounting of the pages.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rand_weights(cfg, rng, std=None, gain_jitter=0.2, dt=np.float64):
    """Float weights with larger spread than the training init, so that softmax
    and SwiGLU are exercised away from their linear regimes, and random gains."""
    h, f, V = cfg.hidden, cfg.ffn, cfg.vocab
    s = std if std is not None else 1.5 / math.sqrt(h)
    mat = lambda *shape: (rng.standard_normal(shape) * s).astype(dt)
    gain = lambda n: (1.0 + gain_jitter * rng.standard_normal(n)).astype(dt)
    layers = []
    for _ in range(cfg.layers):
        layers.append({"g_attn": gain(h), "wqkv": mat(3 * h, h), "wo": mat(h, h), "g_mlp": gain(h),
                       "wgu": mat(2 * f, h), "wd": (rng.standard_normal((h, f)) * 1.5 / math.sqrt(f)).astype(dt)})
    return {"embed": mat(V, h) * 3, "g_final": gain(h), "head": mat(V, h), "layers": layers}


def _loss(Wf, tok, cfg):
    return oracle.forward_backward(Wf, tok, cfg)[0]


def _flat_items(W):
    out = [("embed", None, W["embed"]), ("g_final", None, W["g_final"]), ("head", None, W["head"])]
    for l, lw in enumerate(W["layers"]):
        for k, a in lw.items():
            out.append((k, l, a))
    return out


def _grad_of(grads, name, layer):
    return grads[name] if layer is None else grads["layers"][layer][name]


# ----------------------------------------------------------------------------
# finite differences
# ----------------------------------------------------------------------------

def test_fd_coordinates_every_tensor():
    cfg = synth.preset("micro")
    rng = np.random.default_rng(1)
    W = _rand_weights(cfg, rng)
    tok = synth.make_tokens(cfg)
    loss, _, grads, _ = oracle.forward_backward(W, tok, cfg)
    eps = 1e-5
    checked = 0
    worst = 0.0
    for name, layer, arr in _flat_items(W):
        g = _grad_of(grads, name, layer)
        flat = arr.reshape(-1)
        if name == "embed":
            # rows of tokens that occur, plus one that may not
            rows = np.unique(tok)[:6]
            idx = [r * arr.shape[1] + c for r in rows for c in rng.integers(0, arr.shape[1], 3)]
        else:
            idx = list(rng.integers(0, flat.size, 13))
        for i in idx:
            old = flat[i]
            flat[i] = old + eps
            lp = _loss(W, tok, cfg)
            flat[i] = old - eps
            lm = _loss(W, tok, cfg)
            flat[i] = old
            fd = (lp - lm) / (2 * eps)
            an = g.reshape(-1)[i]
            err = abs(fd - an)
            assert err <= 1e-6 * (abs(fd) + abs(an)) + 2e-10, (name, layer, i, fd, an)
            if abs(an) > 1e-6:
                worst = max(worst, err / abs(an))
            checked += 1
    assert checked >= 200
    assert worst < 1e-5


def test_fd_tied_embedding_gradient_is_the_sum_of_both_uses():
    """Weight tying: the LM head is the embedding array itself.  Central
    differences of the loss w.r.t. entries of the shared matrix (rows of
    tokens that occur and rows that do not) equal the head's gradient plus
    the embedding's, the sum the tied update uses."""
    cfg = synth.preset("micro")
    rng = np.random.default_rng(13)
    W = _rand_weights(cfg, rng)
    W["head"] = W["embed"]  # one array, both uses
    tok = synth.make_tokens(cfg)
    _, _, grads, dx0 = oracle.forward_backward(W, tok, cfg)
    tied = oracle.embed_bwd(dx0, tok, cfg.vocab, init=grads["head"])
    assert np.array_equal(tied, grads["head"] + grads["embed"]) or np.abs(
        tied - (grads["head"] + grads["embed"])).max() <= 1e-15 * np.abs(tied).max()
    E = W["embed"]
    present = np.unique(tok)
    absent = np.setdiff1d(np.arange(cfg.vocab), present)
    rows = list(present[:5]) + list(absent[:3])
    eps = 1e-5
    for r in rows:
        for c in rng.integers(0, E.shape[1], 4):
            old = E[r, c]
            E[r, c] = old + eps
            lp = _loss(W, tok, cfg)
            E[r, c] = old - eps
            lm = _loss(W, tok, cfg)
            E[r, c] = old
            fd = (lp - lm) / (2 * eps)
            an = tied[r, c]
            assert abs(fd - an) <= 1e-6 * (abs(fd) + abs(an)) + 2e-10, (r, c, fd, an)


def test_fd_directional_tiny_init():
    """Directional derivatives on the tiny training shape with its own init."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    W = oracle.to_float(bits, np.float64)
    tok = synth.make_tokens(cfg)
    _, _, grads, _ = oracle.forward_backward(W, tok, cfg)
    rng = np.random.default_rng(7)
    items = _flat_items(W)
    for _ in range(8):
        dirs = [0.02 * rng.standard_normal(a.shape) for _, _, a in items]
        an = sum(float(np.sum(_grad_of(grads, n, l) * d)) for (n, l, _), d in zip(items, dirs))
        eps = 1e-5
        vals = []
        for sgn in (1, -1):
            W2 = {"embed": W["embed"].copy(), "g_final": W["g_final"].copy(), "head": W["head"].copy(),
                  "layers": [{k: v.copy() for k, v in lw.items()} for lw in W["layers"]]}
            for (n, l, _), d in zip(items, dirs):
                tgt = W2[n] if l is None else W2["layers"][l][n]
                tgt += sgn * eps * d
            vals.append(_loss(W2, tok, cfg))
        fd = (vals[0] - vals[1]) / (2 * eps)
        assert abs(fd - an) <= 1e-6 * abs(an) + 1e-10, (fd, an)


# ----------------------------------------------------------------------------
# independent fp64 model from torch library routines + autograd
# ----------------------------------------------------------------------------

def _torch_model_loss(Wt, tok, cfg):
    import torch
    import torch.nn.functional as F
    B, S, h, nh, hd, f, V = cfg.batch, cfg.seq, cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.vocab
    tok_t = torch.from_numpy(tok.astype(np.int64))
    x = F.embedding(tok_t, Wt["embed"])  # [B, S, h]
    theta = torch.tensor(cfg.rope_base, dtype=torch.float64) ** (
        -2.0 * torch.arange(hd // 2, dtype=torch.float64) / hd)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * theta[None, :]
    rot = torch.complex(torch.cos(ang).float().double(), torch.sin(ang).float().double())

    def rope(a):  # a [B, nh, S, hd]
        c = torch.complex(a[..., : hd // 2], a[..., hd // 2:]) * rot
        return torch.cat([c.real, c.imag], dim=-1)

    for lw in Wt["layers"]:
        n1 = F.rms_norm(x, (h,), weight=lw["g_attn"], eps=cfg.eps)
        qkv = n1 @ lw["wqkv"].T
        q, k, v = [t.reshape(B, S, nh, hd).transpose(1, 2) for t in qkv.split(h, dim=-1)]
        o = F.scaled_dot_product_attention(rope(q), rope(k), v, is_causal=True)
        x = x + o.transpose(1, 2).reshape(B, S, h) @ lw["wo"].T
        n2 = F.rms_norm(x, (h,), weight=lw["g_mlp"], eps=cfg.eps)
        gate, up = (n2 @ lw["wgu"].T).split(f, dim=-1)
        x = x + (F.silu(gate) * up) @ lw["wd"].T
    xf = F.rms_norm(x, (h,), weight=Wt["g_final"], eps=cfg.eps)
    z = xf @ Wt["head"].T
    return F.cross_entropy(z[:, :-1].reshape(-1, V), tok_t[:, 1:].reshape(-1))


@pytest.mark.parametrize("preset", ["micro", "tiny"])
def test_against_torch_library_model_fp64(preset):
    torch = pytest.importorskip("torch")
    cfg = synth.preset(preset)
    rng = np.random.default_rng(3)
    W = _rand_weights(cfg, rng)
    tok = synth.make_tokens(cfg)
    loss, _, grads, _ = oracle.forward_backward(W, tok, cfg)
    Wt = {"embed": torch.tensor(W["embed"], requires_grad=True),
          "g_final": torch.tensor(W["g_final"], requires_grad=True),
          "head": torch.tensor(W["head"], requires_grad=True),
          "layers": [{k: torch.tensor(v, requires_grad=True) for k, v in lw.items()} for lw in W["layers"]]}
    lt = _torch_model_loss(Wt, tok, cfg)
    lt.backward()
    assert abs(float(lt.detach()) - loss) <= 1e-12 * abs(loss)
    for name, layer, _ in _flat_items(W):
        tt = Wt[name] if layer is None else Wt["layers"][layer][name]
        ref = tt.grad.numpy()
        got = _grad_of(grads, name, layer)
        scale = np.abs(ref).max()
        assert np.abs(got - ref).max() <= 1e-10 * scale + 1e-300, (name, layer)


# ----------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------

def test_zero_head_gives_log_vocab():
    cfg = synth.preset("tiny")
    W = oracle.to_float(synth.make_weights(cfg), np.float64)
    W["head"][:] = 0
    tok = synth.make_tokens(cfg)
    loss, per_pos, grads, dx0 = oracle.forward_backward(W, tok, cfg)
    assert abs(loss - math.log(cfg.vocab)) < 1e-13
    assert np.all(per_pos == per_pos[0, 0])
    # zero head => no gradient reaches the layers or the embedding
    for lw in grads["layers"]:
        for a in lw.values():
            assert not a.any()
    assert not grads["embed"].any() and not grads["g_final"].any()
    # dW_head = dz^T xf with dz = (1/V - onehot)/N on labelled rows
    N = cfg.batch * (cfg.seq - 1)
    # recompute xf independently of the layer stack through the forward pass
    cos, sin = oracle.rope_tables(cfg.seq, cfg.head_dim, cfg.rope_base)
    x = W["embed"][tok.reshape(-1)]
    for lw in W["layers"]:
        x, _ = oracle.layer_fwd(x, lw, cfg, cos, sin)
    xf = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + cfg.eps) * W["g_final"]
    dz = np.full((cfg.batch, cfg.seq, cfg.vocab), 1.0 / (cfg.vocab * N))
    dz[:, -1, :] = 0
    for b in range(cfg.batch):
        for s in range(cfg.seq - 1):
            dz[b, s, tok[b, s + 1]] -= 1.0 / N
    ref = dz.reshape(-1, cfg.vocab).T @ xf
    np.testing.assert_allclose(grads["head"], ref, rtol=1e-10, atol=1e-15)


def test_attention_zero_queries_is_causal_running_mean():
    rng = np.random.default_rng(0)
    B, nh, S, hd = 2, 3, 17, 8
    q = np.zeros((B, nh, S, hd))
    k = rng.standard_normal((B, nh, S, hd))
    v = rng.standard_normal((B, nh, S, hd))
    o, P = oracle.attention_fwd(q, k, v)
    ref = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-14)
    o1, _ = oracle.attention_fwd(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    assert np.array_equal(o1, v[:, :, :1])


def test_attention_against_torch_sdpa_and_autograd():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(1)
    B, nh, S, hd = 2, 2, 33, 16
    q, k, v, do = (rng.standard_normal((B, nh, S, hd)) for _ in range(4))
    o, P = oracle.attention_fwd(q, k, v)
    dq, dk, dv = oracle.attention_bwd(do, q, k, v, o, P)
    qt, kt, vt = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ot.backward(torch.tensor(do))
    np.testing.assert_allclose(o, ot.detach().numpy(), rtol=1e-12, atol=1e-12)
    for a, t in ((dq, qt), (dk, kt), (dv, vt)):
        np.testing.assert_allclose(a, t.grad.numpy(), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("S,r0", [(41, 0), (41, 29), (41, 40), (7, 3)])
def test_attention_suffix_against_torch_sdpa(S, r0):
    """The suffix evaluation used for long sequences: its rows, logsumexp and
    the gradients of keys >= r0 against torch's SDPA + autograd over the
    whole sequence, and against the full-matrix oracle."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    rng = np.random.default_rng(7 + S + r0)
    hd = 16
    q, k, v, do = (rng.standard_normal((S, hd)) for _ in range(4))
    o, lse, dq, dk, dv = oracle.attention_suffix(q, k, v, do, r0)
    qt, kt, vt = (torch.tensor(a[None, None], requires_grad=True) for a in (q, k, v))
    ot = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    ot.backward(torch.tensor(do[None, None]))
    np.testing.assert_allclose(o, ot.detach().numpy()[0, 0, r0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, qt.grad.numpy()[0, 0, r0:], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dk, kt.grad.numpy()[0, 0, r0:], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dv, vt.grad.numpy()[0, 0, r0:], rtol=1e-11, atol=1e-11)
    sc = torch.tensor(q @ k.T / np.sqrt(hd))
    sc = sc.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=-1).numpy()[r0:], rtol=1e-13, atol=1e-13)
    of, P = oracle.attention_fwd(q[None, None], k[None, None], v[None, None])
    dqf, dkf, dvf = oracle.attention_bwd(do[None, None], q[None, None], k[None, None], v[None, None], of, P)
    np.testing.assert_allclose(dk, dkf[0, 0, r0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, dvf[0, 0, r0:], rtol=1e-12, atol=1e-12)
    # the backward evaluated at a given forward output (rounded o)
    o_given = of + 1e-3 * rng.standard_normal(of.shape)
    _, _, dq2, dk2, _ = oracle.attention_suffix(q, k, v, do, r0, o_rows=o_given[0, 0, r0:])
    dqg, dkg, _ = oracle.attention_bwd(do[None, None], q[None, None], k[None, None], v[None, None], o_given, P)
    np.testing.assert_allclose(dq2, dqg[0, 0, r0:], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dk2, dkg[0, 0, r0:], rtol=1e-12, atol=1e-12)
    assert not np.allclose(dq2, dq, rtol=1e-9, atol=0)


def test_rope_identities():
    rng = np.random.default_rng(2)
    S, hd = 40, 16
    cos, sin = oracle.rope_tables(S, hd, 10000.0)
    a = rng.standard_normal((3, S, hd))
    r = oracle.rope_fwd(a, cos, sin)
    assert np.array_equal(r[:, 0], a[:, 0])  # position 0 is the identity
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(a, axis=-1), rtol=1e-6)
    # complex-multiplication form of the rotate-half convention
    c = (a[..., :hd // 2] + 1j * a[..., hd // 2:]) * (cos.astype(np.float64) + 1j * sin.astype(np.float64))
    np.testing.assert_allclose(r, np.concatenate([c.real, c.imag], axis=-1), rtol=1e-13, atol=1e-14)
    # <R_m q, R_n k> depends only on m - n (exact rotations; tables in fp64 here)
    i = np.arange(hd // 2)
    th = 10000.0 ** (-2.0 * i / hd)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)

    def rot(x, p):
        c, s = np.cos(p * th), np.sin(p * th)
        return np.concatenate([x[:hd // 2] * c - x[hd // 2:] * s, x[hd // 2:] * c + x[:hd // 2] * s])
    assert abs(rot(q, 9) @ rot(k, 4) - rot(q, 25) @ rot(k, 20)) < 1e-12
    # backward is the transpose of the forward rotation
    g = rng.standard_normal((3, S, hd))
    assert abs(np.sum(oracle.rope_fwd(a, cos, sin) * g) - np.sum(a * oracle.rope_bwd(g, cos, sin))) < 1e-10
    # fp64 angles: position 5e5 keeps an accurate angle in the fp32 table
    cos_big, sin_big = oracle.rope_tables(524288, 128, 10000.0)
    p = 524287
    assert abs(cos_big[p, 0] - np.float32(math.cos(p))) == 0


def test_rmsnorm_closed_forms_and_torch():
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    c, eps, h = 0.37, 1e-5, 64
    x = np.full((2, h), c)
    y, xh, r = oracle.rmsnorm_fwd(x, np.ones(h), eps)
    np.testing.assert_allclose(xh, c / math.sqrt(c * c + eps), rtol=1e-15)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, h))
    g = rng.standard_normal(h)
    y, xh, r = oracle.rmsnorm_fwd(x, g, eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.sqrt(np.mean(xh * xh, axis=-1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)
    xt, gt = torch.tensor(x, requires_grad=True), torch.tensor(g, requires_grad=True)
    yt = F.rms_norm(xt, (h,), weight=gt, eps=eps)
    np.testing.assert_allclose(y, yt.detach().numpy(), rtol=1e-13)
    dy = rng.standard_normal((5, h))
    yt.backward(torch.tensor(dy))
    dx, dg = oracle.rmsnorm_bwd(dy, xh, r, g)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_swiglu_closed_forms():
    assert oracle.silu(np.float64(0.0)) == 0.0
    dg, du = oracle.swiglu_bwd(np.array([1.0]), np.array([0.0]), np.array([1.0]))
    assert dg[0] == 0.5 and du[0] == 0.0
    # with up = 1 the product reduces to silu and its derivative
    z = np.linspace(-6, 6, 101)
    dg, _ = oracle.swiglu_bwd(np.ones_like(z), z, np.ones_like(z))
    e = 1e-6
    fd = (oracle.silu(z + e) - oracle.silu(z - e)) / (2 * e)
    np.testing.assert_allclose(dg, fd, rtol=1e-8, atol=1e-10)


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10 ** rng.uniform(-8, 8, 10000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0, 65504.0,
                                  3.0e38, 1e-40], dtype=np.float32)]).astype(np.float32)
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------
# Adam
# ----------------------------------------------------------------------------

def test_adam_first_step_closed_form():
    adam = synth.AdamCfg()
    rng = np.random.default_rng(6)
    w = synth.f32_to_bf16_bits(rng.standard_normal(4096).astype(np.float32) * 0.02)
    g = (rng.standard_normal(4096) * 10 ** rng.uniform(-6, 0, 4096)).astype(np.float32)
    g[:16] = 0.0
    m = np.zeros(4096, np.float32)
    v = np.zeros(4096, np.float32)
    nb, wf = oracle.adam_update(w, g, m, v, adam, 1)
    gh = oracle.bf16_round(g).astype(np.float64)
    wd = synth.bf16_bits_to_f32(w).astype(np.float64)
    ref = wd - adam.lr * gh / (np.abs(gh) + adam.eps)
    np.testing.assert_allclose(wf, ref, rtol=0, atol=4 * np.spacing(np.abs(ref).astype(np.float32)).max())
    assert np.array_equal(wf[:16], synth.bf16_bits_to_f32(w[:16]))  # zero gradient: no move
    assert np.array_equal(nb, synth.f32_to_bf16_bits(wf))


def test_adam_multistep_against_fp64_recurrence():
    adam = synth.AdamCfg(lr=1e-3)
    rng = np.random.default_rng(8)
    n = 512
    # bf16 weights would not move visibly at lr 1e-3 for most entries; use large
    # weights so each update survives rounding, and compare the fp32 w' each step
    w_bits = synth.f32_to_bf16_bits(np.linspace(-0.01, 0.01, n).astype(np.float32))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    m64 = np.zeros(n)
    v64 = np.zeros(n)
    for t in range(1, 6):
        g = rng.standard_normal(n).astype(np.float32) * 1e-2
        w_prev = synth.bf16_bits_to_f32(w_bits).astype(np.float64)
        w_bits, wf = oracle.adam_update(w_bits, g, m, v, adam, t)
        gh = oracle.bf16_round(g).astype(np.float64)
        m64 = adam.beta1 * m64 + (1 - adam.beta1) * gh
        v64 = adam.beta2 * v64 + (1 - adam.beta2) * gh * gh
        ref = w_prev - adam.lr * (m64 / (1 - adam.beta1 ** t)) / (np.sqrt(v64 / (1 - adam.beta2 ** t)) + adam.eps)
        # fp32 recurrences against fp64 ones: error relative to the moment's scale
        np.testing.assert_allclose(m, m64, rtol=0, atol=1e-6 * np.abs(m64).max())
        np.testing.assert_allclose(v, v64, rtol=0, atol=1e-6 * np.abs(v64).max())
        np.testing.assert_allclose(wf, ref, rtol=1e-6, atol=1e-9)


def test_adam_matches_torch_optim_adam():
    torch = pytest.importorskip("torch")
    adam = synth.AdamCfg()
    rng = np.random.default_rng(9)
    n = 2048
    w_bits = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32))
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    _, wf = oracle.adam_update(w_bits, g, m, v, adam, 1)
    p = torch.tensor(synth.bf16_bits_to_f32(w_bits), requires_grad=True)
    opt = torch.optim.Adam([p], lr=adam.lr, betas=(adam.beta1, adam.beta2), eps=adam.eps)
    p.grad = torch.tensor(oracle.bf16_round(g))
    opt.step()
    np.testing.assert_allclose(wf, p.detach().numpy(), rtol=0, atol=2e-7 * 4)


def test_master_adam_tracks_fp64_recurrence_where_bf16_stagnates():
    """With fp32 master weights the update is the plain Adam recurrence on w
    (no bf16 rounding of w between steps): five steps at lr 1e-4 on N(0, 0.02)
    weights follow the fp64 recurrence, while without the master copy most of
    these weights do not move at all (half a bf16 ulp exceeds the step)."""
    adam = synth.AdamCfg()
    rng = np.random.default_rng(11)
    n = 4096
    w0 = synth.f32_to_bf16_bits(rng.standard_normal(n).astype(np.float32) * 0.02)
    master = synth.bf16_bits_to_f32(w0).astype(np.float32)
    w_bits, w_plain = w0.copy(), w0.copy()
    m, v, m2, v2 = (np.zeros(n, np.float32) for _ in range(4))
    m64, v64 = np.zeros(n), np.zeros(n)
    w64 = synth.bf16_bits_to_f32(w0).astype(np.float64)
    for t in range(1, 6):
        g = rng.standard_normal(n).astype(np.float32) * 1e-3
        w_bits, wf = oracle.adam_update(w_bits, g, m, v, adam, t, master=master)
        w_plain, _ = oracle.adam_update(w_plain, g, m2, v2, adam, t)
        gh = oracle.bf16_round(g).astype(np.float64)
        m64 = adam.beta1 * m64 + (1 - adam.beta1) * gh
        v64 = adam.beta2 * v64 + (1 - adam.beta2) * gh * gh
        w64 = w64 - adam.lr * (m64 / (1 - adam.beta1 ** t)) / (np.sqrt(v64 / (1 - adam.beta2 ** t)) + adam.eps)
        assert np.array_equal(master, wf)
        assert np.array_equal(w_bits, synth.f32_to_bf16_bits(master))
        np.testing.assert_allclose(master, w64, rtol=0, atol=2e-6 * np.abs(w64).max())
    w0f = synth.bf16_bits_to_f32(w0)
    moved = np.abs(master - w0f) > 0
    assert moved.mean() > 0.99
    # without the master copy, weights with |w| >= 2^-5 (half a bf16 ulp
    # >= 1.2e-4 > lr) stay where they are
    big = np.abs(w0f) >= 2.0 ** -5
    assert big.sum() > 100 and (w_plain[big] == w0[big]).mean() > 0.9 and moved[big].all()


@pytest.mark.parametrize("n", [2, 3, 4])
def test_identical_micro_batches_equal_one_batch(n):
    """n micro-batches with the same tokens: the accumulated mean is exactly
    the single micro-batch's bf16 gradient (n * g is exact in fp32, its
    division by n correctly rounded), so the step is bit-identical."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    for master in (False, True):
        a = oracle.HostState(bits, master=master)
        b = oracle.HostState(bits, master=master)
        for step in range(2):
            tk = synth.make_tokens(cfg, step)
            ra = oracle.train_step(a, [tk] * n, cfg, adam)
            rb = oracle.train_step(b, tk, cfg, adam)
            assert ra["loss"] == rb["loss"]
        for l in range(cfg.layers):
            for k in a.bits["layers"][l]:
                assert np.array_equal(a.bits["layers"][l][k], b.bits["layers"][l][k])
                assert np.array_equal(a.m["layers"][l][k], b.m["layers"][l][k])
                assert np.array_equal(a.v["layers"][l][k], b.v["layers"][l][k])
        for k in ("embed", "head", "g_final"):
            assert np.array_equal(a.bits[k], b.bits[k]) and np.array_equal(a.v[k], b.v[k])


def test_micro_batch_mean_is_the_full_batch_gradient():
    """In fp64 without the bf16 storage roundings, the mean of the
    micro-batches' gradients is the gradient of the loss over all of their
    rows as one batch (every micro-batch has the same number of labelled
    positions), and the mean of their losses is that loss."""
    import dataclasses
    cfg = synth.preset("tiny")
    rng = np.random.default_rng(12)
    Wf = _rand_weights(cfg, rng)
    micro = [synth.make_tokens(cfg, s) for s in range(3)]
    full_cfg = dataclasses.replace(cfg, batch=3 * cfg.batch)
    loss_f, _, g_full, _ = oracle.forward_backward(Wf, np.concatenate(micro, axis=0), full_cfg)
    outs = [oracle.forward_backward(Wf, tk, cfg) for tk in micro]
    assert abs(np.mean([o[0] for o in outs]) - loss_f) <= 1e-13 * abs(loss_f)
    for name, layer, _ in _flat_items(Wf):
        mean = sum(_grad_of(o[2], name, layer) for o in outs) / 3
        ref = _grad_of(g_full, name, layer)
        assert np.abs(mean - ref).max() <= 1e-12 * np.abs(ref).max(), (name, layer)


def test_streamed_equals_resident_with_micro_batches_and_master():
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    a = oracle.HostState(bits, master=True)
    b = oracle.HostState(bits, master=True)
    for step in range(2):
        mb = [synth.make_tokens(cfg, 2 * step), synth.make_tokens(cfg, 2 * step + 1)]
        ra = oracle.train_step(a, mb, cfg, adam, mode="resident")
        rb = oracle.train_step(b, mb, cfg, adam, mode="streamed", ckpt_every=1)
        assert ra["loss"] == rb["loss"]
    for l in range(cfg.layers):
        for k in a.bits["layers"][l]:
            assert np.array_equal(a.master["layers"][l][k], b.master["layers"][l][k])
            assert np.array_equal(a.m["layers"][l][k], b.m["layers"][l][k])


# ----------------------------------------------------------------------------
# invariants of the method
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("K", [1, 2])
def test_streamed_equals_resident_bitwise(K):
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    tok = synth.make_tokens(cfg)
    adam = synth.AdamCfg()
    a = oracle.HostState(bits)
    b = oracle.HostState(bits)
    for step in range(2):
        tk = synth.make_tokens(cfg, step)
        ra = oracle.train_step(a, tk, cfg, adam, mode="resident")
        rb = oracle.train_step(b, tk, cfg, adam, mode="streamed", ckpt_every=K)
        assert ra["loss"] == rb["loss"]
    for l in range(cfg.layers):
        for k in a.bits["layers"][l]:
            assert np.array_equal(a.bits["layers"][l][k], b.bits["layers"][l][k])
            assert np.array_equal(a.m["layers"][l][k], b.m["layers"][l][k])
            assert np.array_equal(a.v["layers"][l][k], b.v["layers"][l][k])
    for k in ("embed", "head", "g_final"):
        assert np.array_equal(a.bits[k], b.bits[k])


def test_causality_of_per_position_loss():
    cfg = synth.preset("micro")
    rng = np.random.default_rng(10)
    W = _rand_weights(cfg, rng)
    tok = synth.make_tokens(cfg)
    s = 5
    tok2 = tok.copy()
    tok2[:, s + 2:] = (tok2[:, s + 2:] + 13) % cfg.vocab
    _, p1, _, _ = oracle.forward_backward(W, tok, cfg)
    _, p2, _, _ = oracle.forward_backward(W, tok2, cfg)
    assert np.array_equal(p1[:, : s + 1], p2[:, : s + 1])
    assert not np.array_equal(p1[:, s + 1:], p2[:, s + 1:])


def test_init_loss_sanity_band():
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    loss, _, _, _ = oracle.forward_backward(oracle.to_float(bits, np.float32), synth.make_tokens(cfg), cfg)
    centre = math.log(cfg.vocab) + 2e-4 * cfg.hidden
    assert abs(loss - centre) < 0.05


# ----------------------------------------------------------------------------
# golden values
# ----------------------------------------------------------------------------

def _read_golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_splitmix64_published_outputs():
    for n, hexval in _read_golden("splitmix64_seed0.txt"):
        assert int(synth.u64(0, 0, np.array([int(n)]))[0]) == int(hexval, 16)


def test_tokens_and_normals_properties():
    toks = synth.tokens(0, 1000, 4, 4096)
    assert toks.min() >= 0 and toks.max() < 1000
    counts = np.bincount(toks.reshape(-1), minlength=1000)
    assert counts.min() > 0
    w = synth.bf16_bits_to_f32(synth.normal_bf16_bits(0, 17, 1 << 18))
    assert abs(w.mean()) < 1e-3 and abs(w.std() - 0.02) < 2e-4
    # element i does not depend on how the tensor is chunked
    part = synth.normal_bf16_bits(0, 17, 1000, start=5000)
    assert np.array_equal(part, synth.normal_bf16_bits(0, 17, 6000)[5000:])


# ----------------------------------------------------------------------------
# the long-context layer mode: layer_rows equals the plain layer
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [7, 64])
def test_layer_rows_equals_plain_layer(chunk):
    """layer_rows (per-token work in token chunks, attention per head and
    query block, dy nonzero on a few row blocks only) reaches the plain
    layer_fwd / layer_bwd result with the same dy, in fp64: y on the
    blocks, dx on every row and every weight gradient; the sampled form
    (dx on some row ranges, chosen QKV gradient rows) gives the same
    entries.  A plausible slip in it (a missed key range, a block's dq on the
    wrong rows, RoPE of dk skipped or the wrong way, a chunk boundary
    dropped) changes some of these by far more than rounding."""
    cfg = synth.preset("micro", batch=1, seq=41, layers=1)
    rng = np.random.default_rng(5)
    W = _rand_weights(cfg, rng)["layers"][0]
    S, h = cfg.seq, cfg.hidden
    x = rng.standard_normal((S, h))
    blocks = [(0, 5), (17, 23), (36, 41)]
    dy = np.zeros((S, h))
    for a, b in blocks:
        dy[a:b] = rng.standard_normal((b - a, h))
    cos, sin = oracle.rope_tables(S, cfg.head_dim, cfg.rope_base)
    y_ref, cache = oracle.layer_fwd(x, W, cfg, cos, sin)
    dx_ref, dW_ref = oracle.layer_bwd(dy, cache, W, cfg, cos, sin)

    def close(a, b):
        assert np.abs(a - b).max() <= 1e-11 * max(1.0, np.abs(b).max())

    r = oracle.layer_rows(x, W, cfg, cos, sin, blocks, [dy[a:b] for a, b in blocks], chunk=chunk)
    for (a, b), yb in zip(blocks, r["y"]):
        close(yb, y_ref[a:b])
    close(r["dx"], dx_ref)
    for name, g in dW_ref.items():
        close(r["dW"][name], g)
    # dk and dv reach rows outside the blocks: dx there is not just the residual
    assert np.abs(dx_ref[6:17]).max() > 1e-3

    sel = [1, h + 3, 2 * h + 60, 3 * h - 1]
    dxb = [(2, 9), (30, 41)]
    r2 = oracle.layer_rows(x, W, cfg, cos, sin, blocks, [dy[a:b] for a, b in blocks], dx_blocks=dxb,
                           wqkv_rows=sel, chunk=chunk)
    for (a, b), d in zip(dxb, r2["dx"]):
        close(d, dx_ref[a:b])
    close(r2["dW"]["wqkv"], dW_ref["wqkv"][sel])
    assert r2["dW"]["g_attn"] is None
    for name in ("wo", "wgu", "wd", "g_mlp"):
        close(r2["dW"][name], dW_ref[name])
