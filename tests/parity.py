"""Parity metrics and tolerances of the training step against the oracle.

Tolerances (the target's stated bar): loss relative error <= 1e-3; every
gradient tensor max|g - g*| / max|g*| <= 2e-2 and cosine >= 0.9995; updated
fp32 weights per tensor ||w' - w'*|| / ||w'*|| <= 1e-3.
"""
import numpy as np

import synth
from host_memory_centric_amd._lib import MT_UNIT_EMBED, MT_UNIT_HEAD
from host_memory_centric_amd.store import REGION_G, tensor_shapes

LOSS_RTOL = 1e-3
GRAD_MAXREL = 2e-2
GRAD_COS = 0.9995
W_RTOL = 1e-3
# The update itself, w' - w, on the entries whose oracle gradient is at least
# DELTA_GRAD_FLOOR of the tensor's largest: there the gradient bar above
# (|g - g*| <= 2e-2 max|g*|) cannot flip the gradient's sign, so Adam's step
# (close to -lr * sign(g) at the first steps) must agree to DELTA_RTOL.  A
# missing, doubled or wrong-sign update of any tensor fails it, including the
# RMSNorm gains, whose updates (1e-4 of a weight of 1) the rel-L2 of w' hides.
DELTA_GRAD_FLOOR = 0.1
DELTA_RTOL = 1e-2


def grad_metrics(got, ref):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    scale = np.abs(ref).max()
    maxrel = np.abs(got - ref).max() / scale if scale > 0 else np.abs(got).max()
    den = np.linalg.norm(got) * np.linalg.norm(ref)
    cos = float(got @ ref / den) if den > 0 else (1.0 if not got.any() and not ref.any() else 0.0)
    return float(maxrel), cos


def rel_l2(got, ref):
    got = np.asarray(got, np.float64).reshape(-1)
    ref = np.asarray(ref, np.float64).reshape(-1)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def unit_tensors(cfg, unit):
    names = [n for n, _ in tensor_shapes(cfg, unit)]
    return names


def oracle_grad(res, unit, name):
    if unit == MT_UNIT_EMBED:
        return res["grads"]["embed"]
    if unit == MT_UNIT_HEAD:
        return res["grads"][name]
    return res["grads"]["layers"][unit][name]


def oracle_w32(res, unit, name):
    if unit == MT_UNIT_EMBED:
        return res["w_fp32"]["embed"]
    if unit == MT_UNIT_HEAD:
        return res["w_fp32"][name]
    return res["w_fp32"]["layers"][unit][name]


def snapshot_weights(state):
    """The oracle state's weights as the next update reads them, per
    (unit, tensor name): the fp32 master copy if it keeps one, else the bf16
    weights widened.  Taken before oracle.train_step to check updates."""
    out = {}
    ms = state.master
    for name in ("embed", "g_final", "head"):
        if state.bits.get(name) is None:
            continue
        unit = MT_UNIT_EMBED if name == "embed" else MT_UNIT_HEAD
        src = ms[name] if ms is not None else synth.bf16_bits_to_f32(state.bits[name])
        out[(unit, name)] = np.array(src, dtype=np.float32)
    for l, lw in enumerate(state.bits["layers"]):
        for name, a in lw.items():
            src = ms["layers"][l][name] if ms is not None else synth.bf16_bits_to_f32(a)
            out[(l, name)] = np.array(src, dtype=np.float32)
    return out


def _state_key(unit, name):
    return (unit, "embed" if unit == MT_UNIT_EMBED else name)


def check_step(trainer, loss, res, cfg, report=None, w_prev=None):
    """Assert the trainer's step matches the oracle result ``res``.  With
    ``w_prev`` (snapshot_weights of the oracle state before its step, which
    the trainer's step started from too) the updates w' - w are checked as
    well (DELTA_* above)."""
    trainer.finish()  # the host updates of the step have landed
    rep = {"loss_rel": abs(loss - float(res["loss"])) / abs(float(res["loss"]))}
    assert rep["loss_rel"] <= LOSS_RTOL, rep
    worst = (0.0, 1.0, 0.0)
    worst_delta = 0.0
    for unit in trainer.store.units:
        lay = trainer.store.layout_of(unit)
        for j, (name, shape) in enumerate(tensor_shapes(cfg, unit)):
            g = synth.bf16_bits_to_f32(trainer.store.tensor(unit, name, REGION_G))
            mr, cos = grad_metrics(g, oracle_grad(res, unit, name))
            assert mr <= GRAD_MAXREL and cos >= GRAD_COS, (unit, name, mr, cos)
            w32 = trainer.w32[unit][lay.tensor_off[j] // 2: lay.tensor_off[j] // 2 + int(np.prod(shape))]
            w32_ref = oracle_w32(res, unit, name)
            wr = rel_l2(w32, w32_ref)
            assert wr <= W_RTOL, (unit, name, wr)
            worst = (max(worst[0], mr), min(worst[1], cos), max(worst[2], wr))
            if w_prev is not None:
                w0 = w_prev[_state_key(unit, name)].reshape(-1)
                gref = np.abs(np.asarray(oracle_grad(res, unit, name), np.float32)).reshape(-1)
                sel = gref >= DELTA_GRAD_FLOOR * gref.max()
                assert sel.any(), (unit, name)
                d_got = (w32.reshape(-1)[sel].astype(np.float64) - w0[sel])
                d_ref = (np.asarray(w32_ref, np.float32).reshape(-1)[sel].astype(np.float64) - w0[sel])
                dr = rel_l2(d_got, d_ref)
                assert dr <= DELTA_RTOL, (unit, name, "update", dr, int(sel.sum()))
                worst_delta = max(worst_delta, dr)
    rep.update(grad_maxrel=worst[0], grad_cos_min=worst[1], w_rel=worst[2])
    if w_prev is not None:
        rep["update_rel"] = worst_delta
    if report is not None:
        report.update(rep)
    return rep


def sync_from_oracle(trainer, state, cfg):
    """Copy the oracle's weights and moments into the trainer's host store so
    that the next step of both starts from identical state."""
    trainer.finish()
    from host_memory_centric_amd.store import REGION_M, REGION_V, REGION_W
    st = trainer.store
    for unit in st.units:
        for name, _ in tensor_shapes(cfg, unit):
            if unit == MT_UNIT_EMBED:
                src = (state.bits["embed"], state.m["embed"], state.v["embed"])
            elif unit == MT_UNIT_HEAD:
                src = (state.bits[name], state.m[name], state.v[name])
            else:
                src = (state.bits["layers"][unit][name], state.m["layers"][unit][name], state.v["layers"][unit][name])
            st.tensor(unit, name, REGION_W)[...] = src[0]
            st.tensor(unit, name, REGION_M)[...] = src[1]
            st.tensor(unit, name, REGION_V)[...] = src[2]
            if state.master is not None:
                from host_memory_centric_amd.store import REGION_P
                ms = state.master
                p = (ms["embed"] if unit == MT_UNIT_EMBED else ms[name] if unit == MT_UNIT_HEAD
                     else ms["layers"][unit][name])
                st.tensor(unit, name, REGION_P)[...] = p
    trainer.store_modified()
