"""GPU parity of full training steps (engine + C ABI) against the oracle, and
the method's invariants on the GPU: streamed == resident bit for bit, and the
checkpoint interval and slot count change nothing."""
import numpy as np
import pytest

import oracle
import synth
from host_memory_centric_amd.store import REGION_G, REGION_M, REGION_V, REGION_W

from parity import check_step, snapshot_weights, sync_from_oracle

pytestmark = pytest.mark.gpu


def _trainer(cfg, bits, **kw):
    from host_memory_centric_amd.engine import Trainer
    return Trainer(cfg, synth.AdamCfg(), weights=bits, capture_w32=True, **kw)


def _store_regions(tr):
    tr.finish()
    regions = (REGION_W, REGION_G, REGION_M, REGION_V) + ((4,) if tr.store.flags & 1 else ())
    return {(u, r): tr.store.region(u, r).copy() for u in tr.store.units for r in regions}


@pytest.mark.parametrize("mode,pinned,carry", [("streamed", False, 0), ("resident", False, 0), ("streamed", True, 0),
                                               ("streamed", True, 1)])
def test_tiny_steps_match_oracle(gpu, mode, pinned, carry):
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    st = oracle.HostState(bits)
    tr = _trainer(cfg, bits, mode=mode, pinned_store=pinned, carry=carry)
    try:
        for step in range(2):
            tok = synth.make_tokens(cfg, step)
            loss = tr.step(tok)
            prev = snapshot_weights(st)
            res = oracle.train_step(st, tok, cfg, adam, mode="resident")
            check_step(tr, loss, res, cfg, w_prev=prev)
            # continue both from the oracle's state so the second step is
            # checked on identical inputs
            sync_from_oracle(tr, st, cfg)
    finally:
        tr.close()


def test_streamed_equals_resident_bitwise(gpu):
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    runs = {}
    for name, kw in {"resident": dict(mode="resident"), "k1_2slot": dict(ckpt_every=1, n_slots=2),
                     "k2_2slot": dict(ckpt_every=2, n_slots=2), "k1_3slot": dict(ckpt_every=1, n_slots=3),
                     "k1_1slab": dict(ckpt_every=1, n_grad_slabs=1), "k1_1slot": dict(ckpt_every=1, n_slots=1),
                     "k2_2slot_urgent": dict(ckpt_every=2, n_slots=2, update_order="urgent"),
                     "k2_2slot_tail": dict(ckpt_every=2, n_slots=2, update_order="tail"),
                     "k1_2slot_pinned_carry1": dict(ckpt_every=1, n_slots=2, pinned_store=True, carry=1),
                     "k2_1slot_pinned_carry2_tail": dict(ckpt_every=2, n_slots=1, pinned_store=True, carry=2,
                                                         update_order="tail"),
                     "k1_2slot_pinned_carry2_carried": dict(ckpt_every=1, n_slots=2, pinned_store=True, carry=2,
                                                            update_order="carried")}.items():
        tr = _trainer(cfg, bits, **kw)
        try:
            losses = [tr.step(synth.make_tokens(cfg, s)) for s in range(3)]
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    ref_losses, ref_regions = runs["resident"]
    for name, (losses, regions) in runs.items():
        assert losses == ref_losses, name
        for key, a in ref_regions.items():
            assert np.array_equal(regions[key], a), (name, key)


def test_chunked_mlp_step_matches_oracle_and_resident(gpu):
    """Above 32768 tokens per layer call the MLP runs in token chunks and its
    backward recomputes the chunk's RMSNorm, gate/up and SwiGLU (20 x 2048 =
    40960 tokens: one whole chunk and a ragged one of 8192).  Two streamed
    steps (K = 1, 2 slots) equal the resident steps bit for bit, and the
    streamed step matches the oracle's full-batch step."""
    cfg = synth.preset("tiny", batch=20, seq=2048)
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    runs = {}
    for name, kw in {"resident": dict(mode="resident"), "k1_2slot": dict(ckpt_every=1, n_slots=2)}.items():
        print(f"chunked MLP step: {name}", flush=True)
        tr = _trainer(cfg, bits, **kw)
        try:
            losses = [tr.step(synth.make_tokens(cfg, s)) for s in range(2)]
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    ref_losses, ref_regions = runs["resident"]
    losses, regions = runs["k1_2slot"]
    assert losses == ref_losses
    for key, a in ref_regions.items():
        assert np.array_equal(regions[key], a), key
    print("chunked MLP step: oracle", flush=True)
    st = oracle.HostState(bits)
    tr = _trainer(cfg, bits, ckpt_every=1, n_slots=2)
    try:
        tok = synth.make_tokens(cfg, 0)
        loss = tr.step(tok)
        prev = snapshot_weights(st)
        res = oracle.train_step(st, tok, cfg, adam, mode="resident")
        check_step(tr, loss, res, cfg, w_prev=prev)
    finally:
        tr.close()


def test_ragged_blocks_and_sequence(gpu):
    """Five layers (blocks of 2, 2, 1 and of 3, 2) at a sequence of 100
    (partial attention and GEMM tiles): every schedule gives the resident
    step's bits, and the streamed step matches the oracle."""
    cfg = synth.preset("tiny", layers=5, ckpt_every=2, seq=100)
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    runs = {}
    for name, kw in {"resident": dict(mode="resident"), "k2_2slot": dict(n_slots=2), "k2_3slot": dict(n_slots=3),
                     "k3_1slot": dict(ckpt_every=3, n_slots=1), "k3_4slot": dict(ckpt_every=3, n_slots=4)}.items():
        tr = _trainer(cfg, bits, **kw)
        try:
            losses = [tr.step(synth.make_tokens(cfg, s)) for s in range(2)]
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    ref_losses, ref_regions = runs["resident"]
    for name, (losses, regions) in runs.items():
        assert losses == ref_losses, name
        for key, a in ref_regions.items():
            assert np.array_equal(regions[key], a), (name, key)
    st = oracle.HostState(bits)
    tok = synth.make_tokens(cfg, 0)
    tr = _trainer(cfg, bits, n_slots=2)
    try:
        loss = tr.step(tok)
        prev = snapshot_weights(st)
        res = oracle.train_step(st, tok, cfg, adam, mode="resident")
        check_step(tr, loss, res, cfg, w_prev=prev)
    finally:
        tr.close()


def test_offloaded_checkpoints_bit_identical(gpu):
    """Block checkpoints held in host memory (the ring of two device buffers,
    copies out in the forward and back in the backward) give the bits of the
    step that keeps them all on the device: one layer per block with one, two
    and the most host blocks, blocks of two, micro-batches, and with the event
    timeline recorded."""
    cfg = synth.preset("tiny", layers=6, ckpt_every=1, seq=100)
    bits = synth.make_weights(cfg)
    runs = {}
    cases = {"k1": dict(), "k1_h1": dict(offload_ckpt=1), "k1_h2": dict(offload_ckpt=2, n_slots=3),
             "k1_h4": dict(offload_ckpt=4), "k1_h3_tl": dict(offload_ckpt=3, timeline=True),
             "k1_h2_pinned": dict(offload_ckpt=2, pinned_store=True),
             "k4": dict(ckpt_every=4), "k2_h1": dict(ckpt_every=2, offload_ckpt=1)}
    for name, kw in cases.items():
        tr = _trainer(cfg, bits, **kw)
        try:
            assert tr.n_host == kw.get("offload_ckpt", 0)
            losses = [tr.step(synth.make_tokens(cfg, s)) for s in range(3)]
            if "timeline" in kw:
                tl = tr.timeline()
                assert len(tl["d2h"]) >= cfg.layers + tr.n_host and len(tl["h2d"]) >= tr.n_host
                # every layer's update, and the moment each backward was seen to end
                assert sorted(u for k, u, _, _ in tl["host"] if k == "update" and 0 <= u < cfg.layers) \
                    == list(range(cfg.layers))
                assert sum(k == "bwd_done" for k, *_ in tl["host"]) == cfg.layers
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    ref_losses, ref_regions = runs["k1"]
    for name, (losses, regions) in runs.items():
        assert losses == ref_losses, name
        for key, a in ref_regions.items():
            assert np.array_equal(regions[key], a), (name, key)
    # ragged blocks (7 layers in blocks of 2, 2, 2, 1), two of them in host memory
    cfg7 = synth.preset("tiny", layers=7, ckpt_every=2, seq=100)
    bits7 = synth.make_weights(cfg7)
    r7 = {}
    for name, kw in {"k2": dict(), "k2_h2": dict(offload_ckpt=2)}.items():
        tr = _trainer(cfg7, bits7, **kw)
        try:
            r7[name] = ([tr.step(synth.make_tokens(cfg7, s)) for s in range(2)], _store_regions(tr))
        finally:
            tr.close()
    assert r7["k2"][0] == r7["k2_h2"][0]
    for key, a in r7["k2"][1].items():
        assert np.array_equal(r7["k2_h2"][1][key], a), key
    # micro-batches: two passes per step, each with its own copies out and back
    mb = {}
    for name, kw in {"mb": dict(), "mb_h3": dict(offload_ckpt=3)}.items():
        tr = _trainer(cfg, bits, micro_batches=2, **kw)
        try:
            losses = [tr.step(np.concatenate([synth.make_tokens(cfg, 2 * s + i) for i in range(2)]))
                      for s in range(2)]
            mb[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    assert mb["mb"][0] == mb["mb_h3"][0]
    for key, a in mb["mb"][1].items():
        assert np.array_equal(mb["mb_h3"][1][key], a), key


def test_run_twice_deterministic(gpu):
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    out = []
    for _ in range(2):
        tr = _trainer(cfg, bits)
        try:
            l = tr.step(synth.make_tokens(cfg, 0))
            tr.finish()
            out.append((l, tr.store.region(0, REGION_W).copy()))
        finally:
            tr.close()
    assert out[0][0] == out[1][0] and np.array_equal(out[0][1], out[1][1])


@pytest.mark.parametrize("mode", ["streamed", "resident"])
def test_micro_batches_with_master_match_oracle(gpu, mode):
    """Two micro-batches per step, gradients accumulated on the host, one
    Adam step on their mean over fp32 master weights, against the oracle."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    st = oracle.HostState(bits, master=True)
    tr = _trainer(cfg, bits, mode=mode, micro_batches=2, master=True)
    try:
        for step in range(2):
            mb = [synth.make_tokens(cfg, 2 * step), synth.make_tokens(cfg, 2 * step + 1)]
            loss = tr.step(np.concatenate(mb, axis=0))
            prev = snapshot_weights(st)
            res = oracle.train_step(st, mb, cfg, adam)
            check_step(tr, loss, res, cfg, w_prev=prev)
            for got, ref in zip(tr.stats["losses"], res["losses"]):
                assert abs(got - float(ref)) <= 1e-3 * abs(float(ref))
            sync_from_oracle(tr, st, cfg)
    finally:
        tr.close()


def test_micro_batches_streamed_equals_resident_and_repeats_equal_one(gpu):
    """With micro-batches and master weights the schedule still changes no
    bit (resident, K = 1 and K = 2, one slot); two identical micro-batches
    give exactly the one-micro-batch step (the mean of two equal bf16
    gradients is exact)."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    runs = {}
    for name, kw in {"resident": dict(mode="resident"), "k1_2slot": dict(ckpt_every=1, n_slots=2),
                     "k2_1slot": dict(ckpt_every=2, n_slots=1)}.items():
        tr = _trainer(cfg, bits, micro_batches=2, master=True, **kw)
        try:
            losses = [tr.step(np.concatenate([synth.make_tokens(cfg, 2 * s), synth.make_tokens(cfg, 2 * s + 1)]))
                      for s in range(2)]
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    ref_losses, ref_regions = runs["resident"]
    for name, (losses, regions) in runs.items():
        assert losses == ref_losses, name
        for key, a in ref_regions.items():
            assert np.array_equal(regions[key], a), (name, key)
    out = []
    for n in (1, 2):
        tr = _trainer(cfg, bits, micro_batches=n)
        try:
            for s in range(2):
                tk = synth.make_tokens(cfg, s)
                tr.step(np.concatenate([tk] * n))
            out.append(_store_regions(tr))
        finally:
            tr.close()
    for key, a in out[0].items():
        assert np.array_equal(out[1][key], a), key


def test_resume_from_checkpoint_is_bit_identical(gpu, tmp_path):
    """Three steps in one run equal one step, a checkpoint of the host store,
    a new trainer (whose own state is first moved by a step of its own) that
    loads it, and two more steps: losses and every store region bit for bit
    (two micro-batches and master weights, so every region is exercised)."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)

    def toks(s):
        return np.concatenate([synth.make_tokens(cfg, 2 * s), synth.make_tokens(cfg, 2 * s + 1)])

    kw = dict(micro_batches=2, master=True)
    a = _trainer(cfg, bits, **kw)
    try:
        la = [a.step(toks(s)) for s in range(3)]
        ra = _store_regions(a)
    finally:
        a.close()
    path = tmp_path / "run.ckpt"
    b = _trainer(cfg, bits, **kw)
    try:
        lb = [b.step(toks(0))]
        b.save(path)
    finally:
        b.close()
    c = _trainer(cfg, bits, **kw)
    try:
        c.step(toks(9))
        c.load(path)
        assert c.t == 1
        lb += [c.step(toks(s)) for s in (1, 2)]
        rc = _store_regions(c)
    finally:
        c.close()
    assert la == lb
    for key, x in ra.items():
        assert np.array_equal(rc[key], x), key


@pytest.mark.parametrize("kw", [dict(), dict(micro_batches=2, master=True)], ids=["plain", "micro2_master"])
def test_resumed_run_matches_oracle(gpu, tmp_path, kw):
    """A run checkpointed after its first step and resumed in a fresh trainer
    (whose own state is first moved by a step of its own, so only the loaded
    checkpoint can give the right state) matches the oracle's three steps:
    each GPU step starts from the oracle's state and is checked against the
    oracle's step at the parity bar, including the Adam step counter that
    the checkpoint carries (its bias corrections enter every update)."""
    cfg = synth.preset("tiny")
    bits = synth.make_weights(cfg)
    adam = synth.AdamCfg()
    n = kw.get("micro_batches", 1)
    st = oracle.HostState(bits, master=kw.get("master", False))

    def toks(s):
        mb = [synth.make_tokens(cfg, n * s + i) for i in range(n)]
        return np.concatenate(mb, axis=0), (mb if n > 1 else mb[0])

    path = tmp_path / "resume.ckpt"
    a = _trainer(cfg, bits, **kw)
    try:
        tk, otk = toks(0)
        loss = a.step(tk)
        prev = snapshot_weights(st)
        res = oracle.train_step(st, otk, cfg, adam)
        check_step(a, loss, res, cfg, w_prev=prev)
        sync_from_oracle(a, st, cfg)
        a.save(path)
    finally:
        a.close()
    b = _trainer(cfg, bits, **kw)
    try:
        b.step(toks(7)[0])  # a state of its own, overwritten by the load
        b.load(path)
        assert b.t == 1
        for s in (1, 2):
            tk, otk = toks(s)
            loss = b.step(tk)
            prev = snapshot_weights(st)
            res = oracle.train_step(st, otk, cfg, adam)
            check_step(b, loss, res, cfg, w_prev=prev)
            sync_from_oracle(b, st, cfg)
    finally:
        b.close()


def test_tied_embeddings_match_oracle_and_schedules_agree(gpu):
    """Weight tying on the tiny model: the head's slot carries the embedding
    matrix, its gradient is summed with the embedding's on the host, one
    Adam updates the shared matrix; against the oracle over two steps, and
    streamed (K = 1, 2 slots) == resident bit for bit."""
    import dataclasses
    cfg = dataclasses.replace(synth.preset("tiny"), tied=True)
    bits = synth.make_weights(cfg)
    assert bits["head"] is None
    adam = synth.AdamCfg()
    st = oracle.HostState(bits)
    tr = _trainer(cfg, bits)
    try:
        for step in range(2):
            tok = synth.make_tokens(cfg, step)
            loss = tr.step(tok)
            prev = snapshot_weights(st)
            res = oracle.train_step(st, tok, cfg, adam)
            check_step(tr, loss, res, cfg, w_prev=prev)
            sync_from_oracle(tr, st, cfg)
    finally:
        tr.close()
    runs = {}
    for name, kw in {"resident": dict(mode="resident"), "k1_2slot": dict(ckpt_every=1, n_slots=2)}.items():
        tr = _trainer(cfg, bits, **kw)
        try:
            losses = [tr.step(synth.make_tokens(cfg, s)) for s in range(3)]
            runs[name] = (losses, _store_regions(tr))
        finally:
            tr.close()
    assert runs["resident"][0] == runs["k1_2slot"][0]
    for key, a in runs["resident"][1].items():
        assert np.array_equal(runs["k1_2slot"][1][key], a), key


def test_carried_slots_across_resume_and_store_writes(gpu, tmp_path):
    """Carried layers keep device copies of their weights across steps; a
    checkpoint load or a direct write of the store must drop them.  A run
    with carried layers that is saved after one step and resumed in a
    trainer whose carried slots already hold other weights (it ran a step of
    its own) equals the uninterrupted run without carried layers, losses and
    every store region bit for bit; so does a run whose store is overwritten
    with the same run's state between steps."""
    cfg = synth.preset("tiny", layers=5)
    bits = synth.make_weights(cfg)
    kw = dict(ckpt_every=2, n_slots=2, pinned_store=True)
    ref = _trainer(cfg, bits, **kw)
    try:
        lref = [ref.step(synth.make_tokens(cfg, s)) for s in range(3)]
        rref = _store_regions(ref)
    finally:
        ref.close()
    path = tmp_path / "carry.ckpt"
    b = _trainer(cfg, bits, carry=3, **kw)
    try:
        lb = [b.step(synth.make_tokens(cfg, 0))]
        b.save(path)
        mid = _store_regions(b)
    finally:
        b.close()
    c = _trainer(cfg, bits, carry=3, **kw)
    try:
        c.step(synth.make_tokens(cfg, 9))
        c.step(synth.make_tokens(cfg, 8))
        c.load(path)
        lb += [c.step(synth.make_tokens(cfg, s)) for s in (1, 2)]
        rc = _store_regions(c)
    finally:
        c.close()
    assert lb == lref
    for key, a in rref.items():
        assert np.array_equal(rc[key], a), key
    # the same through direct writes of the store (weights, moments, counter)
    d = _trainer(cfg, bits, carry=3, **kw)
    try:
        d.step(synth.make_tokens(cfg, 9))
        d.step(synth.make_tokens(cfg, 8))
        d.finish()
        for (u, r), a in mid.items():
            d.store.region(u, r)[...] = a
        d.t = 1
        d.store_modified()
        ld = [lb[0]] + [d.step(synth.make_tokens(cfg, s)) for s in (1, 2)]
        rd = _store_regions(d)
    finally:
        d.close()
    assert ld == lref
    for key, a in rref.items():
        assert np.array_equal(rd[key], a), key


@pytest.mark.parametrize("variant", ["k1_2slot", "k2_1slot_micro_master", "tied_k1_2slot", "resident"])
def test_pinned_store_equals_pageable_bitwise(gpu, variant, tmp_path):
    """Copying weights straight from the page-locked W regions and gradients
    straight into G (no packer, no slabs) changes no bit: losses and every
    store region over three steps equal the pageable store's.  The
    checkpoint format is the same for both placements: a pinned run saved
    after one step and resumed in a pageable store continues identically."""
    import dataclasses
    cfg = synth.preset("tiny")
    kw = {"k1_2slot": dict(ckpt_every=1, n_slots=2),
          "k2_1slot_micro_master": dict(ckpt_every=2, n_slots=1, micro_batches=2, master=True),
          "tied_k1_2slot": dict(ckpt_every=1, n_slots=2),
          "resident": dict(mode="resident")}[variant]
    if variant.startswith("tied"):
        cfg = dataclasses.replace(cfg, tied=True)
    bits = synth.make_weights(cfg)
    n = kw.get("micro_batches", 1)

    def toks(s):
        return np.concatenate([synth.make_tokens(cfg, n * s + i) for i in range(n)])

    runs = {}
    for pinned in (False, True):
        tr = _trainer(cfg, bits, pinned_store=pinned, **kw)
        try:
            assert tr.direct == pinned and (not pinned or not tr.wslab and not tr.gslab)
            losses = [tr.step(toks(s)) for s in range(3)]
            runs[pinned] = (losses, _store_regions(tr))
        finally:
            tr.close()
    assert runs[True][0] == runs[False][0]
    for key, a in runs[False][1].items():
        assert np.array_equal(runs[True][1][key], a), key
    if variant != "k1_2slot":
        return
    path = tmp_path / "pinned.ckpt"
    b = _trainer(cfg, bits, pinned_store=True, **kw)
    try:
        lb = [b.step(toks(0))]
        b.save(path)
    finally:
        b.close()
    c = _trainer(cfg, bits, pinned_store=False, **kw)
    try:
        c.load(path)
        lb += [c.step(toks(s)) for s in (1, 2)]
        rc = _store_regions(c)
    finally:
        c.close()
    assert lb == runs[False][0]
    for key, a in runs[False][1].items():
        assert np.array_equal(rc[key], a), key
