"""The schedule's ordering and the device footprint, on the GPU.

* Poison and delays: every buffer is filled with NaN as soon as the event
  that frees it fires (device weight slots after their last reader,
  device gradient slots after their evacuation, pinned staging buffers after
  the copy that read them, pinned gradient slabs after the update that
  consumed them), and the packer and optimizer threads sleep for random
  times before each job.  A read or write that the events (weights-ready,
  buffer-free, backward-done, copy completion) do not order would then see
  NaN or land late; with correct ordering every loss and every host region
  equals the clean run's bit for bit.
* Footprint: at a fixed width the streamed step's device peak does not grow
  with depth except by the one [T, h] bf16 block checkpoint per block.
"""
import numpy as np
import pytest

import synth
from host_memory_centric_amd.store import REGION_G, REGION_M, REGION_V, REGION_W

pytestmark = pytest.mark.gpu


def _regions(tr):
    tr.finish()
    regions = (REGION_W, REGION_G, REGION_M, REGION_V) + ((4,) if tr.store.flags & 1 else ())
    return {(u, r): tr.store.region(u, r).copy() for u in tr.store.units for r in regions}


def _run(cfg, bits, steps, **kw):
    from host_memory_centric_amd.engine import Trainer
    n = kw.get("micro_batches", 1)
    tr = Trainer(cfg, synth.AdamCfg(), weights=bits, **kw)
    try:
        losses = [tr.step(np.concatenate([synth.make_tokens(cfg, n * s + i) for i in range(n)])) for s in range(steps)]
        regions = _regions(tr)
        if kw.get("poison"):
            # the poison did run: each device gradient slot was filled after its last
            # evacuation, and (with slabs) every recycled gradient slab after its update
            import torch
            torch.cuda.synchronize()
            for g in tr.gslots:
                for off, nb in tr._tensor_ranges(tr.lay):
                    assert bool((g[off:off + nb] == 0xFF).all())
            off, nb = tr._tensor_ranges(tr.lay)[1]
            poisoned = [bool((slab.view(np.uint8, tr.lay.w_bytes)[off:off + nb] == 0xFF).all()) for slab in tr.gslab]
            assert not tr.gslab or any(poisoned)
        return losses, regions
    finally:
        tr.close()


VARIANTS = {"k1_2slot": dict(ckpt_every=1, n_slots=2),
            "k2_1slot": dict(ckpt_every=2, n_slots=1),
            "k2_3slot_1slab": dict(ckpt_every=2, n_slots=3, n_grad_slabs=1),
            "pinned_k1_2slot": dict(ckpt_every=1, n_slots=2, pinned_store=True),
            "micro_master_k1_2slot": dict(ckpt_every=1, n_slots=2, micro_batches=2, master=True),
            "tied_k2_2slot": dict(ckpt_every=2, n_slots=2),
            "pinned_carry3_k2_2slot": dict(ckpt_every=2, n_slots=2, pinned_store=True, carry=3),
            "pinned_carry5_k1_1slot_tail": dict(ckpt_every=1, n_slots=1, pinned_store=True, carry=5,
                                                update_order="tail"),
            "pinned_carry2_micro_urgent": dict(ckpt_every=2, n_slots=2, pinned_store=True, carry=2,
                                               micro_batches=2, update_order="urgent"),
            "gslots3_k1_3slot_1slab": dict(ckpt_every=1, n_slots=3, n_grad_slabs=1, grad_slots=3),
            "pinned_carry3_k2_2slot_carried": dict(ckpt_every=2, n_slots=2, pinned_store=True, carry=3,
                                                   update_order="carried")}


@pytest.mark.parametrize("variant", list(VARIANTS))
def test_poison_and_delays_change_no_bit(gpu, variant):
    import dataclasses
    kw = VARIANTS[variant]
    cfg = synth.preset("tiny", layers=5, seq=100)
    if variant.startswith("tied"):
        cfg = dataclasses.replace(cfg, tied=True)
    bits = synth.make_weights(cfg)
    ref_losses, ref = _run(cfg, bits, 3, **kw)
    assert all(np.isfinite(ref_losses))
    for seed in (1, 2):
        losses, regions = _run(cfg, bits, 3, poison=True, delay_seed=seed, **kw)
        assert losses == ref_losses, (variant, seed, losses, ref_losses)
        for key, a in ref.items():
            assert np.array_equal(regions[key], a), (variant, seed, key)


def test_carried_layers_change_no_bit(gpu):
    """Carried layers (slots of their own, refilled right after each update)
    and the update order change no bit: losses and every host region over
    three steps equal the plain streamed run's, also with micro-batches."""
    cfg = synth.preset("tiny", layers=5, seq=100)
    bits = synth.make_weights(cfg)
    for micro in (1, 2):
        base = dict(ckpt_every=2, n_slots=2, pinned_store=True, micro_batches=micro)
        ref_losses, ref = _run(cfg, bits, 3, **base)
        for extra in (dict(carry=1), dict(carry=3, update_order="tail"), dict(carry=5, n_slots=1),
                      dict(carry=4, update_order="urgent"), dict(grad_slots=1), dict(grad_slots=3, carry=2)):
            losses, regions = _run(cfg, bits, 3, **dict(base, **extra))
            assert losses == ref_losses, (micro, extra)
            for key, a in ref.items():
                assert np.array_equal(regions[key], a), (micro, extra, key)


@pytest.mark.parametrize("carry", [0, 4])
def test_device_peak_independent_of_depth(gpu, carry):
    """The 7B layer shape (hidden 4096, batch 4 x 2048) streamed with
    checkpoints every 4 layers and 2 slots (and, with carried layers, 4 more
    slots of their own), at 8 and at 16 layers: the device peak differs by
    exactly the two extra block checkpoints ([T, h] bf16, 64 MiB each); the
    weight slots, gradient slots, one block's internals and the workspace are
    sized per layer."""
    import torch

    from host_memory_centric_amd.engine import Trainer
    peaks = {}
    for L in (8, 16):
        cfg = synth.preset("7b", layers=L)
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        tr = Trainer(cfg, synth.AdamCfg(), n_slots=2, carry=carry, pinned_store=carry > 0)
        try:
            for s in range(2):  # (the second step runs from the carried slots)
                tr.step(synth.make_tokens(cfg, s))
            tr.finish()
            torch.cuda.synchronize()
            peaks[L] = torch.cuda.max_memory_allocated() - base
        finally:
            tr.close()
            del tr
    ckpt = 4 * 2048 * 4096 * 2
    blocks = {L: (L + 3) // 4 for L in peaks}
    print(f"device peaks: {peaks}, block checkpoint {ckpt} bytes", flush=True)
    assert peaks[16] - peaks[8] == (blocks[16] - blocks[8]) * ckpt, peaks


@pytest.mark.parametrize("fail_at", [3, 12])
def test_failed_pass_releases_the_copy_threads(gpu, fail_at):
    """An error raised while a pass is being enqueued (here: the bind of the
    fail_at-th op, a host-side error) propagates from step(); the weight-load
    and gradient-copy issuer threads, which wait for ops that will never be
    enqueued, are released, and close() returns.  A new trainer on the same
    weights then runs its steps normally (losses equal a clean run's)."""
    import threading

    from host_memory_centric_amd.engine import Trainer
    cfg = synth.preset("tiny", layers=5, seq=100)
    bits = synth.make_weights(cfg)
    kw = dict(ckpt_every=2, n_slots=2, pinned_store=True, carry=2)
    tr = Trainer(cfg, synth.AdamCfg(), weights=bits, **kw)
    calls = [0]
    bind = tr._bind

    def failing_bind(*a):
        calls[0] += 1
        if calls[0] == fail_at:
            raise RuntimeError("planted host-side error")
        return bind(*a)
    tr._bind = failing_bind
    with pytest.raises(RuntimeError, match="planted"):
        tr.step(synth.make_tokens(cfg, 0))
    done = threading.Event()
    th = threading.Thread(target=lambda: (tr.close(), done.set()), daemon=True)
    th.start()
    assert done.wait(60), "close() did not return after a failed pass"
    ref_losses, _ = _run(cfg, bits, 2, **kw)
    losses, _ = _run(cfg, bits, 2, **kw)
    assert losses == ref_losses and all(np.isfinite(losses))
