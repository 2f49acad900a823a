"""Full training steps at the configurations' shapes against the oracle.

Each workload's model is cut to 2 layers but keeps its width, heads, FFN,
vocabulary (32000) and its full batch x sequence: the 7B shape (4 x 2048),
the 14B shape (8 x 1024), the depth-stress layer (hidden 2048, 4 x 2048)
and the width-stress layer (hidden 10240, ffn 27648, 2 x 1024).  One step
of the streamed trainer (checkpoint every layer, 2 device slots: every
layer re-streamed and recomputed in its backward) is checked against the
oracle's plain step at the parity bar -- loss, every gradient tensor, the
updated fp32 weights and the updates themselves -- and the resident run
(all layers on the device, internals kept, no recompute) must give the
streamed run's bits in every host region.
"""
import numpy as np
import pytest

import oracle
import synth
from host_memory_centric_amd.store import REGION_G, REGION_M, REGION_V, REGION_W

from parity import check_step, snapshot_weights

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _digest(tr):
    import xxhash
    tr.finish()
    return {(u, r): xxhash.xxh3_64_hexdigest(tr.store.region(u, r))
            for u in tr.store.units for r in (REGION_W, REGION_G, REGION_M, REGION_V)}


@pytest.mark.parametrize("name", ["depth180", "7b", "14b", "width5x"])
def test_config_step_matches_oracle(gpu, name):
    import time

    from host_memory_centric_amd.engine import Trainer
    t0 = time.time()
    cfg = synth.preset(name, layers=2, ckpt_every=1)
    adam = synth.AdamCfg()
    _log(f"config {name}: 2 layers, batch {cfg.batch} x seq {cfg.seq}, hidden {cfg.hidden}, vocab {cfg.vocab}")
    bits = synth.make_weights(cfg)
    tok = synth.make_tokens(cfg, 0)
    runs = {}
    for mode in ("streamed", "resident"):
        _log(f"  GPU {mode} step ({time.time() - t0:.0f} s)")
        tr = Trainer(cfg, adam, mode=mode, n_slots=2, weights=bits, capture_w32=(mode == "streamed"))
        try:
            loss = tr.step(tok)
            runs[mode] = (loss, _digest(tr))
            if mode == "streamed":
                _log(f"  oracle step ({time.time() - t0:.0f} s)")
                st = oracle.HostState(bits)
                prev = snapshot_weights(st)
                res = oracle.train_step(st, tok, cfg, adam)
                del st
                rep = check_step(tr, loss, res, cfg, w_prev=prev)
                _log(f"  parity: {rep}")
                del res, prev
        finally:
            tr.close()
    assert runs["streamed"][0] == runs["resident"][0]
    assert runs["streamed"][1] == runs["resident"][1]
    # the initial loss of a random model: ln V plus the logits' variance
    lnV = np.log(cfg.vocab)
    assert lnV - 0.1 < runs["streamed"][0] < lnV + 2e-4 * cfg.hidden + 0.1
    _log(f"  done ({time.time() - t0:.0f} s)")
