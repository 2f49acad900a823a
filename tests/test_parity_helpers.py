"""The parity checker itself (CPU): a trainer state written from the
oracle's own step passes check_step, and planted mistakes in the update --
a wrong-sign, missing or doubled update of one tensor, the RMSNorm gains
included -- fail it, although each leaves the updated weights within the
rel-L2 bar of w'."""
import numpy as np
import pytest

import oracle
import synth
from host_memory_centric_amd.store import REGION_G, HostStore, tensor_shapes

from parity import check_step, oracle_grad, oracle_w32, snapshot_weights


class _FakeTrainer:
    """The parts of Trainer that check_step reads, filled from the oracle."""

    def __init__(self, cfg, res):
        self.store = HostStore(cfg)
        self.w32 = {}
        for unit in self.store.units:
            lay = self.store.layout_of(unit)
            w = np.zeros(lay.w_bytes // 2, np.float32)
            for j, (name, shape) in enumerate(tensor_shapes(cfg, unit)):
                g = np.asarray(oracle_grad(res, unit, name), np.float32)
                self.store.tensor(unit, name, REGION_G)[...] = synth.f32_to_bf16_bits(g)
                off = lay.tensor_off[j] // 2
                w[off:off + int(np.prod(shape))] = np.asarray(oracle_w32(res, unit, name), np.float32).reshape(-1)
            self.w32[unit] = w

    def finish(self):
        pass

    def tensor_w32(self, unit, name, cfg):
        lay = self.store.layout_of(unit)
        for j, (nm, shape) in enumerate(tensor_shapes(cfg, unit)):
            if nm == name:
                off = lay.tensor_off[j] // 2
                return self.w32[unit][off:off + int(np.prod(shape))]
        raise KeyError(name)


@pytest.fixture(scope="module")
def step():
    cfg = synth.preset("tiny", layers=1)
    st = oracle.HostState(synth.make_weights(cfg))
    prev = snapshot_weights(st)
    tok = synth.make_tokens(cfg, 0)
    res = oracle.train_step(st, tok, cfg, synth.AdamCfg())
    return cfg, prev, res


def test_oracle_state_passes(step):
    cfg, prev, res = step
    tr = _FakeTrainer(cfg, res)
    rep = check_step(tr, float(res["loss"]), res, cfg, w_prev=prev)
    assert rep["update_rel"] < 1e-6 and rep["w_rel"] < 1e-7


@pytest.mark.parametrize("unit,name", [(0, "g_attn"), (0, "wqkv"), (-2, "g_final"), (0, "g_mlp")])
@pytest.mark.parametrize("kind", ["flip", "missing", "double"])
def test_planted_update_mistakes_fail(step, unit, name, kind):
    cfg, prev, res = step
    tr = _FakeTrainer(cfg, res)
    w = tr.tensor_w32(unit, name, cfg)
    w0 = prev[(unit, name)].reshape(-1)
    d = w - w0
    w[...] = {"flip": w0 - d, "missing": w0, "double": w0 + 2 * d}[kind]
    with pytest.raises(AssertionError) as e:
        check_step(tr, float(res["loss"]), res, cfg, w_prev=prev)
    if name.startswith("g_"):  # caught by the update check; the weights alone would have passed
        assert "update" in str(e.value)
        check_step(tr, float(res["loss"]), res, cfg)
