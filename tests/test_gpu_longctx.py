"""One layer at the long-context shapes (batch 1 x 131072 and x 524288
tokens, the 7B layer) against the oracle, through the same entry points,
shapes and workspaces as a training step.

The output gradient is zero outside three row blocks (the first, a middle
and the last 128 positions).  Then the oracle's long-context mode
(oracle.layer_rows: per-token work in token chunks, attention exact per
head and query block) computes the exact layer result from those rows'
softmax rows alone, while the GPU runs the full layer unaware of it: its
forward over all rows, the attention backward whose dK and dV reach every
key, RoPE at every position (the last block sits at positions >= 130944 and
>= 524160), and every weight gradient as a reduction over all tokens.

* 131072 tokens: y on the blocks, dx on every row, every weight and gain
  gradient;
* 524288 tokens: y on the blocks, dx on the blocks and on two more row
  ranges, the output-projection, MLP and MLP-gain gradients whole, and
  twelve rows of the QKV weight gradient (each a sum over all 524288 tokens).
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import metrics
from layer_run import run_layer
from parity import GRAD_COS, GRAD_MAXREL

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _check(name, got, ref, fails):
    mar, cos = metrics(got, ref)
    ok = mar <= GRAD_MAXREL and cos >= GRAD_COS
    _log(f"  {name}: max-abs-rel {mar:.3e} cos {cos:.7f}{'' if ok else '  FAIL'}")
    if not ok:
        fails.append((name, mar, cos))


@pytest.mark.parametrize("name,sampled", [("lc128k", False), ("lc512k", True)])
def test_long_context_layer_vs_oracle(gpu, name, sampled):
    import time

    import torch
    cfg = synth.preset(name)
    S, h = cfg.seq, cfg.hidden
    assert cfg.batch == 1
    t0 = time.time()
    _log(f"long-context layer {name}: S={S} inputs")
    W = {}
    for j, (nm, shape) in enumerate(synth.layer_tensor_shapes(cfg).items()):
        W[nm] = (synth.torch_normal_bf16_bits(300 + j, shape, std=0.1, mean=1.0) if nm.startswith("g_")
                 else synth.torch_normal_bf16_bits(300 + j, shape, std=0.02))
    x = synth.torch_normal_bf16_bits(310, (S, h), std=1.0)
    R = 128
    blocks = [(0, R), (S // 2 - R // 2, S // 2 + R // 2), (S - R, S)]
    dy_blocks = [synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(320 + i, (R, h), std=1.0))
                 for i in range(len(blocks))]
    dy = torch.zeros((S, h), dtype=torch.float32, device=gpu)
    for (a, b), d in zip(blocks, dy_blocks):
        dy[a:b] = torch.from_numpy(d).to(gpu)

    _log(f"  GPU layer forward + recompute-backward ({time.time() - t0:.0f} s)")
    d_y, d_dx, g_gpu = run_layer(gpu, cfg, W, x, dy)
    y_gpu = [d_y[a:b].view(torch.bfloat16).float().cpu().numpy() for a, b in blocks]
    dx_blocks = None
    if sampled:
        dx_blocks = blocks + [(S // 4, S // 4 + R), (3 * S // 4 - R // 2, 3 * S // 4 + R // 2)]
        dx_gpu = [d_dx[a:b].cpu().numpy() for a, b in dx_blocks]
    else:
        dx_gpu = d_dx.cpu().numpy()
    del d_y, d_dx, dy
    torch.cuda.empty_cache()

    _log(f"  oracle ({time.time() - t0:.0f} s)")
    xf = synth.bf16_bits_to_f32(x)
    Wf = {n: synth.bf16_bits_to_f32(a) for n, a in W.items()}
    cos, sin = oracle.rope_tables(S, cfg.head_dim, cfg.rope_base)
    sel = None
    if sampled:
        sel = [0, 129, 2047, h - 1, h, h + 1000, h + 3001, 2 * h - 1, 2 * h + 5, 2 * h + 2000, 2 * h + 4000, 3 * h - 1]
    ref = oracle.layer_rows(xf, Wf, cfg, cos, sin, blocks, dy_blocks, dx_blocks=dx_blocks, wqkv_rows=sel)
    _log(f"  compare ({time.time() - t0:.0f} s)")

    fails = []
    yg, yr = np.concatenate(y_gpu), np.concatenate(ref["y"])
    xb = np.concatenate([xf[a:b] for a, b in blocks])
    _check("y (blocks)", yg, yr, fails)
    _check("y - x (blocks)", yg - xb, yr - xb, fails)
    if sampled:
        dg, dr = np.concatenate(dx_gpu), np.concatenate(ref["dx"])
        _check("dx (sampled rows)", dg, dr, fails)
    else:
        dyf = np.zeros_like(xf)
        for (a, b), d in zip(blocks, dy_blocks):
            dyf[a:b] = d
        _check("dx", dx_gpu, ref["dx"], fails)
        _check("dx - dy", dx_gpu - dyf, ref["dx"] - dyf, fails)
        # rows outside the blocks get their gradient only through the keys and values
        outside = np.ones(S, bool)
        for a, b in blocks:
            outside[a:b] = False
        _check("dx (rows outside the blocks)", dx_gpu[outside], ref["dx"][outside], fails)
    for n, g in g_gpu.items():
        r = ref["dW"][n]
        if r is None:
            continue
        got = g[sel] if (n == "wqkv" and sel is not None) else g
        _check("d" + n + (" (sampled rows)" if n == "wqkv" and sel is not None else ""), got, r, fails)
    _log(f"  done ({time.time() - t0:.0f} s)")
    assert not fails, fails
