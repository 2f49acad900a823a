"""Model shapes, optimizer settings and seeded weight/token construction.

Shapes follow the workloads the method is measured on (a tiny decoder, 7B- and
14B-shaped dense decoders, a depth and a width stress, and long-context 7B
layer shapes).  Architecture reading: Llama-style pre-norm decoder, fused QKV
[3h, h], output projection [h, h], fused gate/up [2f, h] (gate rows first),
down projection [h, f], untied embedding [V, h] and LM head [V, h], RMSNorm
gains initialised to 1, matrices ~N(0, 0.02).
"""
from dataclasses import dataclass, replace

import numpy as np

from .gen import normal_bf16_bits, tokens as _tokens

STREAM_TOKENS = 0
STREAM_EMBED = 1
STREAM_FINAL_NORM = 2
STREAM_HEAD = 3
BF16_ONE = 0x3F80
LAYER_TENSORS = ("g_attn", "wqkv", "wo", "g_mlp", "wgu", "wd")


def layer_stream(layer, j):
    return 16 + 8 * layer + j


@dataclass(frozen=True)
class ModelCfg:
    name: str
    layers: int
    hidden: int
    heads: int
    head_dim: int
    ffn: int
    vocab: int
    batch: int
    seq: int
    ckpt_every: int = 1
    eps: float = 1e-5
    rope_base: float = 10000.0
    seed: int = 0
    tied: bool = False  # LM head = embedding matrix

    @property
    def tokens(self):
        return self.batch * self.seq

    def with_(self, **kw):
        return replace(self, **kw)


@dataclass(frozen=True)
class AdamCfg:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


PRESETS = {
    # Tiny decoder: one full training step is checked element by element.
    "tiny": ModelCfg("tiny", 2, 256, 4, 64, 688, 1024, 2, 128, ckpt_every=1),
    # 7B-shaped dense decoder, batch 4 x 2048.
    "7b": ModelCfg("7b", 32, 4096, 32, 128, 11008, 32000, 4, 2048, ckpt_every=4),
    # 14B-shaped dense decoder, batch 8 x 1024.
    "14b": ModelCfg("14b", 48, 5120, 40, 128, 13824, 32000, 8, 1024, ckpt_every=4),
    # Depth stress: 180 narrow layers.
    "depth180": ModelCfg("depth180", 180, 2048, 16, 128, 5504, 32000, 4, 2048, ckpt_every=4),
    # Width stress: 24 layers at 5x width.
    "width5x": ModelCfg("width5x", 24, 10240, 80, 128, 27648, 32000, 2, 1024, ckpt_every=4),
    # Long-context 7B layer shapes, 4 layers, batch 1.
    "lc128k": ModelCfg("lc128k", 4, 4096, 32, 128, 11008, 32000, 1, 131072, ckpt_every=1),
    "lc256k": ModelCfg("lc256k", 4, 4096, 32, 128, 11008, 32000, 1, 262144, ckpt_every=1),
    "lc512k": ModelCfg("lc512k", 4, 4096, 32, 128, 11008, 32000, 1, 524288, ckpt_every=1),
    # Small shape used for finite-difference pins of the oracle (fp64).
    "micro": ModelCfg("micro", 2, 64, 2, 32, 96, 97, 2, 12, ckpt_every=1),
}


def preset(name, **overrides):
    cfg = PRESETS[name]
    return cfg.with_(**overrides) if overrides else cfg


def layer_tensor_shapes(cfg):
    h, f = cfg.hidden, cfg.ffn
    return {"g_attn": (h,), "wqkv": (3 * h, h), "wo": (h, h), "g_mlp": (h,),
            "wgu": (2 * f, h), "wd": (h, f)}


def make_layer_weights(cfg, layer, std=0.02):
    """Dict of bf16 bit arrays (uint16) for one layer, in tensor order."""
    out = {}
    for j, (name, shape) in enumerate(layer_tensor_shapes(cfg).items()):
        n = int(np.prod(shape))
        if name.startswith("g_"):
            out[name] = np.full(shape, BF16_ONE, dtype=np.uint16)
        else:
            out[name] = normal_bf16_bits(cfg.seed, layer_stream(layer, j), n, std).reshape(shape)
    return out


def make_weights(cfg, std=0.02):
    """All weights of the model as bf16 bit arrays (no separate LM head when
    the embedding is tied to it)."""
    h, V = cfg.hidden, cfg.vocab
    return {
        "embed": normal_bf16_bits(cfg.seed, STREAM_EMBED, V * h, std).reshape(V, h),
        "g_final": np.full((h,), BF16_ONE, dtype=np.uint16),
        "head": None if getattr(cfg, "tied", False) else normal_bf16_bits(cfg.seed, STREAM_HEAD, V * h, std).reshape(V, h),
        "layers": [make_layer_weights(cfg, l, std) for l in range(cfg.layers)],
    }


def make_tokens(cfg, step=0):
    return _tokens(cfg.seed, cfg.vocab, cfg.batch, cfg.seq, step)
