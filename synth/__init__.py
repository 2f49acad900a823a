"""Seeded synthetic inputs shared by the oracle and the GPU path.

This module holds model shapes, training hyper-parameters and a counter-based
random generator.  It contains none of the training arithmetic: it only turns
(seed, stream, index) into numbers.  Both the CPU oracle and the HIP path read
their weights and tokens from here (or, for the HIP library's bulk filler, from
an independent implementation of the same published generator that a test
checks bit for bit against this one).

Generator (SplitMix64 of Steele, Lea and Flood, OOPSLA 2014, used in counter
form):  ``u(key) = mix64(key * 0x9E3779B97F4A7C15)`` with SplitMix64's output
mix, ``key = seed << 48 | stream << 32 | i``.

* Normal weights ~N(0, 0.02): Box-Muller on the pair (u(2i), u(2i+1)) in fp64,
  ``u1 = ((u(2i) >> 11) + 1) * 2**-53`` in (0, 1], ``u2 = (u(2i+1) >> 11) * 2**-53``,
  ``z = sqrt(-2 ln u1) * cos(2 pi u2)``, stored as bf16(fp32(0.02 z)), both
  roundings to nearest-even.
* Tokens uniform in [0, V): ``tok = (u(i) * V) >> 64`` (multiply-high,
  Lemire 2019).  Training step n uses ``i = n*T + b*S + s``.
* Streams: tokens 0, embedding 1, final-norm gain 2, LM head 3, layer l
  tensor j = 16 + 8 l + j, tensor order (gain_attn, Wqkv, Wo, gain_mlp, Wgu,
  Wd).  RMSNorm gains are 1 and are not drawn.

Full-size kernel tests (hundreds of millions of elements) draw their inputs
from torch's seeded CPU generator instead (``torch_normal_bf16_bits``,
``torch_int_bf16_bits``): same bits on both sides, much faster than numpy.
"""
from .gen import (mix64, u64, normal_bf16_bits, tokens, bf16_bits_to_f32,
                  f32_to_bf16_bits, uniform_int_bf16_bits, torch_normal_bf16_bits, torch_int_bf16_bits,
                  torch_normal_bf16_device, torch_int_bf16_device)
from .configs import ModelCfg, AdamCfg, PRESETS, preset, layer_tensor_shapes, STREAM_TOKENS, \
    STREAM_EMBED, STREAM_FINAL_NORM, STREAM_HEAD, layer_stream, make_weights, make_layer_weights, make_tokens, LAYER_TENSORS, BF16_ONE

__all__ = ["mix64", "u64", "normal_bf16_bits", "tokens", "bf16_bits_to_f32", "f32_to_bf16_bits",
           "uniform_int_bf16_bits", "torch_normal_bf16_bits", "torch_int_bf16_bits",
           "torch_normal_bf16_device", "torch_int_bf16_device", "ModelCfg", "AdamCfg", "PRESETS", "preset", "layer_tensor_shapes",
           "STREAM_TOKENS", "STREAM_EMBED", "STREAM_FINAL_NORM", "STREAM_HEAD", "layer_stream",
           "make_weights", "make_layer_weights", "make_tokens", "LAYER_TENSORS", "BF16_ONE"]
