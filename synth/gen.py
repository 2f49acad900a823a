"""Counter-based SplitMix64 generator and the bf16 bit conversions of inputs.

See the package docstring for the exact definition.  Everything here is
vectorised numpy over uint64 (wrap-around multiplication is the intended
modular arithmetic).  Large tensors are produced chunk by chunk on a thread
pool; numpy releases the GIL inside its ufuncs.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
M1 = np.uint64(0xBF58476D1CE4E5B9)
M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def mix64(z):
    """SplitMix64 output mix of a uint64 array (returns a new array)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * M1
        z = (z ^ (z >> np.uint64(27))) * M2
    return z ^ (z >> np.uint64(31))


def _key(seed, stream, i):
    if not (0 <= seed < (1 << 16) and 0 <= stream < (1 << 16)):
        raise ValueError("seed and stream must fit in 16 bits")
    base = np.uint64((seed << 48) | (stream << 32))
    return base | np.asarray(i, dtype=np.uint64)


def u64(seed, stream, i):
    """u(key) for key = seed<<48 | stream<<32 | i (i: array of indices < 2**32)."""
    with np.errstate(over="ignore"):
        return mix64(_key(seed, stream, i) * GAMMA)


def f32_to_bf16_bits(x):
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_chunk(seed, stream, lo, hi, std):
    i = np.arange(lo, hi, dtype=np.uint64)
    a = u64(seed, stream, np.uint64(2) * i)
    b = u64(seed, stream, np.uint64(2) * i + np.uint64(1))
    u1 = ((a >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * (2.0 ** -53)
    u2 = (b >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return f32_to_bf16_bits((std * z).astype(np.float32))


def _pool_map(fn, n, chunk=_CHUNK):
    starts = list(range(0, n, chunk))
    if len(starts) <= 1:
        return [fn(0, n)]
    workers = min(len(starts), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda s: fn(s, min(n, s + chunk)), starts))


def normal_bf16_bits(seed, stream, n, std=0.02, start=0):
    """n bf16 values (uint16 bits) ~N(0, std) for elements start..start+n-1."""
    if start + n > (1 << 31):
        raise ValueError("per-tensor index must stay below 2**31")
    parts = _pool_map(lambda lo, hi: _normal_chunk(seed, stream, start + lo, start + hi, std), n)
    return np.concatenate(parts) if len(parts) > 1 else parts[0]


def tokens(seed, vocab, B, S, step=0):
    """int32 [B, S] tokens uniform in [0, vocab) for training step `step`."""
    T = B * S
    i = np.arange(step * T, step * T + T, dtype=np.uint64)
    u = u64(seed, 0, i)
    v = np.uint64(vocab)
    hi = u >> np.uint64(32)
    lo = u & np.uint64(0xFFFFFFFF)
    with np.errstate(over="ignore"):
        t = (hi * v + ((lo * v) >> np.uint64(32))) >> np.uint64(32)
    return t.astype(np.int32).reshape(B, S)


def uniform_int_bf16_bits(seed, stream, n, lo_val=-4, hi_val=4):
    """bf16 bits of integers uniform in [lo_val, hi_val] (exact in bf16); for GEMM tests."""
    i = np.arange(n, dtype=np.uint64)
    u = u64(seed, stream, i)
    span = np.uint64(hi_val - lo_val + 1)
    hi = u >> np.uint64(32)
    lo = u & np.uint64(0xFFFFFFFF)
    with np.errstate(over="ignore"):
        t = (hi * span + ((lo * span) >> np.uint64(32))) >> np.uint64(32)
    vals = t.astype(np.int64) + lo_val
    return f32_to_bf16_bits(vals.astype(np.float32))


def torch_normal_bf16_bits(seed, shape, std=1.0, mean=0.0):
    """bf16 bits (uint16 numpy) of N(mean, std^2) samples for full-size tests.

    Drawn with torch's CPU generator (Mersenne Twister seeded with ``seed``),
    scaled in fp32 and rounded to bf16 to nearest-even.  Used where the
    counter-based generator above would be too slow in numpy (hundreds of
    millions of elements); both sides of a comparison read the same bits."""
    import torch
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    t = t * float(std) + float(mean)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_int_bf16_bits(seed, shape, lo_val=-4, hi_val=4):
    """bf16 bits of integers uniform in [lo_val, hi_val] from torch's CPU
    generator; exact in bf16 (full-size GEMM tests)."""
    import torch
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randint(lo_val, hi_val + 1, tuple(shape), generator=g, dtype=torch.int32)
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def torch_normal_bf16_device(seed, shape, std=1.0, device="cuda:0"):
    """Like ``torch_normal_bf16_bits`` but drawn on the device with torch's
    seeded device generator (Philox) and returned as an int16 device tensor of
    bf16 bits; for inputs of several GB whose sampled parts are copied back."""
    import torch
    g = torch.Generator(device=device).manual_seed(int(seed))
    t = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    t.normal_(0.0, float(std), generator=g)
    return t.view(torch.int16)


def torch_int_bf16_device(seed, shape, lo_val=-4, hi_val=4, device="cuda:0"):
    """Integers uniform in [lo_val, hi_val] as bf16 bits (int16 device tensor)."""
    import torch
    g = torch.Generator(device=device).manual_seed(int(seed))
    t = torch.randint(lo_val, hi_val + 1, tuple(shape), generator=g, dtype=torch.int8, device=device)
    return t.to(torch.bfloat16).view(torch.int16)
