"""Host store wrapper: the library-owned, layer-contiguous master copy.

numpy views over a unit's regions are provided for filling weights and for
inspection; all arithmetic on the store happens inside the library
(``mt_step``, ``mt_embed_grad``, ``mt_pack_layer``).
"""
import ctypes

import numpy as np

from ._lib import (MT_STORE_GRAD_ACCUM, MT_STORE_MASTER_FP32, MT_STORE_PINNED_DMA, MT_UNIT_EMBED, MT_UNIT_HEAD, call,
                   load, model_cfg, unit_layout)

REGION_W, REGION_G, REGION_M, REGION_V, REGION_P, REGION_A = 0, 1, 2, 3, 4, 5
LAYER_TENSORS = ("g_attn", "wqkv", "wo", "g_mlp", "wgu", "wd")


def tensor_shapes(cfg, unit):
    h, f, V = cfg.hidden, cfg.ffn, cfg.vocab
    if unit == MT_UNIT_EMBED:
        return [("embed", (V, h))]
    if unit == MT_UNIT_HEAD:  # with tied weights the LM head is the embedding
        return [("g_final", (h,))] if getattr(cfg, "tied", False) else [("g_final", (h,)), ("head", (V, h))]
    return [("g_attn", (h,)), ("wqkv", (3 * h, h)), ("wo", (h, h)), ("g_mlp", (h,)), ("wgu", (2 * f, h)),
            ("wd", (h, f))]


class HostStore:
    """master: keep fp32 master weights (region P); accum: keep an fp32
    gradient accumulator for micro-batches (region A); pinned: page-lock the
    W and G regions so that the DMA engines read weights from and write
    gradients to the store itself (needs a HIP device)."""

    def __init__(self, cfg, master=False, accum=False, pinned=False):
        load()
        self.cfg = cfg
        self.mcfg = model_cfg(cfg)
        self.flags = ((MT_STORE_MASTER_FP32 if master else 0) | (MT_STORE_GRAD_ACCUM if accum else 0)
                      | (MT_STORE_PINNED_DMA if pinned else 0))
        self.pinned = bool(pinned)
        p = ctypes.c_void_p()
        call("mt_store_create_ex", ctypes.byref(self.mcfg), self.flags, ctypes.byref(p))
        self.ptr = p
        self.units = [MT_UNIT_HEAD, MT_UNIT_EMBED] + list(range(cfg.layers))
        self.layout = {u: unit_layout(self.mcfg, u, self.flags) for u in (MT_UNIT_HEAD, MT_UNIT_EMBED, 0)}

    def layout_of(self, unit):
        return self.layout[unit if unit < 0 else 0]

    def close(self):
        if self.ptr is not None and self.ptr.value:
            load().mt_store_destroy(self.ptr)
        self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def total_bytes(self):
        out = ctypes.c_uint64()
        call("mt_store_bytes", self.ptr, ctypes.byref(out))
        return out.value

    def block_addr(self, unit):
        """Base address of a unit's block (pageable stores only)."""
        p = ctypes.c_void_p()
        call("mt_store_block", self.ptr, unit, ctypes.byref(p))
        return p.value

    def region_addr(self, unit, r):
        p = ctypes.c_void_p()
        call("mt_store_region", self.ptr, unit, r, ctypes.byref(p))
        return p.value

    def region(self, unit, r):
        """numpy view of a region over the W indexing (uint16 for W/G, float32 for M/V/P/A)."""
        L = self.layout_of(unit)
        if L.region_bytes[r] == 0:
            raise ValueError(f"the store has no region {r}")
        n = L.w_bytes // 2
        dt = np.uint16 if r in (REGION_W, REGION_G) else np.float32
        addr = self.region_addr(unit, r)
        buf = (ctypes.c_char * (n * np.dtype(dt).itemsize)).from_address(addr)
        return np.frombuffer(buf, dtype=dt, count=n)

    def tensor(self, unit, name, r=REGION_W):
        L = self.layout_of(unit)
        reg = self.region(unit, r)
        for j, (nm, shape) in enumerate(tensor_shapes(self.cfg, unit)):
            if nm == name:
                off = L.tensor_off[j] // 2
                return reg[off:off + int(np.prod(shape))].reshape(shape)
        raise KeyError(name)

    def save(self, path, t):
        """Checkpoint every block (and the step counter t) to a file."""
        call("mt_store_save", self.ptr, str(path).encode(), int(t))

    def load(self, path):
        """Restore a checkpoint written by save() for this config and flags; returns t."""
        t = ctypes.c_int64()
        call("mt_store_load", self.ptr, str(path).encode(), ctypes.byref(t))
        return t.value

    def fill_normal(self, seed=None, std=0.02):
        call("mt_store_fill_normal", self.ptr, self.cfg.seed if seed is None else seed, std)

    def load_bits(self, bits):
        """Copy weights given as bf16 bit arrays (the synth layout) into the W regions; zero G, M, V
        (and A); the master weights P, if any, become the exact fp32 values of W."""
        for u in self.units:
            for r in (REGION_G, REGION_M, REGION_V) + ((REGION_A,) if self.flags & MT_STORE_GRAD_ACCUM else ()):
                self.region(u, r)[:] = 0
        self.tensor(MT_UNIT_EMBED, "embed")[:] = bits["embed"]
        self.tensor(MT_UNIT_HEAD, "g_final")[:] = bits["g_final"]
        if bits.get("head") is not None:
            self.tensor(MT_UNIT_HEAD, "head")[:] = bits["head"]
        for l, lw in enumerate(bits["layers"]):
            for name in LAYER_TENSORS:
                self.tensor(l, name)[:] = lw[name]
        if self.flags & MT_STORE_MASTER_FP32:
            call("mt_store_sync_master", self.ptr)

    def read_bits(self):
        """Copy of all weights as bf16 bit arrays (the synth layout)."""
        out = {"embed": self.tensor(MT_UNIT_EMBED, "embed").copy(),
               "g_final": self.tensor(MT_UNIT_HEAD, "g_final").copy(),
               "head": None if getattr(self.cfg, "tied", False) else self.tensor(MT_UNIT_HEAD, "head").copy(),
               "layers": []}
        for l in range(self.cfg.layers):
            out["layers"].append({n: self.tensor(l, n).copy() for n in LAYER_TENSORS})
        return out
