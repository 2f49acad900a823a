"""Timing of the layer template's attention kernels through the C ABI.

    python -m host_memory_centric_amd.kernel_bench BxSxHEADS [...]

For each shape (batch x sequence x heads, head_dim 128) it runs
``mt_op_attention_fwd`` and ``mt_op_attention_bwd`` (the bf16
instantiations) on seeded random q, k, v and dO, times repeated launches with
HIP events on the current stream, and prints one line per kernel with the
average time and the counted rate: 4*hd flops per causal (query, key) pair
for the forward, 10*hd for the backward (QK^T recompute, dP, dV, dK, dQ).
"""
import ctypes
import sys

import torch

from . import _lib


def time_attention(B, S, heads, hd=128, seed=0):
    """Average milliseconds of one forward and one backward launch."""
    H = heads * hd
    T = B * S
    g = torch.Generator(device="cuda").manual_seed(seed)
    qkv = (torch.randn(T, 3 * H, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    o = torch.empty(T, H, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(B * heads * S, device="cuda", dtype=torch.float32)
    d_o = (torch.randn(T, H, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    dqkv = torch.empty(T, 3 * H, device="cuda", dtype=torch.bfloat16)
    nws = ctypes.c_size_t()
    _lib.call("mt_op_attention_ws_bytes", B, S, heads, hd, ctypes.byref(nws))
    ws = torch.empty(max(256, nws.value), device="cuda", dtype=torch.uint8)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def p(t):
        return ctypes.c_void_p(t.data_ptr())

    def fwd():
        _lib.call("mt_op_attention_fwd", B, S, heads, hd, p(qkv), p(o), p(lse), p(ws), ws.numel(), st)

    def bwd():
        _lib.call("mt_op_attention_bwd", B, S, heads, hd, p(qkv), p(o), p(lse), p(d_o), p(dqkv), p(ws), ws.numel(),
                  st)
    reps = max(2, min(20, int(2e10 / (B * heads * S * S))))
    out = {}
    for name, f in (("fwd", fwd), ("bwd", bwd)):
        f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            f()
        b.record()
        torch.cuda.synchronize()
        out[name] = a.elapsed_time(b) / reps
    return out


def main(argv):
    _lib.load()
    if not torch.cuda.is_available():
        raise SystemExit("kernel_bench needs a GPU")
    for spec in argv or ["8x1024x40", "4x2048x32"]:
        B, S, heads = (int(x) for x in spec.split("x"))
        ms = time_attention(B, S, heads)
        pairs = B * heads * S * (S + 1) / 2
        for name, fl in (("fwd", 4.0), ("bwd", 10.0)):
            print(f"attention {name} B={B} S={S} heads={heads}: {ms[name]:.4f} ms, "
                  f"{fl * 128 * pairs / (ms[name] * 1e-3) / 1e12:.1f} TFLOP/s counted", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
