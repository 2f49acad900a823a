"""The allocation-free attention backward (mt_op_attention_bwd_noalloc)
against the workspace entry point (mt_op_attention_bwd): the same kernels,
so the same bits, on two calls in a row with the second on a smaller input
(the static scratch keeps the first call's contents); sizes beyond its
static scratch are refused with an error; and the result still meets the
oracle at the gradient bar."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from host_memory_centric_amd import _lib
from host_memory_centric_amd._lib import MtError, call

from gpu_util import metrics, ptr, stream
from parity import GRAD_COS, GRAD_MAXREL

pytestmark = pytest.mark.gpu


def _inputs(gpu, B, S, nh, hd, seed):
    import torch
    H = nh * hd
    qkv = synth.torch_normal_bf16_device(seed, (B * S, 3 * H), std=0.9, device=gpu)
    do = synth.torch_normal_bf16_device(seed + 1, (B * S, H), std=1.0, device=gpu)
    o = torch.zeros((B * S, H), dtype=torch.int16, device=gpu)
    lse = torch.zeros((B, nh, S), dtype=torch.float32, device=gpu)
    nws = ctypes.c_size_t()
    call("mt_op_attention_ws_bytes", B, S, nh, hd, ctypes.byref(nws))
    ws = torch.empty(max(nws.value, 256), dtype=torch.uint8, device=gpu)
    call("mt_op_attention_fwd", B, S, nh, hd, ptr(qkv), ptr(o), ptr(lse), ptr(ws), ws.numel(), stream())
    return qkv, do, o, lse, ws


def test_noalloc_attention_bwd_matches_workspace_entry(gpu):
    import torch
    _lib.load()
    for i, (B, S, nh, hd) in enumerate([(2, 1000, 4, 128), (1, 333, 2, 64)]):  # second call smaller
        print(f"no-alloc attention backward: B={B} S={S} heads={nh} hd={hd}", flush=True)
        qkv, do, o, lse, ws = _inputs(gpu, B, S, nh, hd, seed=70 + 10 * i)
        H = nh * hd
        ref = torch.zeros((B * S, 3 * H), dtype=torch.int16, device=gpu)
        got = torch.full((B * S, 3 * H), 0x7fc0, dtype=torch.int16, device=gpu)
        call("mt_op_attention_bwd", B, S, nh, hd, ptr(qkv), ptr(o), ptr(lse), ptr(do), ptr(ref), ptr(ws), ws.numel(),
             stream())
        call("mt_op_attention_bwd_noalloc", B, S, nh, hd, ptr(qkv), ptr(o), ptr(lse), ptr(do), ptr(got), stream())
        torch.cuda.synchronize()
        assert torch.equal(got, ref), i
        # and the oracle at the gradient bar (one head of the first batch row)
        f = lambda t, c0: t[:S, c0:c0 + hd].view(torch.bfloat16).double().cpu().numpy()
        q, k, v = f(qkv, 0), f(qkv, H), f(qkv, 2 * H)
        _, _, dq, dk, dv = oracle.attention_suffix(q, k, v, f(do, 0), 0, o_rows=f(o, 0))
        for nm, r, c0 in (("dq", dq, 0), ("dk", dk, H), ("dv", dv, 2 * H)):
            mar, cos = metrics(f(got, c0), r)
            print(f"  {nm}: max-abs-rel {mar:.3e} cos {cos:.7f}", flush=True)
            assert mar <= GRAD_MAXREL and cos >= GRAD_COS, (nm, mar, cos)
        del qkv, do, o, lse, ws, ref, got


def test_noalloc_attention_bwd_rejects_oversize(gpu):
    import torch
    _lib.load()
    t = torch.zeros(64, dtype=torch.int16, device=gpu)
    lse = torch.zeros(64, dtype=torch.float32, device=gpu)
    # 2 x 64 heads x 131073 rows = 16777344 > 16777216: refused before any launch
    with pytest.raises(MtError) as e:
        call("mt_op_attention_bwd_noalloc", 2, 131073, 64, 128, ptr(t), ptr(t), ptr(lse), ptr(t), ptr(t), stream())
    assert e.value.code == -1 and "static buffer" in str(e.value)
