"""Run one layer's forward and recompute-backward through the C ABI on the
GPU (the entry points, shapes and workspaces of a training step), for the
full-size parity tests."""
import ctypes

import numpy as np

from host_memory_centric_amd import _lib
from host_memory_centric_amd._lib import MtAct, MtLayerView, call

from gpu_util import ptr, stream


def layer_slot(gpu, mcfg, unit, tensors):
    """Device W slot of a unit with the library's layout, filled from bf16 bits."""
    import torch
    lay = _lib.unit_layout(mcfg, unit)
    slot = torch.zeros(lay.w_bytes // 2, dtype=torch.int16, device=gpu)
    for j, arr in enumerate(tensors):
        off = lay.tensor_off[j] // 2
        slot[off:off + arr.size] = torch.from_numpy(arr.reshape(-1).view(np.int16)).to(gpu)
    return slot, lay


def unslot(gslot, lay, shapes):
    """fp32 numpy copies of the tensors of a bf16 gradient slot."""
    import torch
    out = []
    for j, shape in enumerate(shapes):
        off = lay.tensor_off[j] // 2
        n = int(np.prod(shape))
        out.append(gslot[off:off + n].view(torch.bfloat16).float().cpu().numpy().reshape(shape))
    return out


def run_layer(gpu, cfg, W, x_bits, dy_dev):
    """mt_layer_fwd (keeping the internals) then mt_layer_recompute_bwd on
    weights W (name -> bf16 bits), input x_bits (bf16 bits [T, h], host) and
    output gradient dy_dev (fp32 device tensor [T, h]).  Returns device
    tensors (y as int16 bf16 bits, dx fp32) and the weight gradients as fp32
    numpy arrays by name."""
    import torch
    B, S, h = cfg.batch, cfg.seq, cfg.hidden
    T = B * S
    names = list(W)
    mcfg = _lib.model_cfg(cfg)
    slot, lay = layer_slot(gpu, mcfg, 0, [W[n] for n in names])
    gslot = torch.zeros_like(slot)
    v = MtLayerView()
    call("mt_bind", ctypes.byref(mcfg), 0, ptr(slot), ptr(gslot), ctypes.byref(v))
    saved_bytes = _lib.size_query("mt_layer_saved_bytes", mcfg, B, S)
    ws_bytes = _lib.size_query("mt_layer_workspace_bytes", mcfg, B, S)
    saved = torch.empty(saved_bytes, dtype=torch.uint8, device=gpu)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=gpu)
    cs = np.empty((S, cfg.head_dim // 2), dtype=np.float32)
    sn = np.empty_like(cs)
    call("mt_rope_tables", ctypes.byref(mcfg), S, cs.ctypes.data_as(ctypes.c_void_p),
         sn.ctypes.data_as(ctypes.c_void_p))
    d_cs, d_sn = torch.from_numpy(cs).to(gpu), torch.from_numpy(sn).to(gpu)
    d_x = torch.from_numpy(x_bits.view(np.int16)).to(gpu)
    d_y = torch.empty_like(d_x)
    d_dyb = dy_dev.to(torch.bfloat16).view(torch.int16)
    d_dx = torch.empty((T, h), dtype=torch.float32, device=gpu)
    d_dxb = torch.empty((T, h), dtype=torch.int16, device=gpu)
    a = MtAct()
    a.batch, a.seq = B, S
    a.x_in, a.x_out = d_x.data_ptr(), d_y.data_ptr()
    a.dy, a.dy_bf16, a.dx, a.dx_bf16 = dy_dev.data_ptr(), d_dyb.data_ptr(), d_dx.data_ptr(), d_dxb.data_ptr()
    a.rope_cos, a.rope_sin = d_cs.data_ptr(), d_sn.data_ptr()
    a.saved, a.saved_bytes = saved.data_ptr(), saved_bytes
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws_bytes
    call("mt_layer_fwd", ctypes.byref(v), ctypes.byref(mcfg), ctypes.byref(a), stream())
    call("mt_layer_recompute_bwd", ctypes.byref(v), ctypes.byref(mcfg), ctypes.byref(a), stream())
    torch.cuda.synchronize()
    grads = dict(zip(names, unslot(gslot, lay, [W[n].shape for n in names])))
    del saved, ws, slot, gslot, d_dxb, d_dyb, d_x
    torch.cuda.empty_cache()
    return d_y, d_dx, grads
