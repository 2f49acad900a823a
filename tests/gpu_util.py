"""Helpers shared by the GPU tests: device copies, raw pointers, the current
stream, and the comparison metrics of the parity bar."""
import ctypes

import numpy as np


def dev(a, gpu):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(gpu)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def bits_to_f32(t):
    """int16 tensor of bf16 bits (any device) -> float32 numpy."""
    import torch
    return t.view(torch.bfloat16).float().cpu().numpy()


def metrics(got, ref):
    """(max|got - ref| / max|ref|, cosine) over all elements, in fp64."""
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1)
    mar = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    cos = got @ ref / max(np.linalg.norm(got) * np.linalg.norm(ref), 1e-300)
    return float(mar), float(cos)
