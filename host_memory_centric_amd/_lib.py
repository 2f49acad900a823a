"""ctypes binding of ``libmt.so`` (argument marshalling only).

Every function here forwards to the C entry point of the same name and raises
``MtError`` (with the library's thread-local message) when it returns a
negative code.  Loading fails loudly if the library has not been built: there
is no fallback implementation.
"""
import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_uint32, c_uint64, \
    c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmt.so")

MT_UNIT_EMBED = -1
MT_UNIT_HEAD = -2
MT_STORE_MASTER_FP32 = 1
MT_STORE_GRAD_ACCUM = 2
MT_STORE_PINNED_DMA = 4
ERRORS = {-1: "MT_E_ARG", -2: "MT_E_SHAPE", -3: "MT_E_ALIGN", -4: "MT_E_NOMEM", -5: "MT_E_HIP", -6: "MT_E_STATE",
          -7: "MT_E_IO"}


class MtError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with {ERRORS.get(code, code)}: {msg}")
        self.code = code


class MtModelCfg(ctypes.Structure):
    _fields_ = [("layers", c_int32), ("hidden", c_int32), ("heads", c_int32), ("head_dim", c_int32),
                ("ffn", c_int32), ("vocab", c_int32), ("eps", c_float), ("rope_base", c_float), ("tied", c_int32)]


class MtUnitLayout(ctypes.Structure):
    _fields_ = [("n_tensors", c_int32), ("pad_", c_int32), ("tensor_off", c_uint64 * 6),
                ("tensor_numel", c_uint64 * 6), ("w_bytes", c_uint64), ("region_off", c_uint64 * 6),
                ("region_bytes", c_uint64 * 6), ("block_bytes", c_uint64), ("params", c_uint64)]


class MtAdamCfg(ctypes.Structure):
    _fields_ = [("lr", c_double), ("beta1", c_double), ("beta2", c_double), ("eps", c_double),
                ("weight_decay", c_double)]


class MtLayerView(ctypes.Structure):
    _fields_ = [("w", c_void_p * 6), ("g", c_void_p * 6)]


class MtAct(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("seq", c_int32), ("x_in", c_void_p), ("x_out", c_void_p), ("dy", c_void_p),
                ("dy_bf16", c_void_p), ("dx", c_void_p), ("dx_bf16", c_void_p), ("rope_cos", c_void_p),
                ("rope_sin", c_void_p), ("saved", c_void_p), ("workspace", c_void_p), ("saved_bytes", c_size_t),
                ("workspace_bytes", c_size_t)]


class MtHeadIO(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("seq", c_int32), ("x", c_void_p), ("tokens", c_void_p), ("dx", c_void_p),
                ("dx_bf16", c_void_p), ("loss", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


class MtProfEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 24), ("launches", c_int64), ("ms", c_double), ("flops", c_double)]


# name -> (argtypes)
_SIGS = {
    "mt_unit_layout_get": [POINTER(MtModelCfg), c_int, POINTER(MtUnitLayout)],
    "mt_unit_layout_get_ex": [POINTER(MtModelCfg), c_uint32, c_int, POINTER(MtUnitLayout)],
    "mt_store_create": [POINTER(MtModelCfg), POINTER(c_void_p)],
    "mt_store_create_ex": [POINTER(MtModelCfg), c_uint32, POINTER(c_void_p)],
    "mt_store_sync_master": [c_void_p],
    "mt_grad_accumulate": [c_void_p, c_int, c_void_p],
    "mt_store_save": [c_void_p, ctypes.c_char_p, c_int64],
    "mt_store_load": [c_void_p, ctypes.c_char_p, POINTER(c_int64)],
    "mt_store_block": [c_void_p, c_int, POINTER(c_void_p)],
    "mt_store_region": [c_void_p, c_int, c_int, POINTER(c_void_p)],
    "mt_store_bytes": [c_void_p, POINTER(c_uint64)],
    "mt_store_fill_normal": [c_void_p, c_uint32, c_double],
    "mt_set_threads": [c_int],
    "mt_set_optimizer_threads": [c_int],
    "mt_pack_layer": [c_void_p, c_int, c_void_p, c_size_t],
    "mt_pinned_alloc": [c_size_t, POINTER(c_void_p)],
    "mt_pinned_free": [c_void_p],
    "mt_host_copy": [c_void_p, c_void_p, c_size_t],
    "mt_copy_h2d": [c_void_p, c_void_p, c_size_t, c_void_p],
    "mt_copy_d2h": [c_void_p, c_void_p, c_size_t, c_void_p],
    "mt_step": [c_void_p, c_int, c_void_p, POINTER(MtAdamCfg), c_int64, c_void_p],
    "mt_embed_gather": [c_void_p, c_void_p, c_int64, c_void_p],
    "mt_embed_grad": [c_void_p, c_void_p, c_int64, c_void_p],
    "mt_embed_grad_tied": [c_void_p, c_void_p, c_int64, c_void_p, c_void_p],
    "mt_pack_head_tied": [c_void_p, c_void_p, c_size_t],
    "mt_rope_tables": [POINTER(MtModelCfg), c_int32, c_void_p, c_void_p],
    "mt_bind": [POINTER(MtModelCfg), c_int, c_void_p, c_void_p, POINTER(MtLayerView)],
    "mt_layer_saved_bytes": [POINTER(MtModelCfg), c_int32, c_int32, POINTER(c_size_t)],
    "mt_layer_workspace_bytes": [POINTER(MtModelCfg), c_int32, c_int32, POINTER(c_size_t)],
    "mt_layer_fwd": [POINTER(MtLayerView), POINTER(MtModelCfg), POINTER(MtAct), c_void_p],
    "mt_layer_recompute_bwd": [POINTER(MtLayerView), POINTER(MtModelCfg), POINTER(MtAct), c_void_p],
    "mt_head_workspace_bytes": [POINTER(MtModelCfg), c_int32, c_int32, POINTER(c_size_t)],
    "mt_head_fwd_bwd": [POINTER(MtLayerView), POINTER(MtModelCfg), POINTER(MtHeadIO), c_void_p],
    "mt_op_gemm": [c_int64, c_int64, c_int64, c_void_p, c_int64, c_int, c_void_p, c_int64, c_int, c_void_p, c_void_p,
                   c_void_p, c_int64, c_int, c_void_p, c_size_t, c_void_p],
    "mt_probe_mfma": [c_int32, c_void_p, c_void_p, POINTER(c_double)],
    "mt_prof_enable": [c_int],
    "mt_prof_collect": [POINTER(MtProfEntry), c_int, POINTER(c_int), c_int],
    "mt_op_attention_fwd": [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                            c_void_p],
    "mt_op_attention_bwd": [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p, c_size_t, c_void_p],
    "mt_op_attention_bwd_noalloc": [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p],
    "mt_op_attention_ws_bytes": [c_int32, c_int32, c_int32, c_int32, POINTER(c_size_t)],
}
VOID_FUNCS = {"mt_store_destroy": [c_void_p]}
EXPORTED = sorted(list(_SIGS) + list(VOID_FUNCS) + ["mt_last_error"])

_lib = None


def load(path=None):
    """Load libmt.so (once).  Raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is missing: build it with `python -m host_memory_centric_amd.build` "
                      "(there is no fallback implementation)")
    lib = ctypes.CDLL(p, mode=ctypes.RTLD_GLOBAL)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int
    for name, args in VOID_FUNCS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = None
    lib.mt_last_error.argtypes = []
    lib.mt_last_error.restype = c_char_p
    _lib = lib
    return lib


def call(name, *args):
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != 0:
        raise MtError(name, rc, lib.mt_last_error().decode(errors="replace"))
    return rc


def model_cfg(cfg):
    """MtModelCfg from any object with the model-shape attributes."""
    return MtModelCfg(cfg.layers, cfg.hidden, cfg.heads, cfg.head_dim, cfg.ffn, cfg.vocab, cfg.eps, cfg.rope_base,
                      int(bool(getattr(cfg, "tied", False))))


def adam_cfg(a):
    return MtAdamCfg(a.lr, a.beta1, a.beta2, a.eps, a.weight_decay)


def unit_layout(mcfg, unit, flags=0):
    out = MtUnitLayout()
    call("mt_unit_layout_get_ex", ctypes.byref(mcfg), flags, unit, ctypes.byref(out))
    return out


def size_query(name, mcfg, batch, seq):
    out = c_size_t()
    call(name, ctypes.byref(mcfg), batch, seq, ctypes.byref(out))
    return out.value


def prof_collect(reset=True):
    """{class: (launches, ms, flops)} of the timed kernel classes."""
    out = (MtProfEntry * 8)()
    n = c_int()
    call("mt_prof_collect", out, 8, ctypes.byref(n), int(reset))
    return {out[i].name.decode(): (out[i].launches, out[i].ms, out[i].flops) for i in range(n.value)}
