"""Host-side parts of libmt.so, on the CPU (no GPU needed).

The library must load and export every entry point the header declares; the
host store layout must follow the layer-contiguous, 4 KB-aligned block format;
the seeded filler must reproduce the synthetic-input generator bit for bit;
the packer must copy the W region; the host Adam must equal the oracle's Adam
bit for bit; the embedding gather/scatter and RoPE tables must match the
oracle.  The schedule planner (pure Python) is checked for the number of
weight loads the method implies.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
from host_memory_centric_amd import _lib
from host_memory_centric_amd._lib import MT_UNIT_EMBED, MT_UNIT_HEAD, MtError, call
from host_memory_centric_amd.engine import plan_slots, plan_step
from host_memory_centric_amd.store import (REGION_G, REGION_M, REGION_P, REGION_V, REGION_W, HostStore,
                                          tensor_shapes)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    hdr = open(os.path.join(ROOT, "include", "mt.h")).read()
    declared = set(re.findall(r"\b(mt_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 25
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(_lib.EXPORTED)


def _units(cfg):
    return [MT_UNIT_HEAD, MT_UNIT_EMBED] + list(range(cfg.layers))


@pytest.mark.parametrize("name", ["tiny", "7b", "14b", "depth180", "width5x"])
def test_layout_alignment_and_accounting(lib, name):
    cfg = synth.preset(name)
    m = _lib.model_cfg(cfg)
    total_params = 0
    total_bytes = 0
    for u in (MT_UNIT_HEAD, MT_UNIT_EMBED, 0):
        L = _lib.unit_layout(m, u)
        shapes = tensor_shapes(cfg, u)
        assert L.n_tensors == len(shapes)
        for j, (_, shp) in enumerate(shapes):
            assert L.tensor_off[j] % 256 == 0
            assert L.tensor_numel[j] == int(np.prod(shp))
            if j:
                assert L.tensor_off[j] >= L.tensor_off[j - 1] + 2 * L.tensor_numel[j - 1]
        for r in range(4):
            assert L.region_off[r] % 4096 == 0 and L.region_bytes[r] % 4096 == 0
        assert L.region_off[1] == L.region_bytes[0] and L.region_bytes[1] == L.region_bytes[0]
        assert L.region_bytes[2] >= 2 * L.w_bytes and L.region_bytes[3] == L.region_bytes[2]
        assert L.block_bytes == sum(L.region_bytes)
        mult = cfg.layers if u == 0 else 1
        total_params += mult * L.params
        total_bytes += mult * L.block_bytes
    per_param = total_bytes / total_params
    assert 12.0 <= per_param < 12.0 + 0.05 if name != "tiny" else per_param < 12.3


def test_state_accounting_matches_pages(lib):
    rows = {}
    for line in open(os.path.join(ROOT, "tests", "golden", "state_accounting.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split()
            rows[k] = int(v)
    # bytes per real parameter of the block format, padding excluded
    cfg = synth.preset("7b")
    L = _lib.unit_layout(_lib.model_cfg(cfg), 0)
    per = (2 * L.w_bytes + 2 * 4 * (L.w_bytes // 2)) / L.params  # W + G + M + V over the W indexing
    assert round(per) == rows["bytes_per_param"]
    assert rows["bytes_per_param"] * rows["params"] == rows["bytes"]


def test_shape_errors(lib):
    cfg = synth.preset("tiny").with_(heads=3)
    with pytest.raises(MtError) as e:
        _lib.unit_layout(_lib.model_cfg(cfg), 0)
    assert e.value.code == -2
    with pytest.raises(MtError) as e:
        _lib.unit_layout(_lib.model_cfg(synth.preset("tiny")), 7)
    assert e.value.code == -1


def _bits_cfg():
    # wide enough that every tensor spans many generator chunks
    return synth.ModelCfg("host", 2, 512, 8, 64, 1376, 2048, 1, 16)


def test_store_fill_matches_synth_generator(lib):
    cfg = _bits_cfg()
    st = HostStore(cfg)
    try:
        st.fill_normal(seed=0)
        ref = synth.make_weights(cfg)
        assert np.array_equal(st.tensor(MT_UNIT_EMBED, "embed"), ref["embed"])
        assert np.array_equal(st.tensor(MT_UNIT_HEAD, "head"), ref["head"])
        assert np.array_equal(st.tensor(MT_UNIT_HEAD, "g_final"), ref["g_final"])
        for l in range(cfg.layers):
            for k, a in ref["layers"][l].items():
                assert np.array_equal(st.tensor(l, k), a), (l, k)
        for u in _units(cfg):
            for r in (REGION_G, REGION_M, REGION_V):
                assert not st.region(u, r).any()
    finally:
        st.close()


def test_store_fill_sampled_large_indices(lib):
    """Elements near the end of a 7B-sized fused gate/up tensor (index ~9e7)."""
    cfg = synth.ModelCfg("probe", 1, 4096, 32, 128, 11008, 8, 1, 8)
    st = HostStore(cfg)
    try:
        st.fill_normal(seed=0)
        wgu = st.tensor(0, "wgu").reshape(-1)
        n = wgu.size
        for start in (0, n // 3, n - 4096):
            ref = synth.normal_bf16_bits(0, synth.layer_stream(0, 4), 4096, start=start)
            assert np.array_equal(wgu[start:start + 4096], ref)
    finally:
        st.close()


def test_pack_copies_w_region(lib):
    cfg = synth.preset("tiny")
    st = HostStore(cfg)
    try:
        st.fill_normal()
        L = st.layout_of(0)
        dst = np.zeros(L.w_bytes // 2 + 100, dtype=np.uint16)
        call("mt_pack_layer", st.ptr, 1, dst.ctypes.data_as(ctypes.c_void_p), dst.nbytes)
        assert np.array_equal(dst[: L.w_bytes // 2], st.region(1, REGION_W))
        with pytest.raises(MtError):
            call("mt_pack_layer", st.ptr, 1, dst.ctypes.data_as(ctypes.c_void_p), 16)
    finally:
        st.close()


def test_host_copy(lib):
    """The library's multi-threaded host copy (used for block checkpoints held in
    host memory): every byte, aligned or not, across several 4 MB chunks, and
    overlapping buffers rejected."""
    rng = np.random.default_rng(5)
    src = rng.integers(0, 256, size=(9 << 20) + 77, dtype=np.uint8)
    for off, n in [(0, 0), (0, 1), (0, 255), (0, 257), (64, 9 << 20), (3, (9 << 20) + 13), (0, src.nbytes)]:
        dst = np.zeros(src.nbytes + 64, dtype=np.uint8)
        pd = ctypes.c_void_p(dst.ctypes.data + off)
        call("mt_host_copy", pd, src.ctypes.data_as(ctypes.c_void_p), n)
        assert np.array_equal(dst[off:off + n], src[:n]), (off, n)
        assert not dst[:off].any() and not dst[off + n:].any(), (off, n)
    buf = src.copy()
    for d in (0, 1000):
        with pytest.raises(MtError) as e:
            call("mt_host_copy", ctypes.c_void_p(buf.ctypes.data + d), ctypes.c_void_p(buf.ctypes.data + 500), 4096)
        assert e.value.code == -1
    with pytest.raises(MtError):
        call("mt_host_copy", None, buf.ctypes.data_as(ctypes.c_void_p), 16)
    assert np.array_equal(buf, src)


@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_host_adam_bitwise_equals_oracle(lib, wd):
    cfg = synth.preset("tiny")
    adam = synth.AdamCfg(weight_decay=wd)
    st = HostStore(cfg)
    try:
        bits = synth.make_weights(cfg)
        st.load_bits(bits)
        rng = np.random.default_rng(0)
        L = st.layout_of(0)
        n = L.w_bytes // 2
        m_ref = {k: np.zeros(a.shape, np.float32) for k, a in bits["layers"][1].items()}
        v_ref = {k: np.zeros(a.shape, np.float32) for k, a in bits["layers"][1].items()}
        w_bits = {k: a.copy() for k, a in bits["layers"][1].items()}
        for t in (1, 2, 3):
            g32 = {k: (rng.standard_normal(a.shape) * 10 ** rng.uniform(-7, -2)).astype(np.float32)
                   for k, a in bits["layers"][1].items()}
            slab = np.zeros(n, dtype=np.uint16)
            for j, (name, shp) in enumerate(tensor_shapes(cfg, 1)):
                off = L.tensor_off[j] // 2
                slab[off:off + int(np.prod(shp))] = synth.f32_to_bf16_bits(g32[name]).reshape(-1)
            wout = np.zeros(n, dtype=np.float32)
            call("mt_step", st.ptr, 1, slab.ctypes.data_as(ctypes.c_void_p), ctypes.byref(_lib.adam_cfg(adam)), t,
                 wout.ctypes.data_as(ctypes.c_void_p))
            for j, (name, shp) in enumerate(tensor_shapes(cfg, 1)):
                off = L.tensor_off[j] // 2
                cnt = int(np.prod(shp))
                nb, wf = oracle.adam_update(w_bits[name], g32[name], m_ref[name], v_ref[name], adam, t)
                w_bits[name] = nb
                assert np.array_equal(wout[off:off + cnt].view(np.uint32), wf.reshape(-1).view(np.uint32)), name
                assert np.array_equal(st.tensor(1, name), nb), name
                assert np.array_equal(st.tensor(1, name, REGION_M), m_ref[name]), name
                assert np.array_equal(st.tensor(1, name, REGION_V), v_ref[name]), name
                assert np.array_equal(st.tensor(1, name, REGION_G).reshape(-1),
                                      slab[off:off + cnt]), name
        # padding elements stay zero
        wreg = st.region(1, REGION_W)
        mask = np.ones(n, dtype=bool)
        for j in range(L.n_tensors):
            mask[L.tensor_off[j] // 2: L.tensor_off[j] // 2 + L.tensor_numel[j]] = False
        assert not wreg[mask].any()
    finally:
        st.close()


@pytest.mark.parametrize("master,n_micro", [(False, 2), (True, 1), (True, 3)])
def test_host_accumulate_and_master_bitwise_equal_oracle(lib, master, n_micro):
    """mt_grad_accumulate + mt_step on a store with fp32 master weights and
    a gradient accumulator against the oracle's accumulate_micro /
    accumulated_mean / adam_update(master=...), over three steps."""
    cfg = synth.preset("tiny")
    adam = synth.AdamCfg()
    st = HostStore(cfg, master=master, accum=n_micro > 1)
    try:
        bits = synth.make_weights(cfg)
        st.load_bits(bits)
        rng = np.random.default_rng(3)
        L = st.layout_of(0)
        n = L.w_bytes // 2
        shapes = tensor_shapes(cfg, 1)
        ref = {k: dict(w=a.copy(), m=np.zeros(a.shape, np.float32), v=np.zeros(a.shape, np.float32),
                       p=synth.bf16_bits_to_f32(a).astype(np.float32) if master else None)
               for k, a in bits["layers"][1].items()}

        def slab_of(g32):
            slab = np.zeros(n, dtype=np.uint16)
            for j, (name, shp) in enumerate(shapes):
                off = L.tensor_off[j] // 2
                slab[off:off + int(np.prod(shp))] = synth.f32_to_bf16_bits(g32[name]).reshape(-1)
            return slab

        for t in (1, 2, 3):
            gs = [{k: (rng.standard_normal(a.shape) * 10 ** rng.uniform(-7, -2)).astype(np.float32)
                   for k, a in bits["layers"][1].items()} for _ in range(n_micro)]
            for i in range(n_micro - 1):
                slab = slab_of(gs[i])
                call("mt_grad_accumulate", st.ptr, 1, slab.ctypes.data_as(ctypes.c_void_p))
            slab = slab_of(gs[-1])
            wout = np.zeros(n, dtype=np.float32)
            call("mt_step", st.ptr, 1, slab.ctypes.data_as(ctypes.c_void_p), ctypes.byref(_lib.adam_cfg(adam)), t,
                 wout.ctypes.data_as(ctypes.c_void_p))
            for j, (name, shp) in enumerate(shapes):
                off = L.tensor_off[j] // 2
                cnt = int(np.prod(shp))
                r = ref[name]
                if n_micro > 1:
                    acc = None
                    for i in range(n_micro - 1):
                        acc = oracle.accumulate_micro(acc, gs[i][name], i == 0)
                    g = oracle.accumulated_mean(acc, gs[-1][name], n_micro)
                else:
                    g = gs[-1][name]
                nb, wf = oracle.adam_update(r["w"], g, r["m"], r["v"], adam, t, master=r["p"])
                r["w"] = nb
                assert np.array_equal(wout[off:off + cnt].view(np.uint32), wf.reshape(-1).view(np.uint32)), name
                assert np.array_equal(st.tensor(1, name), nb), name
                assert np.array_equal(st.tensor(1, name, REGION_M), r["m"]), name
                assert np.array_equal(st.tensor(1, name, REGION_G), synth.f32_to_bf16_bits(g)), name
                if master:
                    assert np.array_equal(st.tensor(1, name, REGION_P).view(np.uint32), r["p"].view(np.uint32)), name
    finally:
        st.close()


def test_store_regions_and_flags(lib):
    cfg = synth.preset("tiny")
    mcfg = _lib.model_cfg(cfg)
    plain = _lib.unit_layout(mcfg, 0)
    both = _lib.unit_layout(mcfg, 0, _lib.MT_STORE_MASTER_FP32 | _lib.MT_STORE_GRAD_ACCUM)
    assert plain.region_bytes[4] == 0 and plain.region_bytes[5] == 0
    for r in range(4):
        assert both.region_off[r] == plain.region_off[r] and both.region_bytes[r] == plain.region_bytes[r]
    assert both.region_bytes[4] == both.region_bytes[5] == plain.region_bytes[2]
    assert both.region_off[4] == plain.block_bytes and both.region_off[5] % 4096 == 0
    assert both.block_bytes == plain.block_bytes + 2 * plain.region_bytes[2]
    with pytest.raises(MtError):
        _lib.unit_layout(mcfg, 0, 8)
    # the page-locking flag is placement only: the layout does not change
    pinned = _lib.unit_layout(mcfg, 0, _lib.MT_STORE_PINNED_DMA | _lib.MT_STORE_MASTER_FP32 | _lib.MT_STORE_GRAD_ACCUM)
    for r in range(6):
        assert pinned.region_off[r] == both.region_off[r] and pinned.region_bytes[r] == both.region_bytes[r]
    assert pinned.block_bytes == both.block_bytes
    st = HostStore(cfg)
    try:  # no accumulator, no master copy
        for u in (MT_UNIT_EMBED, MT_UNIT_HEAD, 0, cfg.layers - 1):
            L = st.layout_of(u)
            for r in range(4):  # a pageable block is contiguous
                assert st.region_addr(u, r) == st.block_addr(u) + L.region_off[r]
            with pytest.raises(MtError) as e:
                st.region_addr(u, 4)
            assert e.value.code == -6
        with pytest.raises(MtError):
            st.region_addr(0, 6)
        g = np.zeros(st.layout_of(0).w_bytes // 2, np.uint16)
        with pytest.raises(MtError) as e:
            call("mt_grad_accumulate", st.ptr, 0, g.ctypes.data_as(ctypes.c_void_p))
        assert e.value.code == -6
        with pytest.raises(MtError):
            call("mt_store_sync_master", st.ptr)
    finally:
        st.close()
    st = HostStore(cfg, master=True)
    try:  # the seeded fill leaves P = fp32(W)
        st.fill_normal()
        for u in (MT_UNIT_EMBED, MT_UNIT_HEAD, 0):
            assert np.array_equal(st.region(u, REGION_P), synth.bf16_bits_to_f32(st.region(u, REGION_W)))
    finally:
        st.close()


def test_store_checkpoint_round_trip(lib, tmp_path):
    """save/load restore every region (incl. the optional ones and the
    accumulation counts) and t; a file for another config or other flags is
    refused; a missing file is an I/O error."""
    cfg = synth.preset("tiny")
    st = HostStore(cfg, master=True, accum=True)
    st2 = HostStore(cfg, master=True, accum=True)
    try:
        st.fill_normal()
        rng = np.random.default_rng(5)
        n = st.layout_of(1).w_bytes // 2
        g = synth.f32_to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
        call("mt_step", st.ptr, 1, g.ctypes.data_as(ctypes.c_void_p), ctypes.byref(_lib.adam_cfg(synth.AdamCfg())), 1,
             None)
        call("mt_grad_accumulate", st.ptr, 0, g.ctypes.data_as(ctypes.c_void_p))  # a pending accumulation
        path = tmp_path / "store.ckpt"
        st.save(path, 7)
        assert st2.load(path) == 7
        for u in st.units:
            for r in range(6):
                assert np.array_equal(st.region(u, r), st2.region(u, r)), (u, r)
        # the restored accumulation count: the next step on unit 0 averages 2 micro-batches in both
        outs = []
        for s_ in (st, st2):
            w = np.zeros(n, np.float32)
            call("mt_step", s_.ptr, 0, g.ctypes.data_as(ctypes.c_void_p), ctypes.byref(_lib.adam_cfg(synth.AdamCfg())),
                 2, w.ctypes.data_as(ctypes.c_void_p))
            outs.append(w)
        assert np.array_equal(outs[0], outs[1])
        other = HostStore(cfg)
        try:
            with pytest.raises(MtError) as e:
                other.load(path)
            assert e.value.code == -1
        finally:
            other.close()
        with pytest.raises(MtError) as e:
            st2.load(tmp_path / "missing.ckpt")
        assert e.value.code == -7
    finally:
        st.close()
        st2.close()


def test_tied_head_pack_and_summed_embedding_gradient(lib):
    """Tied weights: the head's device slot is packed as [final gain | E] in
    the untied head layout, and the embedding's landed gradient is bf16 of
    the head's bf16 gradient plus the token rows, as the oracle sums them."""
    import dataclasses
    cfg = dataclasses.replace(synth.preset("tiny"), tied=True)
    st = HostStore(cfg)
    try:
        st.fill_normal()
        assert [n for n, _ in tensor_shapes(cfg, MT_UNIT_HEAD)] == ["g_final"]
        dev = _lib.unit_layout(_lib.model_cfg(dataclasses.replace(cfg, tied=False)), MT_UNIT_HEAD)
        slab = np.full(dev.w_bytes // 2, 0x7777, dtype=np.uint16)
        call("mt_pack_head_tied", st.ptr, slab.ctypes.data_as(ctypes.c_void_p), slab.nbytes)
        h, V = cfg.hidden, cfg.vocab
        assert np.array_equal(slab[:h], st.tensor(MT_UNIT_HEAD, "g_final"))
        assert not slab[h:dev.tensor_off[1] // 2].any()
        off = dev.tensor_off[1] // 2
        assert np.array_equal(slab[off:off + V * h].reshape(V, h), st.tensor(MT_UNIT_EMBED, "embed"))
        rng = np.random.default_rng(4)
        T = 300
        tok = rng.integers(0, V // 3, T).astype(np.int32)  # most rows absent
        dx0 = (rng.standard_normal((T, h)) * 1e-2).astype(np.float32)
        hg = synth.f32_to_bf16_bits((rng.standard_normal((V, h)) * 1e-3).astype(np.float32))
        call("mt_embed_grad_tied", st.ptr, tok.ctypes.data_as(ctypes.c_void_p), T, dx0.ctypes.data_as(ctypes.c_void_p),
             hg.ctypes.data_as(ctypes.c_void_p))
        ref = oracle.embed_bwd(dx0, tok, V, init=synth.bf16_bits_to_f32(hg))
        assert np.array_equal(st.tensor(MT_UNIT_EMBED, "embed", REGION_G), synth.f32_to_bf16_bits(ref))
        untied = HostStore(synth.preset("tiny"))
        try:
            with pytest.raises(MtError):
                call("mt_pack_head_tied", untied.ptr, slab.ctypes.data_as(ctypes.c_void_p), slab.nbytes)
        finally:
            untied.close()
    finally:
        st.close()


def test_host_adam_scalar_path_equals_simd(lib, monkeypatch):
    """The AVX-512 and scalar paths give identical bits (checked in a subprocess)."""
    import subprocess
    import sys
    code = r'''
import ctypes, numpy as np, synth
from host_memory_centric_amd import _lib
from host_memory_centric_amd.store import HostStore
cfg = synth.preset("tiny")
st = HostStore(cfg); st.fill_normal()
n = st.layout_of(0).w_bytes // 2
g = synth.f32_to_bf16_bits((np.random.default_rng(1).standard_normal(n) * 1e-3).astype(np.float32))
out = np.zeros(n, np.float32)
_lib.call("mt_step", st.ptr, 0, g.ctypes.data_as(ctypes.c_void_p), ctypes.byref(_lib.adam_cfg(synth.AdamCfg())), 1,
          out.ctypes.data_as(ctypes.c_void_p))
# the extended path: master weights and three accumulated micro-batches
st2 = HostStore(cfg, master=True, accum=True); st2.fill_normal()
rng = np.random.default_rng(2)
for i in range(3):
    gi = synth.f32_to_bf16_bits((rng.standard_normal(n) * 1e-3).astype(np.float32))
    _lib.call("mt_grad_accumulate" if i < 2 else "mt_step", st2.ptr, 0, gi.ctypes.data_as(ctypes.c_void_p),
              *((ctypes.byref(_lib.adam_cfg(synth.AdamCfg())), 1, None) if i == 2 else ()))
import sys; sys.stdout.write(out.view(np.uint32).tobytes().hex()[:200000])
sys.stdout.write(st2.region(0, 4).view(np.uint32).tobytes().hex()[:200000])
'''
    env = dict(os.environ, PYTHONPATH=ROOT)
    a = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    env["MT_NO_AVX512"] = "1"
    b = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT)
    assert a.returncode == 0 and b.returncode == 0, a.stderr + b.stderr
    assert a.stdout == b.stdout and len(a.stdout) > 1000


def test_embed_gather_and_grad(lib):
    cfg = synth.preset("tiny")
    st = HostStore(cfg)
    try:
        bits = synth.make_weights(cfg)
        st.load_bits(bits)
        tok = synth.make_tokens(cfg).reshape(-1).astype(np.int32)
        T = tok.size
        x0 = np.zeros((T, cfg.hidden), np.uint16)
        call("mt_embed_gather", st.ptr, tok.ctypes.data_as(ctypes.c_void_p), T, x0.ctypes.data_as(ctypes.c_void_p))
        assert np.array_equal(x0, bits["embed"][tok])
        # repeated tokens exercise the ordered accumulation
        tok[::3] = tok[0]
        dx0 = np.random.default_rng(2).standard_normal((T, cfg.hidden)).astype(np.float32)
        call("mt_embed_grad", st.ptr, tok.ctypes.data_as(ctypes.c_void_p), T, dx0.ctypes.data_as(ctypes.c_void_p))
        ref = synth.f32_to_bf16_bits(oracle.embed_bwd(dx0, tok, cfg.vocab))
        assert np.array_equal(st.tensor(MT_UNIT_EMBED, "embed", REGION_G), ref)
        bad = tok.copy()
        bad[5] = cfg.vocab
        with pytest.raises(MtError):
            call("mt_embed_gather", st.ptr, bad.ctypes.data_as(ctypes.c_void_p), T, x0.ctypes.data_as(ctypes.c_void_p))
    finally:
        st.close()


@pytest.mark.parametrize("name,seq", [("tiny", 128), ("lc512k", 524288)])
def test_rope_tables_match_oracle(lib, name, seq):
    cfg = synth.preset(name)
    half = cfg.head_dim // 2
    cs = np.empty((seq, half), np.float32)
    sn = np.empty_like(cs)
    call("mt_rope_tables", ctypes.byref(_lib.model_cfg(cfg)), seq, cs.ctypes.data_as(ctypes.c_void_p),
         sn.ctypes.data_as(ctypes.c_void_p))
    rc, rs = oracle.rope_tables(seq, cfg.head_dim, cfg.rope_base)
    # independent fp64 evaluations (two libms) rounded to fp32: they may differ
    # by one fp32 rounding step, i.e. at most one ulp of 1.0, and rarely
    assert np.abs(cs - rc).max() <= 2.0 ** -23 and np.abs(sn - rs).max() <= 2.0 ** -23
    assert (cs != rc).mean() < 1e-3 and (sn != rs).mean() < 1e-3


# ----------------------------------------------------------------------------
# schedule planning (host logic)
# ----------------------------------------------------------------------------

def _loads(L, K, slots, resident=False):
    ops = plan_step(L, K, resident)
    units = [-2 if k == "head" else l for k, l, _ in ops]
    slot_of, load = plan_slots(units, slots)
    return ops, units, slot_of, load


def test_plan_orders_ops_as_the_method():
    ops, units, slot_of, load = _loads(8, 4, 2)
    kinds = [(k, l) for k, l, _ in ops]
    assert kinds[:8] == [("fwd", l) for l in range(8)]
    assert kinds[8] == ("head", None)
    # last block: backward straight away (internals kept in the forward)
    assert kinds[9:13] == [("bwd", 7), ("bwd", 6), ("bwd", 5), ("bwd", 4)]
    # earlier block: recompute, then backward top-down
    assert kinds[13:] == [("refwd", 0), ("refwd", 1), ("refwd", 2), ("refwd", 3),
                          ("bwd", 3), ("bwd", 2), ("bwd", 1), ("bwd", 0)]


@pytest.mark.parametrize("L,K", [(32, 4), (4, 1), (2, 1)])
def test_one_slot_loads_every_change(L, K):
    # one slot (no double buffering): every use of another unit than the op
    # before it is a load into the same slot
    _, units, slot_of, load = _loads(L, K, 1)
    assert set(slot_of) == {0}
    assert load == [i == 0 or units[i] != units[i - 1] for i in range(len(units))]


@pytest.mark.parametrize("L,K", [(32, 4), (48, 4), (180, 4), (24, 4), (4, 1), (2, 1)])
def test_two_slot_load_count(L, K):
    _, units, slot_of, load = _loads(L, K, 2)
    nblk = L // K
    # forward L + head; the last block's backward reloads all but its top layer
    # (the head took the other slot); every other block streams K layers for
    # the recompute and K - 2 more for the backward (its top two are resident)
    if K >= 2:
        expect = L + 1 + (K - 1) + (nblk - 1) * (2 * K - 2)
    else:
        expect = L + 1 + 0 + (nblk - 1) * 1
    assert sum(load) == expect
    # no two consecutive uses evict each other's slot while both are needed
    for i in range(1, len(units)):
        if units[i] != units[i - 1]:
            assert slot_of[i] != slot_of[i - 1]


def test_k_slot_keeps_recomputed_block_resident():
    L, K = 32, 4
    _, units, slot_of, load = _loads(L, K, K + 1)
    # at most: forward + head + the recompute of every block but the last
    assert sum(load) <= L + 1 + (L // K - 1) * K
    assert sum(load) < sum(_loads(L, K, 2)[3])


def test_resident_loads_each_unit_once():
    ops, units, slot_of, load = _loads(6, 6, 7, resident=True)
    assert sum(load) == 7
    assert not any(k == "refwd" for k, _, _ in ops)


@pytest.mark.parametrize("L", [1, 2, 3, 5, 7, 9])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_plan_invariants_any_depth(L, K):
    """For any depth and checkpoint interval (the last block may be short):
    one forward and one backward per layer, the head between them, backward
    top-down, every block but the last recomputed (bottom-up, before its
    backward) from its checkpoint, saved-buffer indices within the block;
    and for any slot count the slot plan keeps every used unit resident,
    loads exactly when it is not, and never reuses the slot of the op just
    before."""
    for resident in (False, True):
        Kr = L if resident else K
        ops = plan_step(L, K, resident)
        kinds = [(k, l) for k, l, _ in ops]
        assert [l for k, l in kinds if k == "fwd"] == list(range(L))
        assert [l for k, l in kinds if k == "bwd"] == list(reversed(range(L)))
        h = kinds.index(("head", None))
        assert all(k == "fwd" for k, _ in kinds[:h]) and all(k != "fwd" for k, _ in kinds[h + 1:])
        nblk = (L + Kr - 1) // Kr
        for b in range(nblk):
            lo, hi = b * Kr, min(L, (b + 1) * Kr)
            re = [i for i, (k, l) in enumerate(kinds) if k == "refwd" and lo <= l < hi]
            if b == nblk - 1:
                assert not re
            else:
                assert [kinds[i][1] for i in re] == list(range(lo, hi))
                assert max(re) < kinds.index(("bwd", hi - 1)) and min(re) > kinds.index(("bwd", hi))
        for k, l, si in ops:
            if k in ("refwd", "bwd"):
                assert si == l - (l // Kr) * Kr
            elif k == "fwd":
                last0 = (nblk - 1) * Kr
                assert si == (l - last0 if l >= last0 else None)
        units = [-2 if k == "head" else l for k, l, _ in ops]
        for slots in sorted({1, 2, 3, Kr + 1}):
            slot_of, load = plan_slots(units, slots)
            content = [None] * slots
            for i, u in enumerate(units):
                assert load[i] == (u not in content)
                if load[i] and slots > 1 and i > 0:
                    assert slot_of[i] != slot_of[i - 1]
                content[slot_of[i]] = u
                assert content[slot_of[i]] == u and content.count(u) == 1


class _FakeEvent:
    """A gradient copy's completion event for the scheduler test: completes
    when the test says so (threading.Event), queried or waited on."""

    def __init__(self):
        import threading
        self.done = threading.Event()
        self.queries = 0

    def query(self):
        self.queries += 1
        return self.done.is_set()

    def synchronize(self):
        self.done.wait()


@pytest.mark.parametrize("by_priority", [False, True])
def test_update_scheduler_order(by_priority):
    """Jobs run only once their event has completed; events complete in
    submission order (one in-order stream); among the ready jobs the first
    submitted runs, or with priorities the lowest priority value; a thread
    with nothing ready waits on the first pending event instead of polling."""
    import time

    from host_memory_centric_amd.engine import UpdateScheduler
    sch = UpdateScheduler(by_priority=by_priority)
    ran = []
    evs = [_FakeEvent() for _ in range(6)]
    prio = [5, 4, 3, 2, 1, 0]  # like gradients of layers 5..0 arriving top-down
    futs = [sch.submit(prio[i], evs[i], ran.append, i) for i in range(6)]
    time.sleep(0.05)
    assert ran == []
    assert sum(e.queries for e in evs) <= 2  # no polling while nothing is ready
    # complete events 2, 1, 0 (the waiting thread wakes at 0, the last), then 5, 4, 3
    for e in reversed(evs[:3]):
        e.done.set()
    for f in futs[:3]:
        f.result(timeout=5)
    time.sleep(0.05)
    for e in reversed(evs[3:]):
        e.done.set()
    for f in futs:
        f.result(timeout=5)
    sch.shutdown()
    assert sorted(ran) == list(range(6))
    if not by_priority:
        assert ran == list(range(6))
    else:
        assert ran == [2, 1, 0, 5, 4, 3]


@pytest.mark.parametrize("L,K,slots,carry", [(48, 4, 5, 12), (48, 4, 2, 48), (9, 2, 3, 4), (5, 1, 1, 2), (8, 4, 5, 3)])
def test_carried_layers_plan(L, K, slots, carry):
    """Layers with slots of their own: every use of a carried layer is in its
    slot; the first pass loads it once (at its forward), a pass whose carried
    slots already hold the weights loads it never; the other units stay in
    the shared pool, and the step loads at least ``carry`` fewer times than
    without carried layers."""
    ops = plan_step(L, K, False)
    units = [-2 if k == "head" else l for k, l, _ in ops]
    fixed = {l: slots + i for i, l in enumerate(range(L - carry, L))}
    for warm in (False, True):
        slot_of, load = plan_slots(units, slots, fixed, set(fixed) if warm else ())
        for i, u in enumerate(units):
            if u in fixed:
                assert slot_of[i] == fixed[u]
                assert load[i] == (not warm and units.index(u) == i)
            else:
                assert slot_of[i] < slots
    cold = sum(plan_slots(units, slots, fixed)[1])
    warm = sum(plan_slots(units, slots, fixed, set(fixed))[1])
    assert cold - warm == carry
    assert warm <= sum(plan_slots(units, slots)[1]) - carry


@pytest.mark.parametrize("L", [1, 2, 5, 9, 32, 48, 180])
def test_carried_layers_evenly_spaced(L):
    """carried_layers(L, c) holds c layers; the L - c streamed ones are spread
    so that runs of carried layers between them differ by at most one, and the
    last layer streams whenever any does."""
    from host_memory_centric_amd.engine import carried_layers
    for c in range(L + 1):
        cl = carried_layers(L, c)
        assert len(cl) == c and cl == sorted(set(cl)) and all(0 <= l < L for l in cl)
        streamed = [l for l in range(L) if l not in cl]
        if streamed:
            assert streamed[-1] == L - 1
            runs = [b - a - 1 for a, b in zip([-1] + streamed[:-1], streamed)]
            assert max(runs) - min(runs) <= 1, (L, c, runs)


def test_carry_argument_checked(lib):
    from host_memory_centric_amd.engine import Trainer
    cfg = synth.preset("tiny")
    for kw in (dict(carry=1), dict(carry=3, pinned_store=True), dict(carry=1, mode="resident", pinned_store=True),
               dict(carry=-1, pinned_store=True)):
        with pytest.raises(ValueError, match="carry"):
            Trainer(cfg, synth.AdamCfg(), **kw)


@pytest.mark.parametrize("kw", [dict(offload_ckpt=5), dict(offload_ckpt=-1), dict(offload_ckpt=1, mode="resident"),
                                dict(offload_ckpt=3, ckpt_every=2)])
def test_offload_ckpt_argument_checked_before_any_allocation(lib, kw):
    """Host-held block checkpoints need a streamed step and leave at least the
    two top blocks on the device (6 layers: 6 blocks of 1, or 3 of 2)."""
    from host_memory_centric_amd.engine import Trainer
    cfg = synth.preset("tiny", layers=6, ckpt_every=1)
    with pytest.raises(ValueError, match="offload_ckpt"):
        Trainer(cfg, synth.AdamCfg(), **kw)


def test_device_entries_reject_bad_arguments_before_any_launch(lib):
    """The layer, head and bind entry points check shapes, pointers, alignment
    and buffer sizes on the host and return the documented code (with a
    message) before anything is enqueued: the fake, aligned device addresses
    below are never touched."""
    from host_memory_centric_amd._lib import MtAct, MtHeadIO, MtLayerView
    cfg = synth.preset("tiny")
    mc = _lib.model_cfg(cfg)
    base = 1 << 28  # a fake device address, 256-byte aligned
    ws = ctypes.c_size_t()
    _lib.call("mt_layer_workspace_bytes", ctypes.byref(mc), 2, 128, ctypes.byref(ws))
    view = MtLayerView()
    for j in range(6):
        view.w[j] = base + j * 4096
        view.g[j] = base + (1 << 20) + j * 4096

    def act(**kw):
        a = MtAct()
        a.batch, a.seq = 2, 128
        for f in ("x_in", "x_out", "dy", "dy_bf16", "dx", "dx_bf16", "rope_cos", "rope_sin", "workspace"):
            setattr(a, f, base)
        a.workspace_bytes = 1 << 40
        for k, v in kw.items():
            setattr(a, k, v)
        return a

    def code(name, *args):
        with pytest.raises(MtError) as e:
            _lib.call(name, *args)
        assert str(e.value).split(": ", 1)[1].strip()  # a message, not only the code
        return e.value.code

    def fwd(a, m=mc):
        return code("mt_layer_fwd", ctypes.byref(view), ctypes.byref(m), ctypes.byref(a), None)

    assert fwd(act(batch=0)) == -2                       # empty batch
    assert fwd(act(batch=2, seq=3)) == -2                # batch*seq not a multiple of 8
    assert fwd(act(x_in=None)) == -1                     # missing input
    assert fwd(act(x_out=base + 8)) == -3                # misaligned output
    assert fwd(act(workspace_bytes=ws.value - 256)) == -1  # workspace too small (no saved buffer)
    assert fwd(act(saved=base, saved_bytes=16, workspace_bytes=ws.value)) == -1  # saved buffer too small
    assert fwd(act(), _lib.model_cfg(cfg.with_(hidden=288, heads=3, head_dim=96))) == -2  # head_dim not 64 or 128
    assert code("mt_layer_recompute_bwd", ctypes.byref(view), ctypes.byref(mc), ctypes.byref(act(dy=None)),
                None) == -1
    hv = MtLayerView()
    for j in range(2):
        hv.w[j] = base + j * 4096
        hv.g[j] = base + (1 << 20) + j * 4096
    hio = MtHeadIO()
    hio.batch, hio.seq = 8, 1                            # no next token to predict
    hio.x = hio.tokens = hio.dx = hio.dx_bf16 = hio.loss = hio.workspace = base
    hio.workspace_bytes = 1 << 40
    assert code("mt_head_fwd_bwd", ctypes.byref(hv), ctypes.byref(mc), ctypes.byref(hio), None) == -2
    hio.batch, hio.seq, hio.workspace_bytes = 2, 128, 256
    assert code("mt_head_fwd_bwd", ctypes.byref(hv), ctypes.byref(mc), ctypes.byref(hio), None) == -1
    out = MtLayerView()
    assert code("mt_bind", ctypes.byref(mc), 0, ctypes.c_void_p(base + 128), None, ctypes.byref(out)) == -3
    assert code("mt_bind", ctypes.byref(mc), 0, None, None, ctypes.byref(out)) == -1


class _ClockEvent:
    """A timing event at a fixed moment of the event clock (ms)."""

    def __init__(self, t):
        self.t = t

    def elapsed_time(self, other):
        return other.t - self.t


def test_timeline_report_host_updates():
    """bench.py's merged timeline puts the host updates on the event clock
    (shifted by the smallest delay between a backward's end and the moment the
    copy thread saw it) and the report counts the share of the window in which
    updates run."""
    import bench
    E = _ClockEvent
    # two steps of 100 ms: a forward 0..40, a backward 40..90 (one layer), a
    # copy out 90..95 and one update; the host clock runs 1000 s ahead and the
    # copy thread sees each backward 0.5 ms late (2 ms the second time)
    raws = []
    for s in range(2):
        b = 100.0 * s
        h0 = 1000.0 + b * 1e-3
        raws.append({"ref": E(b), "ops": [("fwd", E(b), E(b + 40)), ("bwd", E(b + 40), E(b + 90))],
                     "h2d": [(E(b), E(b + 10))], "d2h": [(E(b + 90), E(b + 95))],
                     "host": [("bwd_done", 0, h0 + (90.5 + 1.5 * s) * 1e-3, h0 + (90.5 + 1.5 * s) * 1e-3),
                              ("update", 0, h0 + 95.5e-3, h0 + 120.5e-3)],
                     "t_host": 1000.0 if s == 0 else 1000.1})
    tl = bench.merged_timeline(raws)
    upd = [x for k, _, a, b in tl["host"] if k == "update" for x in (a, b)]
    assert upd == pytest.approx([95.0, 120.0, 195.0, 220.0])
    rep = bench.overlap_report(tl, 2)
    # the window ends with the last op or copy (195 ms): 25 + 0 ms of updates inside it
    assert rep["window_ms"] == pytest.approx(195.0)
    assert rep["host_update_busy_frac"] == pytest.approx(25.0 / 195.0, abs=1e-4)
    assert rep["compute_busy_frac"] == pytest.approx(180.0 / 195.0, abs=1e-4)


def test_trainer_timeline_conversion():
    """Trainer.timeline() on a recorded timeline (events of a fixed clock):
    intervals relative to the step's reference event, host intervals shifted
    onto the event clock by the smallest delay after a backward's end."""
    from host_memory_centric_amd.engine import Trainer

    class _Done(_ClockEvent):
        def synchronize(self):
            pass

    class _T:
        def finish(self):
            pass
    E = _Done
    t = _T()
    t._tl = {"ref": E(10.0), "ops": [("fwd", E(10.0), E(20.0)), ("bwd", E(20.0), E(30.0)),
                                      ("bwd", E(30.0), E(40.0))],
             "h2d": [(E(10.0), E(15.0))], "d2h": [(E(30.0), E(35.0)), (E(40.0), E(45.0))],
             "host": [("bwd_done", 1, 5.0205, 5.0205), ("bwd_done", 0, 5.0312, 5.0312),
                      ("update", 1, 5.0355, 5.0455)],
             "t_host": 5.0}
    tl = Trainer.timeline(t)
    assert [x for _, a, b in tl["ops"] for x in (a, b)] == pytest.approx([0, 10, 10, 20, 20, 30])
    assert [x for a, b in tl["d2h"] for x in (a, b)] == pytest.approx([20, 25, 30, 35])
    # seen 20.5 and 31.2 ms after the step began on the host clock: shift 0.5 ms
    host = {(k, u): (a, b) for k, u, a, b in tl["host"]}
    assert host[("bwd_done", 0)] == pytest.approx((30.7, 30.7))
    assert host[("update", 1)] == pytest.approx((35.0, 45.0))


def test_update_scheduler_key():
    """With a sort key set, the ready jobs run in the key's order (the
    'carried' update order during the backward), and after set_key(None) by
    priority again."""
    from host_memory_centric_amd.engine import UpdateScheduler
    sch = UpdateScheduler(by_priority=True)
    try:
        for key, want in (((lambda p: (p % 2, p)), [5, 3, 1, 4, 2, 0]), (None, [5, 4, 3, 2, 1, 0])):
            sch.set_key(key)
            ran = []
            evs = [_FakeEvent() for _ in range(6)]
            futs = [sch.submit(5 - i, evs[i], ran.append, i) for i in range(6)]
            for e in reversed(evs):  # the waiting thread wakes at the first job's event, the last set
                e.done.set()
            for f in futs:
                f.result(timeout=5)
            assert ran == want
    finally:
        sch.shutdown()
