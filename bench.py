"""Throughput of layer-streamed full-parameter training on one MI355X.

One step = one full training step of the workload (streamed forward, head,
block recompute + backward, gradient offload, host Adam for every unit) over
one batch of seeded synthetic tokens.  Prints one JSON line:
tokens/s (value), executed and model TFLOPS against the bf16 dense MFMA peak,
host-link GB/s, the copy/compute overlap of the timed steps, the roofline of
the dominant kernel (HIP events around its launches in the timed steps), and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload 14b] [--mode streamed]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "training tokens/s + TFLOPS (% bf16 MFMA peak), host-link GB/s, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)

WORKLOADS = ("7b", "14b", "depth180", "width5x", "lc128k", "lc256k", "lc512k", "tiny")


def workload_text(cfg, slots):
    kind = {"7b": "7B-shaped", "14b": "14B-shaped", "depth180": "depth-stress", "width5x": "width-stress",
            "lc128k": "long-context 7B-layer", "lc256k": "long-context 7B-layer",
            "lc512k": "long-context 7B-layer", "tiny": "tiny"}.get(cfg.name, cfg.name)
    return (f"{kind} dense decoder ({cfg.layers} layers, hidden {cfg.hidden}, {cfg.heads} heads x {cfg.head_dim}, "
            f"SwiGLU ffn {cfg.ffn}, vocab {cfg.vocab}), batch {cfg.batch} x seq {cfg.seq}, checkpoint every "
            f"{cfg.ckpt_every} layers, {slots} device staging slots")


def flops_per_step(cfg, ops):
    T, h, f, V, B, S = cfg.tokens, cfg.hidden, cfg.ffn, cfg.vocab, cfg.batch, cfg.seq
    lin = 2.0 * T * (4 * h * h + 3 * h * f)
    attn = 2.0 * B * S * (S + 1) * h  # causal: scores and products on and below the diagonal
    head = 2.0 * T * h * V
    n_fwd = sum(1 for k, _, _ in ops if k in ("fwd", "refwd"))
    n_bwd = sum(1 for k, _, _ in ops if k == "bwd")
    exec_ = n_fwd * (lin + attn) + n_bwd * (2 * lin + 2.5 * attn) + 3 * head
    model = 3.0 * (cfg.layers * (lin + 2.0 * B * S * S * h) + head)
    return exec_, model


def gemm_source_hash():
    """Hash of the GEMM kernel sources with comments and blank lines removed,
    so that the committed counter figures stay valid across comment edits and
    are dropped (null) once any code changes."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "host_memory_centric_amd", "csrc")
    code = []
    for f in ("gemm.hip", "gemm_kernel.h", "gemm_pipe.h", "gemm_pp.h"):
        for line in open(os.path.join(csrc, f)):
            line = re.sub(r"//.*", "", line).rstrip()
            if line:
                code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of a GEMM class from the committed rocprofv3 PMC
    summary of the workload (profiles/gemm_<workload>_traffic.md), or None if
    there is none or the GEMM sources changed since it was taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    if gemm_source_hash() != data.get("source_sha256_16"):
        return None
    k = data.get("kernels", {}).get(kernel)
    return k["hbm_bytes"] if k else None


def measured_mfma_busy(kernel, workload):
    """Fraction of cycles the MFMA units are busy in a GEMM class, from the
    committed rocprofv3 PMC summary of the workload
    (profiles/mfma_util_<workload>_gemm_attention.md), or None if there is
    none or the GEMM sources changed since it was taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"mfma_util_{workload}_gemm_attention.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    data = json.loads(m.group(1))
    if gemm_source_hash() != data.get("source_sha256_16"):
        return None
    k = data.get("kernels", {}).get(kernel)
    return k["mfma_busy_frac"] if k else None


def _union(iv):
    out = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _total(u):
    return sum(b - a for a, b in u)


def _inter(u, w):
    i = j = 0
    t = 0.0
    while i < len(u) and j < len(w):
        a, b = max(u[i][0], w[j][0]), min(u[i][1], w[j][1])
        if a < b:
            t += b - a
        if u[i][1] < w[j][1]:
            i += 1
        else:
            j += 1
    return t


def merged_timeline(raws):
    """One event timeline over consecutive steps (ms from the first step's
    start): the steps' op, weight-copy and gradient-copy intervals, and the
    host updates moved onto the event clock (a backward's end is seen by the
    host thread that waits for it a little later; the smallest difference
    gives the shift between the clocks)."""
    rel = raws[0]["ref"].elapsed_time
    t0 = raws[0]["t_host"]
    out = {"ops": [], "h2d": [], "d2h": [], "host": []}
    shifts = []
    for tl in raws:
        ops = [(k, rel(a), rel(b)) for k, a, b in tl["ops"]]
        host = [(k, u, 1e3 * (a - t0), 1e3 * (b - t0)) for k, u, a, b in tl["host"]]
        bwd_end = [e for k, _, e in ops if k == "bwd"]
        seen = [a for k, _, a, _ in host if k == "bwd_done"]
        if len(seen) == len(bwd_end):
            shifts += [a - e for a, e in zip(seen, bwd_end)]
        out["ops"] += ops
        out["h2d"] += [(rel(a), rel(b)) for a, b in tl["h2d"]]
        out["d2h"] += [(rel(a), rel(b)) for a, b in tl["d2h"]]
        out["host"] += host
    shift = min(shifts) if shifts else 0.0
    out["host"] = [(k, u, a - shift, b - shift) for k, u, a, b in out["host"]]
    return out


def overlap_report(tl, n_steps=1):
    """Busy and overlap fractions over the timed steps from their event
    timeline: the share of host-to-device and device-to-host copy time during
    which the compute stream is running a layer, head or backward op, and the
    share of the window in which the host optimizer thread runs updates.  The
    window runs from the first step's start to the last copy or op."""
    comp = _union([(a, b) for _, a, b in tl["ops"]])
    h2d, d2h = _union(tl["h2d"]), _union(tl["d2h"])
    copies = _union(tl["h2d"] + tl["d2h"])
    span = max([b for _, _, b in tl["ops"]] + [b for _, b in tl["h2d"] + tl["d2h"]])
    # the host optimizer thread's updates inside the window
    upd = _union([(max(a, 0.0), min(b, span)) for k, _, a, b in tl.get("host", ())
                  if k == "update" and b > 0.0 and a < span])

    def frac(x, y):
        return round(x / y, 4) if y > 0 else None
    return {"window_ms": round(span, 2), "steps": n_steps, "step_ms": round(span / n_steps, 2),
            "compute_busy_frac": frac(_total(comp), span),
            "h2d_busy_frac": frac(_total(h2d), span), "d2h_busy_frac": frac(_total(d2h), span),
            "h2d_overlap_frac": frac(_inter(h2d, comp), _total(h2d)),
            "d2h_overlap_frac": frac(_inter(d2h, comp), _total(d2h)),
            "copy_overlap_frac": frac(_inter(copies, comp), _total(copies)),
            "gpu_busy_ms_per_step": round(_total(comp) / n_steps, 2),
            "gpu_idle_ms_per_step": round((span - _total(comp)) / n_steps, 2),
            "host_update_busy_frac": frac(_total(upd), span) if upd else None}


def host_probe(tr, reps=3, master=False):
    """Host DRAM rates of the two host-side passes, measured on layer 0 after
    the timed steps with the GPU idle: the packer (W region -> pinned slab,
    read + non-temporal write, 4 bytes per parameter; not run with a pinned
    store, which has no packer copy) and the Adam step (slab read, G written,
    W/m/v read and written, 24 bytes per parameter; with a pinned store the
    gradient is already in G: G read, 22 bytes per parameter).  The Adam
    calls advance layer 0's optimizer state; nothing runs after."""
    import ctypes

    from host_memory_centric_amd._lib import call
    lay = tr.lay
    params = lay.w_bytes // 2
    tr.finish()
    out = {"threads": len(os.sched_getaffinity(0)), "pack_ms_per_layer": None, "pack_GBps": None}
    if not tr.direct:
        t = time.perf_counter()
        for _ in range(reps):
            call("mt_pack_layer", tr.store.ptr, 0, tr.wslab[0].ptr, tr.slot_bytes)
        pack_s = (time.perf_counter() - t) / reps
        out.update(pack_ms_per_layer=round(1e3 * pack_s, 2), pack_GBps=round(4 * params / pack_s / 1e9, 1))
    src = None if tr.direct else tr.gslab[0].ptr
    step_t = tr.t + 1
    t = time.perf_counter()
    for i in range(reps):
        call("mt_step", tr.store.ptr, 0, src, ctypes.byref(tr.madam), step_t + i, None)
    adam_s = (time.perf_counter() - t) / reps
    # a master copy: fp32 weight read instead of bf16, fp32 write
    adam_b = (22 if tr.direct else 24) + (6 if master else 0)
    out.update(adam_ms_per_layer=round(1e3 * adam_s, 2), adam_GBps=round(adam_b * params / adam_s / 1e9, 1))
    return out


def probe_mfma(tr, iters=100000):
    """Sustained bf16 MFMA rate of this GPU (mt_probe_mfma: independent MFMA
    chains on every SIMD, no memory traffic, ~50 ms after a warm-up): the peak
    the chip holds under MFMA load, beside the published 2.4 GHz figure."""
    import ctypes

    import torch

    from host_memory_centric_amd import _lib
    sink = torch.empty(2048, dtype=torch.float32, device=tr.dev)
    out = ctypes.c_double()
    _lib.call("mt_probe_mfma", iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(tr.s_comp.cuda_stream),
              ctypes.byref(out))
    return round(out.value, 1)


def link_probe(tr, nbytes=1 << 30, reps=3):
    """Pinned host <-> device copy rates on this machine: each direction alone and
    both at once (the trainer's weight and gradient streams)."""
    import torch

    from host_memory_centric_amd import _lib
    from host_memory_centric_amd.engine import PinnedBuffer
    hb = [PinnedBuffer(nbytes) for _ in range(2)]
    db = [torch.empty(nbytes, dtype=torch.uint8, device=tr.dev) for _ in range(2)]
    sh, sd = tr.s_h2d, tr.s_d2h
    import ctypes

    def run(h2d, d2h):
        torch.cuda.synchronize()
        evs = {}
        for name, on, st in (("h2d", h2d, sh), ("d2h", d2h, sd)):
            if not on:
                continue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            for _ in range(reps):
                if name == "h2d":
                    _lib.call("mt_copy_h2d", ctypes.c_void_p(db[0].data_ptr()), hb[0].ptr, nbytes,
                              ctypes.c_void_p(st.cuda_stream))
                else:
                    _lib.call("mt_copy_d2h", hb[1].ptr, ctypes.c_void_p(db[1].data_ptr()), nbytes,
                              ctypes.c_void_p(st.cuda_stream))
            e1.record(st)
            evs[name] = (e0, e1)
        torch.cuda.synchronize()
        return {k: round(reps * nbytes / (a.elapsed_time(b) * 1e-3) / 1e9, 2) for k, (a, b) in evs.items()}
    try:
        run(True, True)  # warm up
        alone_h, alone_d, both = run(True, False), run(False, True), run(True, True)
    finally:
        for b in hb:
            b.free()
    return {"h2d_GBps": alone_h["h2d"], "d2h_GBps": alone_d["d2h"], "bidir_h2d_GBps": both["h2d"],
            "bidir_d2h_GBps": both["d2h"], "probe_bytes": nbytes}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg):
    """The fp32 CPU oracle on this host, timed on a bounded sample of the
    step: one whole layer forward + backward over the full batch (every
    token of the step), the head (final norm, LM head, cross entropy and
    their backward) over the full batch, and one layer's Adam; the step's
    time is extrapolated from them (layers x (layer + Adam) + head + the
    embedding's and head's Adam at the layer's rate per parameter)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    import synth

    B, S, h, V, f = cfg.batch, cfg.seq, cfg.hidden, cfg.vocab, cfg.ffn
    T = B * S
    W = {}
    for j, (k, shp) in enumerate(synth.layer_tensor_shapes(cfg).items()):
        W[k] = (np.ones(shp, np.float32) if k.startswith("g_") else
                synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(500 + j, shp, std=0.02)))
    x = synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(510, (T, h), std=1.0))
    dy = synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(511, (T, h), std=1e-3))
    cos, sin = oracle.rope_tables(S, cfg.head_dim, cfg.rope_base)
    t0 = time.perf_counter()
    y, cache = oracle.layer_fwd(x, W, cfg, cos, sin)
    oracle.layer_bwd(dy, cache, W, cfg, cos, sin)
    t_layer = time.perf_counter() - t0
    del cache
    head = synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(512, (V, h), std=0.02))
    tok = synth.tokens(0, V, B, S)
    t0 = time.perf_counter()
    oracle.head_fwd_bwd(y, np.ones(h, np.float32), head, tok, cfg)
    t_head = time.perf_counter() - t0
    del head, y
    P_L = sum(v.size for v in W.values())
    t0 = time.perf_counter()
    for j, (k, v) in enumerate(W.items()):
        g = synth.bf16_bits_to_f32(synth.torch_normal_bf16_bits(520 + j, v.shape, std=1e-3))
        oracle.adam_update(synth.f32_to_bf16_bits(v), g, np.zeros(v.shape, np.float32),
                           np.zeros(v.shape, np.float32), synth.AdamCfg(), 1)
    t_adam = time.perf_counter() - t0
    lin = 2.0 * T * (4 * h * h + 3 * h * f)
    attn = 2.0 * B * S * (S + 1) * h
    flops = 3 * lin + 3.5 * attn + 6.0 * T * h * V  # the sample's forward + backward
    sample_s = t_layer + t_head + t_adam
    t_step = cfg.layers * (t_layer + t_adam) + t_head + t_adam * (2 * V * h + h) / P_L
    blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": round(T / t_step, 3), "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": (f"fp32 numpy oracle on the full batch ({B} x {S} tokens): one layer forward+backward "
                       f"{t_layer:.2f} s, head forward+backward {t_head:.2f} s, one layer's Adam ({P_L} params) "
                       f"{t_adam:.2f} s (total {sample_s:.1f} s); the step is {cfg.layers} x (layer + Adam) + head "
                       f"+ embedding/head Adam"),
            "step_s_est": round(t_step, 2), "blas_threads": int(max(blas)) if blas else None,
            "cpu_model": _cpu_model(), "fp32_gflops": round(flops / (t_layer + t_head) / 1e9, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="14b", choices=WORKLOADS)
    ap.add_argument("--mode", default="streamed", choices=["streamed", "resident"])
    ap.add_argument("--slots", type=int, default=5)
    ap.add_argument("--grad-slabs", type=int, default=16)
    ap.add_argument("--grad-slots", type=int, default=4, help="device gradient slots the backward writes in turn")
    ap.add_argument("--update-order", default="carried", choices=["arrival", "urgent", "tail", "carried"],
                    help="order of the host updates: as gradients arrive, most urgent for the next step first, "
                         "as they arrive until the backward ends and most urgent first after it, or carried "
                         "layers first during the backward and most urgent first after it")
    ap.add_argument("--carry", type=int, default=None,
                    help="layers that keep a device slot of their own across steps, refilled right after "
                         "their host update (page-locked store only); default: half the layers for the "
                         "14B-shaped workload with a page-locked store, else 0")
    ap.add_argument("--pageable-store", dest="pinned_store", action="store_false",
                    help="keep the whole store pageable and stream through the packer and the gradient slabs; "
                         "default: the store's W and G regions page-locked, weights and gradients copied directly")
    ap.add_argument("--ckpt-every", type=int, default=None, help="override the workload's checkpoint interval")
    ap.add_argument("--micro-batches", type=int, default=1,
                    help="micro-batches per optimizer step (gradients accumulated on the host)")
    ap.add_argument("--master", action="store_true", help="keep fp32 master weights in the host store")
    ap.add_argument("--batch", type=int, default=None, help="override the workload's batch (sequences per pass)")
    ap.add_argument("--adam-threads", type=int, default=0, help="host threads of the optimizer calls (0: all)")
    ap.add_argument("--seq", type=int, default=None, help="override the workload's sequence length")
    ap.add_argument("--layers", type=int, default=None, help="override the workload's layer count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timeline-out", default=None, help="write the event timeline of the timed steps as JSON")
    ap.add_argument("--no-timeline", action="store_true",
                    help="record no copy/compute event timeline during the timed steps")
    ap.add_argument("--progress", action="store_true",
                    help="print each op as it is enqueued (the enqueue runs a few ops ahead of the GPU)")
    ap.add_argument("--offload-ckpt", type=int, default=0,
                    help="hold the checkpoints of the first N blocks in host memory (long contexts)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU sharding or collectives; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from host_memory_centric_amd import _lib
    from host_memory_centric_amd.engine import Trainer

    cfg = synth.preset(args.workload)
    if any(v is not None for v in (args.ckpt_every, args.batch, args.seq, args.layers)):
        import dataclasses
        cfg = dataclasses.replace(cfg, ckpt_every=args.ckpt_every or cfg.ckpt_every, batch=args.batch or cfg.batch,
                                  seq=args.seq or cfg.seq, layers=args.layers or cfg.layers)
    adam = synth.AdamCfg()
    if args.carry is None:  # 14B-shaped default: every other layer carried, the others stream
        args.carry = cfg.layers // 2 if (cfg.name == "14b" and args.pinned_store and args.mode == "streamed") else 0
    t_init = time.perf_counter()
    nmb = max(1, args.micro_batches)
    _lib.load()
    _lib.call("mt_set_optimizer_threads", args.adam_threads)
    tr = Trainer(cfg, adam, mode=args.mode, n_slots=args.slots, n_grad_slabs=args.grad_slabs, device="cuda:0",
                 micro_batches=nmb, master=args.master, pinned_store=args.pinned_store,
                 update_order=args.update_order, offload_ckpt=args.offload_ckpt, carry=args.carry,
                 grad_slots=args.grad_slots)

    if args.progress:
        t_prog = time.perf_counter()

        def progress(kind, layer):
            print(f"[bench] {time.perf_counter() - t_prog:8.1f} s  {kind} {'' if layer is None else layer}",
                  file=sys.stderr, flush=True)
        tr.progress = progress

    def tokens(step):
        return np.concatenate([synth.make_tokens(cfg, step * nmb + i) for i in range(nmb)], axis=0)
    t_init = time.perf_counter() - t_init
    print(f"[bench] init {t_init:.1f} s, weight loads/step {tr.n_weight_loads()}", file=sys.stderr, flush=True)
    step = 0
    for _ in range(args.warmup):
        loss = tr.step(tokens(step))
        step += 1
        print(f"[bench] warmup step {step}: loss {loss:.4f} {tr.stats['step_s']:.3f} s", file=sys.stderr, flush=True)
    # the warm-up's host updates (and the weight copies they enqueue) are not
    # work of the timed steps: they finish before the timed region opens, as
    # the timed steps' own finish inside it
    tr.finish()
    torch.cuda.synchronize()
    _lib.prof_collect(reset=True)
    _lib.call("mt_prof_enable", 1)
    # the timed steps record their copy/compute event timeline (events only)
    tr.record_timeline = not args.no_timeline
    raws = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        loss = tr.step(tokens(step))
        step += 1
        raws.append(tr._tl)
        print(f"[bench] step {step}: loss {loss:.4f} {tr.stats['step_s']:.3f} s", file=sys.stderr, flush=True)
    tr.finish()  # the last step's host updates belong to the timed work
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    tr.record_timeline = False
    _lib.call("mt_prof_enable", 0)
    prof = _lib.prof_collect(reset=True)

    # the trainer's device footprint: taken before the probes allocate their buffers
    dev_peak = int(torch.cuda.max_memory_allocated())
    overlap = None
    if not args.no_timeline:
        tl = merged_timeline(raws)
        overlap = overlap_report(tl, args.steps)
    if args.timeline_out and overlap is not None:
        with open(args.timeline_out, "w") as fh:
            json.dump(tl, fh)
    link = link_probe(tr)
    mfma_probe = probe_mfma(tr)
    host = host_probe(tr, master=args.master)

    T = cfg.tokens * nmb  # tokens per optimizer step
    ms_step = 1e3 * dt / args.steps
    f_exec, f_model = (nmb * f for f in flops_per_step(cfg, tr.ops))
    tflops_exec = f_exec / (dt / args.steps) / 1e12
    tflops_model = f_model / (dt / args.steps) / 1e12
    lay, lay_h = tr.lay, tr.lay_head_dev
    n_loads = tr.n_weight_loads()  # per micro-batch pass
    # (block checkpoints held in host memory go out and come back once per pass)
    ck = nmb * tr.n_host * tr.ckpt_bytes
    h2d = (nmb * ((n_loads - 1) * lay.w_bytes + lay_h.w_bytes) + tr.n_carry_loads() * lay.w_bytes
           + T * cfg.hidden * 2 + T * 4 + ck)
    d2h = nmb * (cfg.layers * lay.w_bytes + lay_h.w_bytes) + T * cfg.hidden * 4 + ck
    dom = max(prof.items(), key=lambda kv: kv[1][1]) if prof else None
    roof = None
    if dom:
        name, (n, ms, fl) = dom
        ach = fl / (ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": name, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(name, args.workload), "traffic_unit": "HBM bytes per launch",
                "avg_launch_ms": round(ms / n, 4), "launches": n,
                # cycles the MFMA units are busy (rocprofv3 PMC, committed profile): the rest of the
                # gap to the published peak is the clock, which falls well below 2.4 GHz under this load
                "mfma_busy_frac_pmc": measured_mfma_busy(name, args.workload),
                # the same rate against the MFMA rate this GPU sustains (probe, same run)
                "frac_of_probed_peak": round(ach / mfma_probe, 4)}
    kernels = {k: {"launches": n, "avg_ms": round(ms / n, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 1),
                   "share_of_step": round(ms / (1e3 * dt), 3)} for k, (n, ms, fl) in prof.items()}
    out = {
        "metric": METRIC, "value": round(T * args.steps / dt, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (workload_text(cfg, tr.n_slots) if args.mode == "streamed" else
                                workload_text(cfg, tr.n_slots).replace(f"{tr.n_slots} device staging slots",
                                                                       "all layers resident on the device")) +
                   (f", {nmb} micro-batches per optimizer step" if nmb > 1 else "") +
                   (", fp32 master weights" if args.master else "") +
                   (", host store W/G page-locked (direct copies, no packer)" if args.pinned_store else "") +
                   (f", checkpoints of the first {tr.n_host} blocks in host memory" if tr.n_host else "") +
                   (f", {tr.carry} layers (all but {cfg.layers - tr.carry} evenly spaced) in device slots of their "
                    f"own, refilled after each update" if tr.carry else "") +
                   (f", {args.update_order} update order" if args.update_order != "arrival" else ""),
                   "name": cfg.name, "global_batch": cfg.batch * nmb,
                   "seq_len": cfg.seq, "micro_batches": nmb, "master_fp32": bool(args.master),
                   "mode": args.mode, "slots": tr.n_slots, "carried_layers": tr.carry,
                   "grad_slots": tr.n_gslots, "ckpt_every": tr.K,
                   "host_store": "pinned_dma" if args.pinned_store else "pageable",
                   "update_order": args.update_order, "ckpt_host_blocks": tr.n_host,
                   "parallelism": "none (1 GPU)"},
        "tflops_exec": round(tflops_exec, 1), "tflops_model": round(tflops_model, 1),
        "pct_peak_exec": round(100 * tflops_exec / PEAK_BF16_TFLOPS, 2),
        "pct_peak_model": round(100 * tflops_model / PEAK_BF16_TFLOPS, 2),
        "mfma_probe_tflops": mfma_probe,
        "pct_probe_exec": round(100 * tflops_exec / mfma_probe, 2),
        "h2d_GBps": round(h2d * args.steps / dt / 1e9, 2), "d2h_GBps": round(d2h * args.steps / dt / 1e9, 2),
        "weight_loads_per_step": n_loads * nmb + tr.n_carry_loads(), "dev_peak_bytes": dev_peak,
        "host_store_bytes": int(tr.store.total_bytes()), "loss": round(loss, 5), "kernels": kernels,
        "roofline": roof,
        "overlap": overlap,
        "link": dict(link, h2d_bytes_per_step=int(h2d), d2h_bytes_per_step=int(d2h),
                     h2d_link_frac=round(h2d / (ms_step * 1e-3) / (link["h2d_GBps"] * 1e9), 4),
                     h2d_active_GBps=(round(h2d / 1e9 / (overlap["h2d_busy_frac"] * overlap["step_ms"] * 1e-3), 2)
                                      if overlap else None)),
    }
    # host DRAM bytes of one step: with a pageable store every weight load is
    # packed once (4 B per parameter) and every parameter gets one Adam update
    # that lands its gradient from a slab (24 B); with a pinned store there is
    # no packing and Adam reads the gradient from G (22 B).  The DMA engines
    # read the H2D bytes from and write the D2H bytes to host memory; the
    # floor divides the sum by the faster of the measured host rates
    n_params = sum(tr.store.layout_of(u).w_bytes // 2 for u in tr.store.units)
    # (micro-batches: each accumulation reads the gradient and the accumulator and
    # writes the accumulator, 10 B per parameter, and the final step also
    # reads the accumulator; a master copy adds 6 B: fp32 read instead of bf16, fp32 write)
    adam_b = (22 if tr.direct else 24) + (4 if nmb > 1 else 0) + (6 if args.master else 0)
    pack_b = 0 if tr.direct else nmb * (4 * (lay.w_bytes // 2) * (n_loads - 1) + 4 * (lay_h.w_bytes // 2))
    # (checkpoints in host memory: a host copy out of the slab each, and one back into it
    # for all but the two that are still in their slabs, each read plus write)
    ck_copy = 2 * nmb * (tr.n_host + max(0, tr.n_host - 2)) * tr.ckpt_bytes
    host_bytes = pack_b + adam_b * n_params + 10 * (nmb - 1) * n_params + h2d + d2h + ck_copy
    host["bytes_per_step"] = int(host_bytes)
    host["floor_ms"] = round(1e3 * host_bytes / (max(host["pack_GBps"] or 0, host["adam_GBps"]) * 1e9), 1)
    host["floor_frac_of_step"] = round(host["floor_ms"] / ms_step, 3)
    out["host"] = host
    # the three floors of a streamed step: the host link (the step's H2D and
    # D2H bytes at the probed rates), host DRAM (above) and the GPU's own
    # busy time (compute stream over the timed steps); the step's time
    # against the largest of them
    floors = {"link_ms": round(1e3 * max(h2d / (link["h2d_GBps"] * 1e9), d2h / (link["d2h_GBps"] * 1e9)), 1),
              "host_dram_ms": host["floor_ms"],
              "gpu_busy_ms": overlap["gpu_busy_ms_per_step"] if overlap else None}
    bind = max((k for k in floors if floors[k] is not None), key=lambda k: floors[k])
    floors.update(binding=bind, binding_frac_of_step=round(floors[bind] / ms_step, 3),
                  tflops_exec_at_binding=round(f_exec / (floors[bind] * 1e-3) / 1e12, 1))
    out["floors"] = floors
    tr.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
