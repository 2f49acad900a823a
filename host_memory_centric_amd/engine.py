"""Layer-streamed training engine (the schedule around the C ABI).

One training step, in the method's order (MegaTrain paper page, section 3 and
appendix A.2; hyper.ai summary, method; the author blog's block figure):

* forward: for each layer, the packer thread copies its W region from the
  pageable host store into a pinned staging buffer, the weight stream copies
  it into a device slot and records *weights-ready*; the compute stream waits
  for that event, binds the slot to the stateless template and runs the layer;
  an event after the layer marks the slot *buffer-free* for the next copy.
  Block-start activations (one every ``ckpt_every`` layers) stay on the device
  (or, with ``offload_ckpt``, the first blocks' go to host memory and come
  back for their backward); the last block also keeps its layer internals.
* head: final RMSNorm, LM head and cross entropy with their backward.
* backward, block by block from the top: re-stream and recompute the block's
  layers from its checkpoint (keeping their internals), then run their
  backward top-down.  After each layer's backward (*backward-done*) the
  gradient stream copies its gradient slot into a pinned gradient slab; a host
  optimizer thread lands the slab into the store and runs Adam on the layer
  once that copy is done, then recycles the slab (updates in arrival order
  by default, or most urgent first, see ``UpdateScheduler``).
* the embedding gradient is scattered on the host and the embedding's Adam
  runs last.

``step()`` returns once the GPU work of the step is done and the loss is
known; the host Adam updates still running continue in the background.  Each
unit's pending update is tracked, and the next step's packer waits for a
unit's update before copying its weights (the embedding gather likewise waits
for the embedding's update), so the next step's front end overlaps the tail
of the previous step's optimizer work.  ``finish()`` waits for everything.

Which device slot receives which weight load is planned for the whole step
before it starts: since the sequence of layer uses is known, each load evicts
the slot whose unit is needed furthest in the future.  With two slots this is
the pages' double buffering; with more slots a recomputed block can stay
resident for its backward.  ``resident`` mode is the same schedule with a
single block covering all layers and one slot per unit (no recompute, no
re-streaming), which must give bit-identical results.

PyTorch provides device memory, streams and events only; every step of the
computation runs in libmt.so.
"""
import ctypes
import dataclasses
import queue
import threading
import time
from concurrent.futures import Future, ThreadPoolExecutor

import numpy as np
import torch

from . import _lib
from ._lib import MT_UNIT_EMBED, MT_UNIT_HEAD, MtAct, MtHeadIO, MtLayerView, call
from .store import HostStore


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


class UpdateScheduler:
    """One host thread running optimizer updates, lowest priority value first.

    Each job carries an event (its gradient copy) and a priority; among the
    jobs whose copy has completed, the thread runs the one with the lowest
    (priority, submission order) when picking by priority, else the first
    submitted.  With the order in which the next step's forward needs the
    units (embedding, then layers bottom-up, then the head) this is most
    urgent first: the backward produces gradients top-down while the next
    forward consumes weights bottom-up, so the updates of some upper layers
    wait and overlap the next step's forward instead of delaying its first
    layers.

    The events of the jobs are recorded on one in-order stream (the gradient
    stream) in submission order, so they complete in that order: the thread
    queries only the first job whose event it has not yet seen complete, and
    when no job is ready it blocks on that event instead of polling."""

    def __init__(self, by_priority=False):
        self._cv = threading.Condition()
        self._jobs = []      # [priority, seq, event, future, fn, args, ready], in submission order
        self._seq = 0
        self._stop = False
        self._by_priority = bool(by_priority)
        self._key = None  # priority -> sort key (None: the priority itself)
        self._thread = threading.Thread(target=self._run, name="mt-adam", daemon=True)
        self._thread.start()

    def submit(self, priority, event, fn, *args):
        fut = Future()
        with self._cv:
            self._jobs.append([priority, self._seq, event, fut, fn, args, event is None])
            self._seq += 1
            self._cv.notify()
        return fut

    def _run(self):
        while True:
            with self._cv:
                while not self._jobs and not self._stop:
                    self._cv.wait()
                if not self._jobs:
                    return
                # readiness in submission order: every job before the first
                # not-ready one is ready
                first = next((j for j in self._jobs if not j[6]), None)
            if first is not None and first[2].query():
                first[6] = True
                continue
            with self._cv:
                ready = [j for j in self._jobs if j[6]]
                if ready:
                    key = self._key
                    job = min(ready, key=lambda j: ((key(j[0]) if key else j[0]) if self._by_priority else 0, j[1]))
                    self._jobs.remove(job)
                else:
                    job = None
            if job is None:
                first[2].synchronize()  # nothing to run before this copy completes
                first[6] = True
                continue
            _, _, _, fut, fn, args, _ = job
            if not fut.set_running_or_notify_cancel():
                continue
            try:
                fut.set_result(fn(*args))
            except BaseException as e:  # propagated to whoever waits on the future
                fut.set_exception(e)

    def set_by_priority(self, on):
        """Pick ready jobs by (priority, submission order) from now on, or by
        submission order alone."""
        with self._cv:
            self._by_priority = bool(on)
            self._cv.notify()

    def set_key(self, fn):
        """Order ready jobs by fn(priority) (None: by the priority) from now on."""
        with self._cv:
            self._key = fn
            self._cv.notify()

    def shutdown(self):
        with self._cv:
            self._stop = True
            self._cv.notify()
        self._thread.join()


class PinnedBuffer:
    """Library-owned pinned host memory with a numpy view."""

    def __init__(self, nbytes):
        p = ctypes.c_void_p()
        call("mt_pinned_alloc", nbytes, ctypes.byref(p))
        self.ptr = p
        self.nbytes = nbytes

    def view(self, dtype, count=None):
        n = self.nbytes // np.dtype(dtype).itemsize if count is None else count
        buf = (ctypes.c_char * (n * np.dtype(dtype).itemsize)).from_address(self.ptr.value)
        return np.frombuffer(buf, dtype=dtype, count=n)

    def free(self):
        if self.ptr is not None and self.ptr.value:
            call("mt_pinned_free", self.ptr)
        self.ptr = None


def plan_step(L, K, resident):
    """Ops of one step: (kind, layer, saved_index).  kind in fwd/head/refwd/bwd."""
    if resident:
        K = L
    nblk = (L + K - 1) // K
    last0 = (nblk - 1) * K
    ops = []
    for l in range(L):
        ops.append(("fwd", l, (l - last0) if l >= last0 else None))
    ops.append(("head", None, None))
    for b in reversed(range(nblk)):
        lo, hi = b * K, min(L, (b + 1) * K)
        if b != nblk - 1:
            for l in range(lo, hi):
                ops.append(("refwd", l, l - lo))
        for l in reversed(range(lo, hi)):
            ops.append(("bwd", l, l - lo))
    return ops


def plan_slots(units, n_slots, fixed=None, preloaded=()):
    """Assign a device slot to every use; returns (slot per use, load flag per use).

    A use of a unit already resident is a hit.  Otherwise the load may not go
    into the slot of the op just before it (that copy would have to wait for
    that op, so nothing would overlap); among the other slots an empty one is
    taken, else the one whose unit is next needed furthest in the future
    (ties: the least recently used).

    fixed: {unit: slot} for units that own a slot of their own (numbered from
    n_slots on, outside the shared pool): every use of such a unit is in its
    slot, and only its first use loads, unless the unit is in ``preloaded``
    (its slot already holds its weights when the step starts)."""
    fixed = fixed or {}
    content = [None] * n_slots
    last_used = [-1] * n_slots
    slot_of, load = [], []
    seen_fixed = set(preloaded)
    for i, u in enumerate(units):
        if u in fixed:
            slot_of.append(fixed[u])
            load.append(u not in seen_fixed)
            seen_fixed.add(u)
            continue
        if u in content:
            s = content.index(u)
            slot_of.append(s)
            load.append(False)
            last_used[s] = i
            continue
        cands = [k for k in range(n_slots) if n_slots == 1 or i == 0 or k != slot_of[i - 1]]
        empty = [k for k in cands if content[k] is None]
        if empty:
            s = empty[0]
        else:
            def next_use(x):
                for j in range(i + 1, len(units)):
                    if units[j] == x:
                        return j
                return len(units) + 1
            s = max(cands, key=lambda k: (next_use(content[k]), -last_used[k]))
        content[s] = u
        last_used[s] = i
        slot_of.append(s)
        load.append(True)
    return slot_of, load


def carried_layers(L, carry):
    """The layers that keep slots of their own: all but L - carry evenly
    spaced ones, which stream.  Streamed layer i (of n = L - carry) is layer
    (i + 1) * L // n - 1, so each streamed layer follows a run of carried
    ones whose compute covers its load (at L = 48, carry = 36: layers 3, 7,
    ..., 47 stream)."""
    n = L - carry
    streamed = {(i + 1) * L // n - 1 for i in range(n)} if n > 0 else set()
    return [l for l in range(L) if l not in streamed]


class Trainer:
    """Host-memory-centric trainer on one GPU.

    cfg: model shape + batch/seq (``synth.ModelCfg``-like); adam: optimizer
    settings; mode: 'streamed' or 'resident'; n_slots: device weight slots
    (2 = the pages' double buffering; 1 = none, each load waits for the op
    before it; more = a recomputed block stays resident for its backward);
    n_grad_slabs: pinned gradient slabs;
    weights: None (seeded fill by the library) or bf16 bit arrays;
    capture_w32: keep each unit's updated fp32 weights before their bf16
    rounding (``self.w32[unit]``, W-region indexing) for parity checks;
    micro_batches: micro-batches of [batch, seq] tokens per step, whose
    gradients the host accumulates (``mt_grad_accumulate``) before one Adam
    step on their mean; master: keep fp32 master weights in the host store;
    update_order: 'arrival' (host updates in the order their gradients
    arrive), 'urgent' (most urgent first, see ``UpdateScheduler``) or 'tail'
    (arrival order while the backward runs, most urgent first once it has
    issued its last gradient).  With 'urgent' or 'tail', updates deferred
    past the end of a step run during the next step's forward; on some
    machines every gradient copy of that step's backward then ran 4x slower
    (30.8 instead of 7.5 ms per layer at the 7B shape, one step in two),
    which arrival order avoids;
    pinned_store: page-lock the store's W and G regions and copy weights to
    the device straight from W and gradients straight into G (no packer
    copy, no gradient slabs; the packer thread only waits for each unit's
    pending update), which removes 4 bytes per parameter of host memory
    traffic per weight load and 2 per update;
    offload_ckpt: hold the checkpoints (block inputs) of the first
    ``offload_ckpt`` blocks in host memory.  Block checkpoints then live in a
    ring of two device buffers (block b in buffer b % 2) up to block
    offload_ckpt + 1, and in buffers of their own above it: in the forward the
    copy of block b to the host (through a pinned slab, then a host copy on
    the checkpoint thread) runs while block b + 1 computes, and the writer of
    block b + 2 waits for it; in the backward block b comes back (host copy
    into the slab, then to its ring buffer) once block b + 2's backward is
    done, while block b + 1's runs.  The last two ring blocks never leave the
    device.  Long contexts at full depth need it: a 7B-shaped block input is
    4.3 GB at 512K tokens.  Results are bit-identical to keeping them all on
    the device;
    grad_slots: device gradient slots the backward writes in turn (a layer's
    backward waits until the copy out of its slot's previous gradient is
    done; more slots let the evacuation lag further behind);
    carry: ``carry`` layers each own a device slot of their own (outside the
    ``n_slots`` pool) that holds their weights from one step to the next
    (page-locked store only); the other layers, evenly spaced (see
    ``carried_layers``), stream through the pool.  Right after the host
    update of a carried layer the optimizer thread enqueues the copy of its
    new weights into its slot, behind the weight stream's pending loads and
    after the layer's backward has read the old ones; the next step's
    forward, recompute and backward of the layer then use the slot without a
    load.  Each carried layer is loaded once per step instead of once per
    forward and once per recompute, and its load moves out of the link-bound
    forward into the backward and the update tail; the streamed layers' loads
    run while the carried layers between them compute.  The device footprint
    grows by ``carry`` layer slots, a fixed count independent of depth.
    Results are bit-identical to ``carry=0``;
    poison (debug): fill every buffer with NaN as soon as the event that
    frees it fires -- a device weight slot after the op that last reads it
    before a reload, a device gradient slot after the copy that evacuates
    it, a pinned weight staging buffer after the copy that read it, a pinned
    gradient slab after the update that consumed it -- so that any read that
    the event ordering does not cover sees NaN;  delay_seed (debug): random
    host-side delays (0-3 ms, seeded) before every packer and optimizer job.
    With correct ordering neither changes a bit of the results."""

    def __init__(self, cfg, adam, mode="streamed", n_slots=2, n_grad_slabs=16, ckpt_every=None, weights=None,
                 device="cuda:0", capture_w32=False, timeline=False, micro_batches=1, master=False,
                 pinned_store=False, update_order="arrival", offload_ckpt=0, poison=False, delay_seed=None,
                 carry=0, grad_slots=2):
        if update_order not in ("arrival", "urgent", "tail", "carried"):
            raise ValueError("update_order must be 'arrival', 'urgent', 'tail' or 'carried'")
        self.carry = int(carry)
        self.n_gslots = int(grad_slots)
        if self.n_gslots < 1:
            raise ValueError("grad_slots must be at least 1")
        if self.carry and (mode == "resident" or not pinned_store or not 0 < self.carry <= cfg.layers):
            raise ValueError(f"carry must be 0, or with a streamed step and a page-locked store between 1 and "
                             f"the layer count ({cfg.layers})")
        self.update_order = update_order
        self.poison = bool(poison)
        self._delay_rng = None if delay_seed is None else np.random.default_rng(delay_seed)
        self._delay_mu = threading.Lock()
        if mode not in ("streamed", "resident"):
            raise ValueError("mode must be 'streamed' or 'resident'")
        _lib.load()
        self.cfg, self.adam_cfg, self.mode = cfg, adam, mode
        self.dev = torch.device(device)
        self.L = cfg.layers
        self.K = self.L if mode == "resident" else (ckpt_every or cfg.ckpt_every)
        self.n_slots = self.L + 1 if mode == "resident" else max(1, n_slots)
        self.n_host = int(offload_ckpt)
        nblk = (self.L + self.K - 1) // self.K
        if self.n_host and (mode == "resident" or not 0 < self.n_host <= nblk - 2):
            raise ValueError(f"offload_ckpt must be 0, or in a streamed step between 1 and the block count "
                             f"less two ({nblk - 2})")
        self.B, self.S = cfg.batch, cfg.seq
        self.T = self.B * self.S
        h = cfg.hidden
        self.mcfg = _lib.model_cfg(cfg)
        self.madam = _lib.adam_cfg(adam)
        self.t = 0
        self.n_micro = max(1, int(micro_batches))

        self.direct = bool(pinned_store)
        self.store = HostStore(cfg, master=master, accum=self.n_micro > 1, pinned=self.direct)
        if weights is None:
            self.store.fill_normal()
        else:
            self.store.load_bits(weights)
        self.lay = self.store.layout_of(0)
        self.lay_head = self.store.layout_of(MT_UNIT_HEAD)
        # the head's device slot, gradient buffer and slab use the untied head
        # layout (final gain, LM head); with tied weights the LM head part is
        # the embedding matrix, packed from the embedding unit
        self.tied = bool(getattr(cfg, "tied", False))
        self.lay_head_dev = _lib.unit_layout(_lib.model_cfg(dataclasses.replace(cfg, tied=False))
                                             if self.tied else self.mcfg, MT_UNIT_HEAD)
        self.slot_bytes = max(self.lay.w_bytes, self.lay_head_dev.w_bytes)

        self.ops = plan_step(self.L, self.K, mode == "resident")
        units = [MT_UNIT_HEAD if k == "head" else l for (k, l, _) in self.ops]
        self.op_unit = units
        # the carried layers' own slots follow the pool's; the plan of a pass
        # whose carried slots already hold the current weights (every pass
        # but the first) has no load for them
        self.carry_slot = {l: self.n_slots + i for i, l in enumerate(carried_layers(self.L, self.carry))}
        self._plans = {warm: plan_slots(units, self.n_slots, self.carry_slot,
                                        set(self.carry_slot) if warm else ())
                       for warm in (False, True)}
        self.op_slot, self.op_load = self._plans[True]
        self._carried = False  # the carried slots hold the store's current weights
        self._carry_ev = {}    # carried layer -> event: its last copy into its slot is done

        d, T = self.dev, self.T
        bf, f32 = torch.bfloat16, torch.float32
        self.slots = [torch.empty(self.slot_bytes, dtype=torch.uint8, device=d)
                      for _ in range(self.n_slots + self.carry)]
        self.gslots = [torch.empty(self.lay.w_bytes, dtype=torch.uint8, device=d) for _ in range(self.n_gslots)]
        self.head_g = torch.empty(self.lay_head_dev.w_bytes, dtype=torch.uint8, device=d)
        n_ring = self.n_host + 2 if self.n_host else 0  # blocks below n_ring use the two ring buffers
        self.n_ring = n_ring
        self.ckpt_ring = [torch.empty((T, h), dtype=bf, device=d) for _ in range(2 if n_ring else 0)]
        self.ckpt = [None if b < n_ring else torch.empty((T, h), dtype=bf, device=d) for b in range(nblk)]
        self.ckpt_bytes = T * h * 2
        self.ckpt_host = [np.empty(self.ckpt_bytes, dtype=np.uint8) for _ in range(self.n_host)]
        self.ckpt_slab = [PinnedBuffer(self.ckpt_bytes) for _ in range(2 if n_ring else 0)]
        self.ckpt_io = ThreadPoolExecutor(1, thread_name_prefix="mt-ckpt") if n_ring else None
        self.blockx = [None] + [torch.empty((T, h), dtype=bf, device=d) for _ in range(1, self.K)]
        self.xscratch = torch.empty((T, h), dtype=bf, device=d)
        self.xL = torch.empty((T, h), dtype=bf, device=d)
        self.dgrad = [torch.empty((T, h), dtype=f32, device=d) for _ in range(2)]
        self.dgrad_b = [torch.empty((T, h), dtype=bf, device=d) for _ in range(2)]
        self.saved_bytes = _lib.size_query("mt_layer_saved_bytes", self.mcfg, self.B, self.S)
        self.saved = [torch.empty(self.saved_bytes, dtype=torch.uint8, device=d) for _ in range(min(self.K, self.L))]
        ws = max(_lib.size_query("mt_layer_workspace_bytes", self.mcfg, self.B, self.S),
                 _lib.size_query("mt_head_workspace_bytes", self.mcfg, self.B, self.S))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=d)
        self.ws_bytes = ws
        cs = np.empty((self.S, cfg.head_dim // 2), dtype=np.float32)
        sn = np.empty_like(cs)
        call("mt_rope_tables", ctypes.byref(self.mcfg), self.S, cs.ctypes.data_as(ctypes.c_void_p),
             sn.ctypes.data_as(ctypes.c_void_p))
        self.rope_cos = torch.from_numpy(cs).to(d)
        self.rope_sin = torch.from_numpy(sn).to(d)
        self.tok_dev = torch.empty((self.B, self.S), dtype=torch.int32, device=d)
        self.loss_dev = torch.zeros(1, dtype=f32, device=d)

        # staging: packed weights and landed gradients pass through pinned
        # slabs, unless the store's own W and G regions are pinned (the tied
        # head's gradient still goes through its slab: it updates two units)
        n_wslab, n_gslab = (0, 0) if self.direct else (2, max(1, n_grad_slabs))
        self.wslab = [PinnedBuffer(self.slot_bytes) for _ in range(n_wslab)]
        self.gslab = [PinnedBuffer(self.lay.w_bytes) for _ in range(n_gslab)]
        self.head_gslab = PinnedBuffer(self.lay_head_dev.w_bytes) if (self.tied or not self.direct) else None
        if self.direct and self.tied:  # the head slot is filled from two W regions
            off = self.lay_head_dev.tensor_off[1]
            if (self.store.layout_of(MT_UNIT_HEAD).w_bytes != off or
                    self.store.layout_of(MT_UNIT_EMBED).w_bytes != self.lay_head_dev.w_bytes - off):
                raise RuntimeError("tied head slot does not match the gain and embedding W regions")
        self.w_addr = {u: ctypes.c_void_p(self.store.region_addr(u, 0)) for u in self.store.units}
        self.g_addr = {u: ctypes.c_void_p(self.store.region_addr(u, 1)) for u in self.store.units}
        self.x0_pin = PinnedBuffer(T * h * 2)
        self.dx0_pin = PinnedBuffer(T * h * 4)
        self.tok_pin = PinnedBuffer(T * 4)

        self.s_comp = torch.cuda.Stream(device=d)
        self.s_h2d = torch.cuda.Stream(device=d)
        self.s_d2h = torch.cuda.Stream(device=d)
        self.packer = ThreadPoolExecutor(1, thread_name_prefix="mt-pack")
        # copy issuers: a weight load is enqueued once its slot's last reader
        # has completed, a gradient copy once its backward has completed, so
        # that no copy command waits for compute work inside a DMA queue
        self.h2d_issuer = ThreadPoolExecutor(1, thread_name_prefix="mt-h2d")
        self.d2h_issuer = ThreadPoolExecutor(1, thread_name_prefix="mt-d2h")
        self.optimizer = UpdateScheduler(by_priority=update_order in ("urgent", "carried"))
        self.slab_free = queue.Queue()
        for k in range(len(self.gslab)):
            self.slab_free.put(k)
        self.pending = {}              # unit -> future of its host update still running
        self.accum_jobs = {}           # unit -> future of its last micro-batch accumulation
        self.gslot_d2h = [None] * self.n_gslots  # last copy out of each device gradient slot
        self.head_d2h = None           # last copy out of the head's gradient buffer
        self.record_timeline = timeline
        self.progress = None  # optional callable(kind, layer), called as each op is enqueued
        self._tl = None
        self.stats = {}
        self.w32 = {}
        if capture_w32:
            for u in self.store.units:
                self.w32[u] = np.zeros(self.store.layout_of(u).w_bytes // 2, dtype=np.float32)

    def _debug_delay(self):
        if self._delay_rng is not None:
            with self._delay_mu:
                d = float(self._delay_rng.uniform(0.0, 3e-3))
            time.sleep(d)

    def _tensor_ranges(self, lay):
        """(byte offset, bytes) of each tensor of a unit layout (its padding excluded)."""
        return [(int(lay.tensor_off[j]), 2 * int(lay.tensor_numel[j])) for j in range(lay.n_tensors)]

    def _poison_dev(self, buf, lay):
        """NaN (all-ones bytes) over the tensors of a device buffer in ``lay``'s
        layout, on the current stream."""
        for off, n in self._tensor_ranges(lay):
            buf[off:off + n].fill_(0xFF)

    def _poison_host(self, pinned, lay):
        v = pinned.view(np.uint8, lay.w_bytes)
        for off, n in self._tensor_ranges(lay):
            v[off:off + n] = 0xFF

    def _w32_ptr(self, unit):
        a = self.w32.get(unit)
        return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None

    # ------------------------------------------------------------------
    def finish(self):
        """Wait for every host update (and accumulation) of the previous steps."""
        for u in list(self.accum_jobs):
            self._wait_acc(u)
        for u in list(self.pending):
            self._wait_unit(u)

    def save(self, path):
        """Checkpoint the training state (host store and step counter) after
        every pending update; a trainer that loads it continues bit-identically
        (the device holds no state across steps)."""
        self.finish()
        self.store.save(path, self.t)

    def load(self, path):
        """Resume from a checkpoint written by save() for the same model,
        store options and batch shape."""
        self.finish()
        self.t = self.store.load(path)
        self._carried = False  # the carried slots hold the weights before the load

    def store_modified(self):
        """Declare that the host store was written directly (weights or
        moments set from elsewhere) after every pending update: the weights
        the carried layers' slots hold are dropped and loaded again at their
        next use."""
        self.finish()
        self.s_h2d.synchronize()  # no copy out of the store is still reading it
        self._carried = False

    def _wait_unit(self, unit):
        f = self.pending.pop(unit, None)
        if f is not None:
            f.result()

    def _wait_acc(self, unit):
        f = self.accum_jobs.pop(unit, None)
        if f is not None:
            f.result()

    def close(self):
        try:
            self.finish()
        finally:
            torch.cuda.synchronize(self.dev)
            self.packer.shutdown(wait=True)
            self.h2d_issuer.shutdown(wait=True)
            self.d2h_issuer.shutdown(wait=True)
            self.optimizer.shutdown()
            if self.ckpt_io is not None:
                self.ckpt_io.shutdown(wait=True)
        for b in self.wslab + self.gslab + self.ckpt_slab + [self.head_gslab, self.x0_pin, self.dx0_pin,
                                                             self.tok_pin]:
            if b is not None:
                b.free()
        self.store.close()

    def n_weight_loads(self):
        """Weight loads of one pass in the steady state (the carried layers'
        copies after their updates are counted by n_carry_loads)."""
        return sum(self.op_load)

    def n_carry_loads(self):
        """Copies of carried layers into their own slots per optimizer step."""
        return self.carry

    def _x(self, l):
        if l == self.L:
            return self.xL
        if l % self.K == 0:
            b = l // self.K
            return self.ckpt_ring[b % 2] if b < self.n_ring else self.ckpt[b]
        return self.blockx[l % self.K]

    def _bind(self, slot, gslot, unit):
        v = MtLayerView()
        call("mt_bind", ctypes.byref(self.mcfg), unit, _ptr(self.slots[slot]),
             _ptr(gslot) if gslot is not None else None, ctypes.byref(v))
        return v

    def _act(self, x_in, x_out=None, saved=None, dy=None, dyb=None, dx=None, dxb=None):
        a = MtAct()
        a.batch, a.seq = self.B, self.S
        a.x_in = x_in.data_ptr()
        a.x_out = x_out.data_ptr() if x_out is not None else None
        a.dy = dy.data_ptr() if dy is not None else None
        a.dy_bf16 = dyb.data_ptr() if dyb is not None else None
        a.dx = dx.data_ptr() if dx is not None else None
        a.dx_bf16 = dxb.data_ptr() if dxb is not None else None
        a.rope_cos = self.rope_cos.data_ptr()
        a.rope_sin = self.rope_sin.data_ptr()
        a.saved = saved.data_ptr() if saved is not None else None
        a.saved_bytes = self.saved_bytes if saved is not None else 0
        a.workspace = self.ws.data_ptr()
        a.workspace_bytes = self.ws_bytes
        return a

    # ------------------------------------------------------------------
    def step(self, tokens):
        """One training step on int32 tokens [micro_batches * B, S]: each
        micro-batch of B rows runs forward, head and backward; the host
        accumulates their gradients and runs Adam once, on their mean, after
        the last.  Returns the loss (mean over the micro-batches)."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        if tokens.shape != (self.n_micro * self.B, self.S):
            raise ValueError(f"tokens must have shape {(self.n_micro * self.B, self.S)}")
        self.t += 1
        t0 = time.perf_counter()
        tl = self._timeline_begin(self.s_comp) if self.record_timeline else None
        losses = []
        n_loads = 0
        for i in range(self.n_micro):
            loss, n = self._pass(tokens[i * self.B:(i + 1) * self.B], self.t, i == self.n_micro - 1, tl)
            losses.append(loss)
            n_loads += n
        self.stats = {"step_s": time.perf_counter() - t0, "weight_loads": n_loads, "losses": losses}
        if tl is not None:
            self._tl = tl
        # reporting only: every micro-batch's loss and gradients come from the
        # head kernel (mt_head_fwd_bwd); their mean is the value returned to the
        # caller and takes no part in the update
        return float(np.mean(np.asarray(losses, dtype=np.float64)))

    def _pass(self, tokens, t, final, tl):
        """Forward, head and backward of one micro-batch; its gradients go to
        Adam (``final``) or to the host accumulator.  Returns (loss, loads)."""
        h = self.cfg.hidden
        cs, hs, ds = self.s_comp, self.s_h2d, self.s_d2h
        sc, sh, sd = (ctypes.c_void_p(s.cuda_stream) for s in (cs, hs, ds))

        # embedding gather + tokens (host) -> device, after the embedding's
        # update of the previous step (which also still reads the token
        # buffer), or its accumulation of the previous micro-batch
        self._wait_unit(MT_UNIT_EMBED)
        self._wait_acc(MT_UNIT_EMBED)
        tok_host = self.tok_pin.view(np.int32)
        tok_host[:] = tokens.reshape(-1)
        call("mt_embed_gather", self.store.ptr, self.tok_pin.ptr, self.T, self.x0_pin.ptr)
        inputs_ready = torch.cuda.Event()
        with torch.cuda.stream(hs):
            call("mt_copy_h2d", _ptr(self._x(0)), self.x0_pin.ptr, self.T * h * 2, sh)
            call("mt_copy_h2d", _ptr(self.tok_dev), self.tok_pin.ptr, self.T * 4, sh)
            inputs_ready.record(hs)
        cs.wait_event(inputs_ready)

        # block checkpoints held in host memory (offload_ckpt)
        K, nh, ck_bytes = self.K, self.n_host, self.ckpt_bytes
        ck_d2h = {}            # block -> event: its copy out of its ring buffer is done
        ck_h2d = {}            # block -> event: its copy back into its ring buffer is done
        ck_out = [None, None]  # slab -> future of the host copy that last read it
        ck_in = {}             # block -> future: its data is in its slab
        ck_next = [nh - 1]     # next block to copy back to the device (top down)
        op_index = {(k, l): i for i, (k, l, _) in enumerate(self.ops)}

        def ckpt_out(b, ev):
            # ring buffer b % 2 -> slab b % 2 on the D2H stream after the writer (ev), then
            # slab -> host memory on the checkpoint thread
            r = b % 2
            if ck_out[r] is not None:
                ck_out[r].result()  # the slab's previous copy to host memory is done
            d2h = torch.cuda.Event(enable_timing=self.record_timeline)
            with torch.cuda.stream(ds):
                ds.wait_event(ev)
                if tl is not None:
                    tl["d2h"].append([self._ev(ds), d2h])
                call("mt_copy_d2h", self.ckpt_slab[r].ptr, _ptr(self.ckpt_ring[r]), ck_bytes, sd)
                d2h.record(ds)
            ck_d2h[b] = d2h
            dst = self.ckpt_host[b].ctypes.data_as(ctypes.c_void_p)

            def job():
                d2h.synchronize()
                call("mt_host_copy", dst, self.ckpt_slab[r].ptr, ck_bytes)
            ck_out[r] = self.ckpt_io.submit(job)

        def ckpt_fetch(b):
            # host memory -> slab b % 2 on the checkpoint thread, after the slab's copy to
            # the device for block b + 2.  The two top blocks are still in their slabs
            # (each was the last block of its parity that the forward copied out).
            r = b % 2
            if b >= nh - 2:
                f = Future()
                f.set_result(None)
                ck_in[b] = f
                return
            prev = ck_h2d[b + 2]
            src = self.ckpt_host[b].ctypes.data_as(ctypes.c_void_p)

            def job():
                prev.synchronize()
                call("mt_host_copy", self.ckpt_slab[r].ptr, src, ck_bytes)
            ck_in[b] = self.ckpt_io.submit(job)

        def ckpt_in(upto, need=None):
            # issue, top down, the copies back into the ring buffers whose block is in its
            # slab and whose buffer's last reader (block b + 2's backward of its first
            # layer, op <= upto) is enqueued; need: a block whose copy must be issued now
            while ck_next[0] >= 0:
                b = ck_next[0]
                last = op_index[("bwd", (b + 2) * K)]
                if last > upto or b not in ck_in or (b != need and not ck_in[b].done()):
                    return
                ck_in.pop(b).result()
                r = b % 2
                ev = torch.cuda.Event(enable_timing=self.record_timeline)
                with torch.cuda.stream(hs):
                    hs.wait_event(op_done[last])  # the ring buffer is free
                    if tl is not None:
                        tl["h2d"].append([self._ev(hs), ev])
                        tl["h2d_tag"][ev] = ("ckpt", b)
                    call("mt_copy_h2d", _ptr(self.ckpt_ring[r]), self.ckpt_slab[r].ptr, ck_bytes, sh)
                    ev.record(hs)
                ck_h2d[b] = ev
                ck_next[0] -= 1
                if b >= 2:
                    ckpt_fetch(b - 2)

        if nh:
            ckpt_out(0, inputs_ready)

        # weight loads of this step, in order (no loads for the carried layers
        # once their slots hold the current weights)
        warm = self._carried
        op_slot, op_load = self._plans[warm]
        loads = [i for i, ld in enumerate(op_load) if ld]
        load_of_op = {i: j for j, i in enumerate(loads)}
        ready_ev = [torch.cuda.Event(enable_timing=self.record_timeline) for _ in loads]
        op_done = [None] * len(self.ops)
        # previous op that used the same slot (the copy into the slot waits for it)
        slot_prev = [None] * len(self.ops)
        last = {}
        for i, s in enumerate(op_slot):
            slot_prev[i] = last.get(s)
            last[s] = i

        pending = dict(self.pending)  # updates of the previous step still running
        # ops after which their slot is reloaded (the load waits for the op's event)
        poison_slot_after = {slot_prev[i] for i in loads if slot_prev[i] is not None} if self.poison else set()

        def pack(j):
            self._debug_delay()
            unit = self.op_unit[loads[j]]
            if self.direct:  # the copy reads the store itself: only wait for the update
                f = pending.get(unit)
                if f is not None:
                    f.result()
                return
            if j >= 2:
                ready_ev[j - 2].synchronize()  # the copy that read this staging buffer is done
                if self.poison:
                    prev = self.op_unit[loads[j - 2]]
                    self._poison_host(self.wslab[j % 2], self.lay_head_dev if prev == MT_UNIT_HEAD else self.lay)
            f = pending.get(unit)
            if f is not None:
                f.result()  # the unit's update of the previous step has landed
            if unit == MT_UNIT_HEAD and self.tied:
                call("mt_pack_head_tied", self.store.ptr, self.wslab[j % 2].ptr, self.slot_bytes)
            else:
                call("mt_pack_layer", self.store.ptr, unit, self.wslab[j % 2].ptr, self.slot_bytes)

        pack_fut = {j: self.packer.submit(pack, j) for j in range(min(2, len(loads)))}
        op_enq = [threading.Event() for _ in self.ops]  # op i enqueued, op_done[i] recorded
        load_issued = [threading.Event() for _ in loads]
        aborted = [False]  # set when this pass fails: the copy issuers stop waiting for ops

        def issue_load(j):
            i = loads[j]
            pack_fut.pop(j).result()
            unit = self.op_unit[i]
            nbytes = (self.lay_head_dev if unit == MT_UNIT_HEAD else self.lay).w_bytes
            pu = slot_prev[i]
            if pu is not None:
                op_enq[pu].wait()
                if aborted[0]:
                    raise RuntimeError("the pass was abandoned")
                op_done[pu].synchronize()  # buffer-free: the slot's last reader has completed
            with torch.cuda.device(self.dev), torch.cuda.stream(hs):
                if tl is not None:
                    tl["h2d"].append([self._ev(hs), ready_ev[j]])
                    tl["h2d_tag"][ready_ev[j]] = ("load", unit)
                dst = _ptr(self.slots[op_slot[i]])
                if not self.direct:
                    call("mt_copy_h2d", dst, self.wslab[j % 2].ptr, nbytes, sh)
                elif unit == MT_UNIT_HEAD and self.tied:  # [final gain | embedding matrix as the LM head]
                    lh = self.store.layout_of(MT_UNIT_HEAD)
                    off = self.lay_head_dev.tensor_off[1]
                    call("mt_copy_h2d", dst, self.w_addr[MT_UNIT_HEAD], lh.w_bytes, sh)
                    call("mt_copy_h2d", ctypes.c_void_p(dst.value + off), self.w_addr[MT_UNIT_EMBED],
                         nbytes - off, sh)
                else:
                    call("mt_copy_h2d", dst, self.w_addr[unit], nbytes, sh)
                ready_ev[j].record(hs)  # weights-ready
            if j + 2 < len(loads):
                pack_fut[j + 2] = self.packer.submit(pack, j + 2)

        def issue_loads():
            # every load of the pass in order, each as soon as its packing (or
            # the unit's update) is done and its slot is free
            for j in range(len(loads)):
                issue_load(j)
                load_issued[j].set()

        h2d_fut = self.h2d_issuer.submit(issue_loads) if loads else None

        def wait_load(j):
            while not load_issued[j].wait(0.05):
                if h2d_fut.done():
                    h2d_fut.result()  # the issuer failed: raise its error here
                    raise RuntimeError("weight load issuer ended early")

        d2h_futs = []

        def wait_copy_out(entry):
            # (future of the issuer job, event recorded after the copy)
            if entry is None:
                return None
            entry[0].result()
            return entry[1]

        slab_free = self.slab_free
        gslot_d2h = self.gslot_d2h
        cur = 0
        n_bwd = 0

        def adam_layer(ev, unit, src, after=None):
            # src: the pinned slab holding the gradient, or None: already in G;
            # after: a carried layer's backward (its slot's last reader)
            self._debug_delay()
            ev.synchronize()
            t_a = time.perf_counter()
            if final:
                call("mt_step", self.store.ptr, unit, src, ctypes.byref(self.madam), t, self._w32_ptr(unit))
                if after is not None:
                    self._carry_copy(unit, after, tl)
            else:
                call("mt_grad_accumulate", self.store.ptr, unit, src)
            if tl is not None:
                tl["host"].append(("update", unit, t_a, time.perf_counter()))

        def adam_layer_slab(ev, unit, k):
            try:
                adam_layer(ev, unit, self.gslab[k].ptr)
            finally:
                if self.poison:
                    self._poison_host(self.gslab[k], self.lay)
                slab_free.put(k)

        def adam_embed(ev):
            self._debug_delay()
            ev.synchronize()
            t_a = time.perf_counter()
            if self.tied:  # the shared matrix: the head's gradient (in the head slab) plus the embedding's
                head_grad = ctypes.c_void_p(self.head_gslab.ptr.value + self.lay_head_dev.tensor_off[1])
                call("mt_embed_grad_tied", self.store.ptr, self.tok_pin.ptr, self.T, self.dx0_pin.ptr, head_grad)
            else:
                call("mt_embed_grad", self.store.ptr, self.tok_pin.ptr, self.T, self.dx0_pin.ptr)
            if final:
                call("mt_step", self.store.ptr, MT_UNIT_EMBED, None, ctypes.byref(self.madam), t,
                     self._w32_ptr(MT_UNIT_EMBED))
            else:
                call("mt_grad_accumulate", self.store.ptr, MT_UNIT_EMBED, None)
            if tl is not None:
                tl["host"].append(("update", MT_UNIT_EMBED, t_a, time.perf_counter()))

        jobs = self.pending if final else self.accum_jobs

        try:
            for i, (kind, l, si) in enumerate(self.ops):
                if op_load[i]:
                    wait_load(load_of_op[i])
                    cs.wait_event(ready_ev[load_of_op[i]])
                    if l in self.carry_slot and kind != "head":
                        self._carry_ev[l] = ready_ev[load_of_op[i]]
                elif warm and kind == "fwd" and l in self.carry_slot:
                    # the previous step's update of a carried layer enqueued the
                    # copy of its new weights into the layer's slot before it ended
                    self._wait_unit(l)
                    ev_c = self._carry_ev.get(l)
                    if ev_c is not None:
                        cs.wait_event(ev_c)
                slot = op_slot[i]
                if self.progress is not None:
                    self.progress(kind, l)
                # block checkpoints in host memory: the writer of a ring buffer waits for the copy
                # out of its previous block; the first reader in the backward for the copy back
                wb = (l + 1) // K if kind == "fwd" and (l + 1) % K == 0 else None
                if kind == "head" and nh:
                    ckpt_fetch(nh - 1)
                    if nh >= 2:
                        ckpt_fetch(nh - 2)
                if kind == "refwd" and l % K == 0 and l // K < nh:
                    ckpt_in(i - 1, need=l // K)
                    cs.wait_event(ck_h2d[l // K])
                with torch.cuda.stream(cs):
                    if wb is not None and 2 <= wb < self.n_ring:
                        cs.wait_event(ck_d2h[wb - 2])
                    if kind == "head" and self.head_d2h is not None:
                        cs.wait_event(wait_copy_out(self.head_d2h))  # previous step's copy out of the head gradient
                    if kind == "bwd" and gslot_d2h[n_bwd % self.n_gslots] is not None:
                        # buffer-free (gradient slot)
                        cs.wait_event(wait_copy_out(gslot_d2h[n_bwd % self.n_gslots]))
                    if tl is not None:
                        tl["ops"].append([kind, self._ev(cs), None])
                    if kind == "fwd":
                        v = self._bind(slot, None, l)
                        # layers before the last block keep nothing: the first saved
                        # buffer (written again by the last block) is their scratch
                        a = self._act(self._x(l), self._x(l + 1), self.saved[si if si is not None else 0])
                        call("mt_layer_fwd", ctypes.byref(v), ctypes.byref(self.mcfg), ctypes.byref(a), sc)
                    elif kind == "refwd":
                        out = self._x(l + 1) if (l + 1) % self.K != 0 else self.xscratch
                        v = self._bind(slot, None, l)
                        a = self._act(self._x(l), out, self.saved[si])
                        call("mt_layer_fwd", ctypes.byref(v), ctypes.byref(self.mcfg), ctypes.byref(a), sc)
                    elif kind == "head":
                        v = self._bind(slot, self.head_g, MT_UNIT_HEAD)
                        io = MtHeadIO()
                        io.batch, io.seq = self.B, self.S
                        io.x = self.xL.data_ptr()
                        io.tokens = self.tok_dev.data_ptr()
                        io.dx = self.dgrad[cur].data_ptr()
                        io.dx_bf16 = self.dgrad_b[cur].data_ptr()
                        io.loss = self.loss_dev.data_ptr()
                        io.workspace = self.ws.data_ptr()
                        io.workspace_bytes = self.ws_bytes
                        call("mt_head_fwd_bwd", ctypes.byref(v), ctypes.byref(self.mcfg), ctypes.byref(io), sc)
                    else:  # bwd
                        g = n_bwd % self.n_gslots
                        v = self._bind(slot, self.gslots[g], l)
                        a = self._act(self._x(l), None, self.saved[si], dy=self.dgrad[cur], dyb=self.dgrad_b[cur],
                                      dx=self.dgrad[1 - cur], dxb=self.dgrad_b[1 - cur])
                        call("mt_layer_recompute_bwd", ctypes.byref(v), ctypes.byref(self.mcfg), ctypes.byref(a), sc)
                        cur = 1 - cur
                    if i in poison_slot_after or (self.poison and final and kind == "bwd" and l in self.carry_slot):
                        self._poison_dev(self.slots[slot], self.lay_head_dev if kind == "head" else self.lay)
                    ev = torch.cuda.Event(enable_timing=self.record_timeline)
                    ev.record(cs)
                    op_done[i] = ev
                    if tl is not None:
                        tl["ops"][-1][2] = ev
                op_enq[i].set()
                if wb is not None and wb < nh:
                    ckpt_out(wb, ev)
                if kind == "head":
                    d2h = torch.cuda.Event(enable_timing=self.record_timeline)

                    def head_out(ev=ev, d2h=d2h):
                        self._wait_unit(MT_UNIT_HEAD)  # the previous update still reads the head's slab
                        self._wait_acc(MT_UNIT_HEAD)   # (or the previous micro-batch's accumulation)
                        head_dst = self.head_gslab.ptr if self.head_gslab is not None else self.g_addr[MT_UNIT_HEAD]
                        ev.synchronize()  # the head's gradient is complete
                        with torch.cuda.device(self.dev), torch.cuda.stream(ds):
                            if tl is not None:
                                tl["d2h"].append([self._ev(ds), d2h])
                            call("mt_copy_d2h", head_dst, _ptr(self.head_g), self.lay_head_dev.w_bytes, sd)
                            if self.poison:
                                self._poison_dev(self.head_g, self.lay_head_dev)
                            d2h.record(ds)
                        if self.update_order == "tail":
                            self.optimizer.set_by_priority(False)
                        elif self.update_order == "carried":
                            self.optimizer.set_key(self._carried_first)
                        jobs[MT_UNIT_HEAD] = self.optimizer.submit(
                            self._urgency(MT_UNIT_HEAD), d2h, adam_layer, d2h, MT_UNIT_HEAD,
                            self.head_gslab.ptr if self.head_gslab is not None else None)
                    f = self.d2h_issuer.submit(head_out)
                    d2h_futs.append(f)
                    self.head_d2h = (f, d2h)
                elif kind == "bwd":
                    g = n_bwd % self.n_gslots
                    n_bwd += 1
                    d2h = torch.cuda.Event(enable_timing=self.record_timeline)

                    def grad_out(ev=ev, g=g, l=l, d2h=d2h, dx=self.dgrad[cur]):
                        self._wait_unit(l)  # (finished long ago: the previous step's update of this layer)
                        if self.direct:
                            # G is the copy's destination: the previous micro-batch's
                            # accumulation (long finished) must have read it
                            self._wait_acc(l)
                            k, g_dst = None, self.g_addr[l]
                        else:
                            k = slab_free.get()
                            g_dst = self.gslab[k].ptr
                        ev.synchronize()  # backward-done: the layer's gradient is complete
                        if tl is not None:
                            t_s = time.perf_counter()
                            tl["host"].append(("bwd_done", l, t_s, t_s))
                        with torch.cuda.device(self.dev), torch.cuda.stream(ds):
                            if tl is not None:
                                tl["d2h"].append([self._ev(ds), d2h])
                            call("mt_copy_d2h", g_dst, _ptr(self.gslots[g]), self.lay.w_bytes, sd)
                            if self.poison:
                                self._poison_dev(self.gslots[g], self.lay)
                            d2h.record(ds)
                            if l == 0:
                                d2h_x = torch.cuda.Event(enable_timing=self.record_timeline)
                                if tl is not None:
                                    tl["d2h"].append([self._ev(ds), d2h_x])
                                call("mt_copy_d2h", self.dx0_pin.ptr, _ptr(dx), self.T * h * 4, sd)
                                d2h_x.record(ds)
                        if k is None:
                            after = ev if (final and l in self.carry_slot) else None
                            jobs[l] = self.optimizer.submit(self._urgency(l), d2h, adam_layer, d2h, l, None, after)
                        else:
                            jobs[l] = self.optimizer.submit(self._urgency(l), d2h, adam_layer_slab, d2h, l, k)
                        if l == 0:
                            jobs[MT_UNIT_EMBED] = self.optimizer.submit(self._urgency(MT_UNIT_EMBED), d2h_x, adam_embed,
                                                                        d2h_x)
                            if self.update_order == "tail":
                                self.optimizer.set_by_priority(True)
                            elif self.update_order == "carried":
                                self.optimizer.set_key(None)
                    f = self.d2h_issuer.submit(grad_out)
                    d2h_futs.append(f)
                    gslot_d2h[g] = (f, d2h)
                if nh:
                    ckpt_in(i)
        except BaseException:
            aborted[0] = True
            for e in op_enq:
                e.set()
            for f in ([h2d_fut] if h2d_fut is not None else []) + d2h_futs:
                try:
                    f.result()
                except BaseException:
                    pass
            raise

        if h2d_fut is not None:
            h2d_fut.result()
        for f in d2h_futs:
            f.result()
        for f in list(pack_fut.values()):
            f.result()
        for f in ck_out:
            if f is not None:
                f.result()
        cs.synchronize()
        self._carried = bool(self.carry)
        return float(self.loss_dev.item()), len(loads)

    def _carry_copy(self, unit, after, tl):
        """Enqueue the copy of a carried layer's updated weights from the store
        into the layer's own slot, on the weight stream, once ``after`` (the
        layer's backward, the last reader of the old weights) has completed.
        Runs on the optimizer thread right after the layer's update; the next
        pass's first use of the layer waits for this copy's event."""
        hs = self.s_h2d
        after.synchronize()  # (long done: the update waited for the gradient copy that followed it)
        with torch.cuda.device(self.dev):
            ev = torch.cuda.Event(enable_timing=self.record_timeline)
            t0 = self._ev(hs) if tl is not None else None
            call("mt_copy_h2d", _ptr(self.slots[self.carry_slot[unit]]), self.w_addr[unit], self.lay.w_bytes,
                 ctypes.c_void_p(hs.cuda_stream))
            ev.record(hs)
        if tl is not None:
            tl["h2d"].append([t0, ev])
            tl["h2d_tag"][ev] = ("refill", unit)
        self._carry_ev[unit] = ev

    def _carried_first(self, priority):
        """Sort key of the 'carried' order during the backward: the head and
        the carried layers first (their new weights then travel while the
        backward runs), then the streamed layers, whose loads go in the next
        forward anyway; each class by its priority."""
        return (0 if priority == self.L or priority in self.carry_slot else 1, priority)

    def _urgency(self, unit):
        """Scheduling priority of a unit's update: the order in which the next
        step needs its updated weights (used by 'urgent' always, by 'tail'
        and 'carried' once the backward has issued its last gradient, by
        'carried' within its two classes before)."""
        if unit == MT_UNIT_EMBED:
            return -1
        if unit == MT_UNIT_HEAD:
            return self.L
        return unit

    # ------------------------------------------------------------------
    @staticmethod
    def _ev(stream):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def _timeline_begin(self, cs):
        ref = torch.cuda.Event(enable_timing=True)
        ref.record(cs)
        return {"ref": ref, "ops": [], "h2d": [], "d2h": [], "host": [], "h2d_tag": {},
                "t_host": time.perf_counter()}

    def timeline(self):
        """Intervals (ms from the step's start) of the last step recorded with
        timeline=True: {'ops': [(kind, start, end)], 'h2d': [(start, end)],
        'd2h': [(start, end)], 'host': [(kind, unit, start, end)]}; 'host' holds
        the optimizer thread's updates ('update') and the moments the copy
        thread saw each backward end ('bwd_done'), moved onto the event clock.
        Waits for the step's host updates (which enqueue the carried layers'
        copies) and for its copies to finish."""
        tl = self._tl
        if tl is None:
            return None
        self.finish()
        for _, _, e in tl["ops"]:
            e.synchronize()
        for _, e in tl["h2d"] + tl["d2h"]:
            e.synchronize()
        ref = tl["ref"]
        rel = ref.elapsed_time
        ops = [(k, rel(a), rel(b)) for k, a, b in tl["ops"]]
        host = [(k, u, 1e3 * (a - tl["t_host"]), 1e3 * (b - tl["t_host"])) for k, u, a, b in tl["host"]]
        # host clock -> event clock: a backward's end is seen by the thread that
        # waits for it a little later, so the smallest difference estimates the shift
        bwd_end = [e for k, _, e in ops if k == "bwd"]
        seen = [a for k, _, a, _ in host if k == "bwd_done"]
        shift = min((s - e for s, e in zip(seen, bwd_end)), default=0.0) if len(seen) == len(bwd_end) else 0.0
        return {"ops": ops,
                "h2d": [(rel(a), rel(b)) for a, b in tl["h2d"]],
                "d2h": [(rel(a), rel(b)) for a, b in tl["d2h"]],
                "host": [(k, u, a - shift, b - shift) for k, u, a, b in host]}

    # ------------------------------------------------------------------
    def weights(self):
        """bf16 bit arrays of all weights (host store), after every pending update."""
        self.finish()
        return self.store.read_bits()
