"""Denoising schedule of a layer stack and its runner.

Appendix Table 9 of the paper landing page gives, per model, the layers
that always stay dense, the dense warm-up steps and the anchor steps (1-indexed).
The research walkthrough (method steps 4-5) says the other layers reuse the
anchor's metadata with fresh Q/K/V, and that a cache too large for the GPU
goes to host memory and is prefetched one layer ahead.

``plan`` turns those settings into one action per (step, layer):
  "dense"   plain dense attention (warm-up step or always-dense layer);
  "anchor"  anchor step: PDDP grouping, dense attention + LSE, exact top-K,
            residual (the layer's output is the dense output);
  "reuse"   sparse attention over the cached indices + cached R.
An anchor step may coincide with the last warm-up step (its output is dense
anyway). A layer that is not always dense and has no anchor yet runs dense.

``StackRunner`` executes a plan on one GPU through libmcsparse, keeping each
sparse layer's groups and indices on the device and its R in an offload
cache (pinned host memory, two device slots, one-layer-ahead prefetch on a
side stream). With ``offload_idx`` the indices are offloaded too, as
bitmaps (one bit per key), and decoded into one shared device buffer just
before each reuse call (paper landing page, Table 8 offloads both).
"""
from __future__ import annotations

import dataclasses

import torch

from . import binding as mcs

DENSE, ANCHOR, REUSE = "dense", "anchor", "reuse"


@dataclasses.dataclass(frozen=True)
class Schedule:
    steps: int                 # denoising steps, numbered 1..steps
    layers: int                # attention layers, numbered 0..layers-1
    dense_layers: tuple        # layers that always run dense
    warmup_steps: int          # steps 1..warmup_steps run dense
    anchor_steps: tuple        # steps that (re)build the metadata


# Appendix Table 9 (paper landing page): 3D-latent model and the video models
HY3D = Schedule(steps=12, layers=40, dense_layers=(0,), warmup_steps=1, anchor_steps=(1,))
WAN_1_3B_VIDEO = Schedule(steps=50, layers=30, dense_layers=(0,), warmup_steps=10, anchor_steps=(10, 26))


def plan(s: Schedule):
    """List of (step, layer, action)."""
    out = []
    anchored = set()
    for step in range(1, s.steps + 1):
        for layer in range(s.layers):
            if layer in s.dense_layers:
                act = DENSE
            elif step in s.anchor_steps:
                act = ANCHOR
                anchored.add(layer)
            elif step <= s.warmup_steps or layer not in anchored:
                act = DENSE
            else:
                act = REUSE
            out.append((step, layer, act))
    return out


def counts(p):
    c = {DENSE: 0, ANCHOR: 0, REUSE: 0}
    for _, _, a in p:
        c[a] += 1
    return c


class StackRunner:
    """Runs a plan for a stack whose layers share one shape.

    ``inputs(step, layer)`` returns that layer's (q, k, v) device tensors.
    Every sparse layer keeps perm / kv_idx on the device; R lives in the
    offload cache: stored right after the anchor's residual, prefetched on
    ``side`` one layer ahead of its reuse, acquired on the compute stream.
    """

    def __init__(self, sched: Schedule, shape, group_size, topk, power_iters=16, offload=True, offload_idx=False):
        B, N, H, d = shape
        self.s, self.T, self.K = sched, group_size, topk
        self.B, self.N, self.H, self.d = B, N, H, d
        self.G = -(-N // group_size)
        self.sparse_layers = [l for l in range(sched.layers) if l not in sched.dense_layers]
        if offload_idx and not offload:
            raise ValueError("offload_idx needs offload")
        self.offload_idx = offload_idx
        dev = "cuda"
        self.perm = {l: torch.empty((B, H, N), dtype=torch.int32, device=dev) for l in self.sparse_layers}
        idx_shape = (B, H, self.G, topk)
        if offload_idx:
            shared = torch.empty(idx_shape, dtype=torch.int32, device=dev)
            self.idx = {l: shared for l in self.sparse_layers}
        else:
            self.idx = {l: torch.empty(idx_shape, dtype=torch.int32, device=dev) for l in self.sparse_layers}
        self.o = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        self.r = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        # two staging buffers for R at anchors: the D2H store of one overlaps
        # the next anchor's work on the other
        self.r_stage = [self.r, torch.empty(shape, dtype=torch.bfloat16, device=dev)]
        self.out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.desc = mcs.desc_for(self.o)
        self.ws_pddp = torch.empty(mcs.pddp_workspace_size(self.desc, group_size), dtype=torch.uint8, device=dev)
        self.ws_sel = torch.empty(mcs.select_workspace_size(self.desc, group_size, topk), dtype=torch.uint8, device=dev)
        self.power_iters = power_iters
        self.offload = offload
        self.r_bytes = self.r.numel() * self.r.element_size()
        self.cache = mcs.RCache(sched.layers, self.r_bytes) if offload else None
        self.icache = None
        if offload_idx:
            self.bm_bytes = mcs.kv_idx_bitmap_bytes(self.desc, group_size)
            padded = -(-self.bm_bytes // 256) * 256
            self.bm_stage = [torch.zeros(padded // 4, dtype=torch.int32, device=dev) for _ in range(2)]
            self.icache = mcs.RCache(sched.layers, padded)
            self.bm_like = self.bm_stage[0]
        self.r_dev = {} if offload else {l: torch.empty(shape, dtype=torch.bfloat16, device=dev)
                                         for l in self.sparse_layers}
        self.side = torch.cuda.Stream()
        self.plan = plan(sched)

    def close(self):
        if self.cache is not None:
            self.cache.close()
            self.cache = None
        if self.icache is not None:
            self.icache.close()
            self.icache = None

    def _r_view(self, ptr):
        """The R slot returned by the cache, as the caller's bf16 tensor layout."""
        return _DevicePtr(ptr, self.r)

    def run(self, inputs, events=None, outputs=None):
        """Executes the plan. ``events`` (optional dict) collects per-call
        (kind, start, end) CUDA events on the stream that ran the call (an
        anchor call also gives its grouping as "pddp"), and per-step
        ("step", start, end) on the compute stream; ``outputs``
        (optional dict) receives a copy of every layer output by (step, layer)."""
        compute = torch.cuda.current_stream()
        rec = events is not None
        store_done = [None, None]
        n_anchor = 0
        by_step = {}
        for step, layer, act in self.plan:
            by_step.setdefault(step, []).append((layer, act))
        for step in sorted(by_step):
            acts = by_step[step]
            es = _ev(rec)
            reuse_layers = [l for l, a in acts if a == REUSE]
            if self.offload and reuse_layers:
                # the first reuse layer of the step is prefetched before the step starts
                self.side.wait_stream(compute)
                self._prefetch(reuse_layers[0], events)
            for i, (layer, act) in enumerate(acts):
                q, k, v = inputs(step, layer)
                if act == DENSE:
                    e0 = _ev(rec)
                    mcs.anchor_dense_lse(q, k, v, self.out, None)
                    _push(events, "dense", e0, _ev(rec))
                elif act == ANCHOR:
                    e0 = _ev(rec)
                    mcs.pddp_group(q, self.T, self.perm[layer], self.ws_pddp, self.power_iters)
                    _push(events, "pddp", e0, _ev(rec))
                    mcs.anchor_dense_lse(q, k, v, self.o, self.lse)
                    mcs.anchor_select_topk(q, k, self.lse, self.perm[layer], self.T, self.K, self.idx[layer],
                                           ws=self.ws_sel)
                    if self.offload:
                        buf = n_anchor & 1
                        n_anchor += 1
                        if store_done[buf] is not None:
                            compute.wait_event(store_done[buf])  # its previous store has left
                        rdst = self.r_stage[buf]
                    else:
                        rdst = self.r_dev[layer]
                    mcs.residual(q, k, v, self.o, self.perm[layer], self.T, self.idx[layer], self.K, rdst)
                    if self.offload_idx:
                        bdst = self.bm_stage[buf]
                        mcs.kv_idx_encode(self.desc, self.T, self.idx[layer], self.K, bdst)
                    _push(events, "anchor", e0, _ev(rec))
                    if self.offload:
                        # D2H on the side stream, after the residual
                        self.side.wait_stream(compute)
                        e1 = _ev(rec, self.side)
                        self.cache.store(layer, rdst, self.side)
                        if self.offload_idx:
                            self.icache.store(layer, bdst, self.side)
                        _push(events, "store", e1, _ev(rec, self.side))
                        done = torch.cuda.Event()
                        done.record(self.side)
                        store_done[buf] = done
                else:
                    if self.offload:
                        ptr = self.cache.acquire(layer, compute)
                        if self.offload_idx:
                            bptr = self.icache.acquire(layer, compute)
                            e1 = _ev(rec)
                            mcs.kv_idx_decode(self.desc, self.T, _DevicePtr(bptr, self.bm_like), self.K,
                                              self.idx[layer])
                            _push(events, "decode", e1, _ev(rec))
                        nxt = [l for l in reuse_layers if l > layer]
                        if nxt:
                            self._prefetch(nxt[0], events)
                        r_arg = self._r_view(ptr)
                    else:
                        r_arg = self.r_dev[layer]
                    e0 = _ev(rec)
                    mcs.sparse_apply(q, k, v, self.perm[layer], self.T, self.idx[layer], self.K, r_arg, self.out)
                    _push(events, "reuse", e0, _ev(rec))
                if outputs is not None:
                    outputs[(step, layer)] = (self.o if act == ANCHOR else self.out).clone()
            _push(events, "step", es, _ev(rec))

    def _prefetch(self, layer, events):
        rec = events is not None
        e0 = _ev(rec, self.side)
        self.cache.prefetch(layer, self.side)
        if self.icache is not None:
            self.icache.prefetch(layer, self.side)
        _push(events, "prefetch", e0, _ev(rec, self.side))


class _DevicePtr:
    """Stands in for a device tensor at a raw device address (a cache slot),
    with the shape, strides and dtype of ``like``, when passed to the
    binding."""

    is_cuda = True

    def __init__(self, ptr, like):
        self._ptr, self.shape, self._stride, self.dtype = ptr, like.shape, like.stride(), like.dtype
        self._numel, self._esize, self._contig = like.numel(), like.element_size(), like.is_contiguous()

    def data_ptr(self):
        return self._ptr

    def stride(self, *a):
        return self._stride if not a else self._stride[a[0]]

    def numel(self):
        return self._numel

    def element_size(self):
        return self._esize

    def is_contiguous(self):
        return self._contig


def _ev(rec, stream=None):
    if not rec:
        return None
    e = torch.cuda.Event(enable_timing=True)
    e.record(stream)
    return e


def _push(events, kind, e0, e1):
    if events is not None:
        events.setdefault(kind, []).append((e0, e1))
