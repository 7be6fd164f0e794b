"""One sparse MoE layer on the GPU: device buffers plus the sequence of C-ABI calls.

    [moe_router_logits] -> moe_route -> moe_permute -> moe_expert_ffn (+ combine)

and a decode stream over many layers whose experts live in pinned host memory
behind the HBM expert-slot cache (moe_cache_decode_step per layer and token).

This module only allocates torch device memory and calls the library; every
step of the computation runs in libmoe's HIP kernels.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L


def blob_of(ex) -> np.ndarray:
    """Prepack an expert given in canonical layout (objects with fmt/H/I/gate/up/down,
    each projection with w or (q, s, g))."""
    def proj(p):
        if ex.fmt == "bf16":
            return (p.w, None, 1.0)
        return (p.q, p.s, p.g)
    return L.moe_prepack_expert(ex.fmt, ex.H, ex.I, proj(ex.gate), proj(ex.up), proj(ex.down))


class LayerState:
    """Per-batch buffers of one layer call: routing, permutation, outputs, workspace."""

    def __init__(self, layer: "MoELayer", max_tokens: int):
        dev, E, k, H = layer.dev, layer.E, layer.k, layer.H
        T = max(max_tokens, 1)
        self.layer = layer
        self.max_tokens = T
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.zeros(E, dtype=torch.int32, device=dev)
        self.offsets = torch.zeros(E + 1, dtype=torch.int32, device=dev)
        self.perm = torch.zeros(T * k, dtype=torch.int32, device=dev)
        self.inv = torch.zeros(T * k, dtype=torch.int32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.int16, device=dev)
        rows = T * k + (T if layer.shared_blob is not None else 0)
        self.y = torch.empty((rows, H), dtype=torch.float32, device=dev)
        self._ws = None
        self._args = {}

    def args(self, T, x, out=True, mask=None):
        key = (T, x.data_ptr(), out, None if mask is None else mask.data_ptr())
        if key in self._args:
            return self._args[key][0]
        lay = self.layer
        a = L.ffn_args(T=T, k=lay.k, E=lay.E, H=lay.H, I=lay.I, wfmt=lay.fmt, amode=lay.amode, x=x,
                       counts=self.counts, offsets=self.offsets, perm=self.perm,
                       slot_of_expert=lay.slot_of_expert, slot_pool=lay.pool, slot_stride=lay.stride,
                       shared_blob=lay.shared_blob, expert_mask=mask, y=None if out else self.y,
                       topk_w=self.w if out else None, inv=self.inv if out else None,
                       out=self.out if out else None)
        need = L.moe_expert_ffn_workspace_size(a)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=lay.dev)
            self._args.clear()
        a.workspace = self._ws.data_ptr()
        a.workspace_bytes = self._ws.numel()
        self._args[key] = (a, x)  # keep x alive with its args
        return a

    def route(self, T, x=None, w_router=None, logits=None, stream=None):
        lay = self.layer
        if logits is None:
            L.moe_router_logits(x, w_router, T, lay.H, lay.E, self.logits, stream)
            logits = self.logits
        L.moe_route_permute(logits, T, lay.E, lay.k, lay.renormalize, self.ids, self.w, self.counts, self.offsets,
                            self.perm, self.inv, stream)

    def ffn(self, T, x, stream=None, args=None):
        L.moe_expert_ffn(args if args is not None else self.args(T, x), stream)

    def layer_args(self, T, x, logits):
        """moe_layer arguments: routing outputs into this state's buffers, the combined output in out."""
        la = L.LayerArgs()
        la.logits, la.renormalize, la.topk_ids = L.ptr(logits), 1 if self.layer.renormalize else 0, self.ids.data_ptr()
        la.ffn = self.args(T, x)
        return la

    def call(self, T, x, *, logits=None, w_router=None, stream=None, la=None):
        """One layer call: router logits (if w_router is given), then moe_layer."""
        if logits is None:
            L.moe_router_logits(x, w_router, T, self.layer.H, self.layer.E, self.logits, stream)
            logits = self.logits
        L.moe_layer(la if la is not None else self.layer_args(T, x, logits), stream)

    def forward(self, x, *, logits=None, w_router=None, stream=None):
        T = x.shape[0]
        assert T <= self.max_tokens
        self.call(T, x, logits=logits, w_router=w_router, stream=stream)
        self.last_x = x
        return self.out[:T]


class MoELayer:
    """Fully resident layer: expert e's blob sits in slot e of an HBM slot pool."""

    def __init__(self, *, E, k, H, I, fmt, max_tokens, device="cuda", shared=False, amode="bf16",
                 renormalize=True, num_slots=None):
        self.E, self.k, self.H, self.I, self.fmt = E, k, H, I, fmt
        self.amode, self.renormalize = amode, renormalize
        self.dev = torch.device(device)
        self.blob_bytes = L.moe_blob_bytes(fmt, H, I)
        self.stride = (self.blob_bytes + 255) // 256 * 256
        self.num_slots = num_slots or E
        self.pool = torch.empty(self.num_slots * self.stride, dtype=torch.uint8, device=self.dev)
        self.slot_of_expert = torch.arange(E, dtype=torch.int32, device=self.dev)
        self.shared_blob = torch.empty(self.stride, dtype=torch.uint8, device=self.dev) if shared else None
        self.state = LayerState(self, max_tokens)

    # ------------------------------------------------------------ weights
    def load_expert(self, e: int, blob: np.ndarray):
        assert blob.size == self.blob_bytes
        self.pool[e * self.stride:e * self.stride + blob.size].copy_(torch.from_numpy(blob))

    def load_shared(self, blob: np.ndarray):
        assert self.shared_blob is not None and blob.size == self.blob_bytes
        self.shared_blob[:blob.size].copy_(torch.from_numpy(blob))

    def new_state(self, max_tokens: int) -> LayerState:
        return LayerState(self, max_tokens)

    # ------------------------------------------------------------ default state
    def __getattr__(self, name):
        if name in ("logits", "ids", "w", "counts", "offsets", "perm", "inv", "out", "y", "args", "route", "ffn",
                    "forward", "check", "call", "layer_args"):
            return getattr(self.__dict__["state"], name)
        raise AttributeError(name)


class CachedDecoder:
    """Decode through the expert-slot cache: `num_layers` layers of `num_experts`
    experts whose blobs sit in a pinned host bank, `num_slots` HBM slots shared
    by every layer under LRU; misses copied from host memory by a fill kernel
    on the compute stream while the hits run on a side stream (or by the copy
    engine, see moe_cache_decode_step).

    host_blob(layer, e) -> pinned uint8 tensor holding that expert's blob.
    copy_ratio: None copies every miss into the cache; a value in [0, 1] runs
    the hybrid policy (that share of a step's misses copied, the rest run on
    the host with `host_threads` threads, not cached).
    copy_engine: copy misses through the copy engine on the side stream even
    where a fill kernel on the compute stream could copy them.
    """

    def __init__(self, *, num_layers, num_experts, k, H, I, fmt, num_slots, host_blob, max_tokens=1,
                 device="cuda", renormalize=True, copy_ratio=None, host_threads=8, copy_engine=False):
        self.L, self.E, self.k, self.H, self.I, self.fmt = num_layers, num_experts, k, H, I, fmt
        self.dev = torch.device(device)
        self.blob_bytes = L.moe_blob_bytes(fmt, H, I)
        self.stride = (self.blob_bytes + 255) // 256 * 256
        self.pool = torch.empty(num_slots * self.stride, dtype=torch.uint8, device=self.dev)
        self.cache = L.moe_cache_create(num_slots, self.stride, self.pool, num_layers, num_experts)
        if copy_engine:
            L.moe_cache_use_copy_engine(self.cache, True)
        self.copy_stream = torch.cuda.Stream(device=self.dev)
        self._copy_handle = self.copy_stream.cuda_stream
        T, E = max(max_tokens, 1), num_experts
        self.max_tokens = T
        # host blob table per layer (pinned blobs must hold `stride` bytes: the copy moves whole slots)
        self._blobs = [[host_blob(l, e) for e in range(E)] for l in range(num_layers)]
        for row in self._blobs:
            for b in row:
                assert b.is_pinned() and b.numel() >= self.stride
        self._tables = [(ctypes.c_void_p * E)(*[b.data_ptr() for b in row]) for row in self._blobs]
        mb = L.moe_cache_map_bytes(E)
        self.host_counts = torch.empty(E, dtype=torch.int32, pin_memory=True)
        self.host_map = torch.empty(mb, dtype=torch.uint8, pin_memory=True)
        self.dev_map = torch.empty(mb, dtype=torch.uint8, device=self.dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=self.dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=self.dev)
        self.counts = torch.zeros(E, dtype=torch.int32, device=self.dev)
        self.offsets = torch.zeros(E + 1, dtype=torch.int32, device=self.dev)
        self.perm = torch.zeros(T * k, dtype=torch.int32, device=self.dev)
        self.inv = torch.zeros(T * k, dtype=torch.int32, device=self.dev)
        self.y = torch.empty((T * k, H), dtype=torch.float32, device=self.dev)
        self.out = torch.empty((T, H), dtype=torch.int16, device=self.dev)
        self.trace = [np.empty(E, np.int32), np.empty(E, np.int32), np.empty(E, np.uint8), np.empty(E, np.int32)]
        self.hybrid = None
        if copy_ratio is not None:
            self._hx = torch.empty((T, H), dtype=torch.int16, pin_memory=True)
            self._hperm = torch.empty(T * k, dtype=torch.int32, pin_memory=True)
            self._hoff = torch.empty(E + 1, dtype=torch.int32, pin_memory=True)
            self._hy = torch.empty((T * k, H), dtype=torch.float32, pin_memory=True)
            self.hybrid = L.Hybrid(float(copy_ratio), int(host_threads), self._hx.data_ptr(), self._hperm.data_ptr(),
                                   self._hoff.data_ptr(), self._hy.data_ptr(), 0)
        self._trace_ptrs = tuple(t.ctypes.data for t in self.trace)
        self._steps = {}
        self._ws = None

    def _step(self, layer, T, x, logits, out):
        key = (layer, T)
        st = self._steps.get(key)
        if st is None:
            a = L.ffn_args(T=T, k=self.k, E=self.E, H=self.H, I=self.I, wfmt=self.fmt, amode="bf16", x=x,
                           counts=self.counts, offsets=self.offsets, perm=self.perm, slot_pool=self.pool,
                           slot_stride=self.stride, y=self.y, topk_w=self.w, inv=self.inv, out=out)
            need = L.moe_expert_ffn_workspace_size(a)
            if self._ws is None or self._ws.numel() < need:
                self._ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.dev)
                for s in self._steps.values():
                    s.ffn.workspace, s.ffn.workspace_bytes = self._ws.data_ptr(), self._ws.numel()
            a.workspace, a.workspace_bytes = self._ws.data_ptr(), self._ws.numel()
            st = L.CacheStep()
            st.layer, st.renormalize = layer, 1
            st.topk_ids = self.ids.data_ptr()
            st.host_counts, st.host_map, st.dev_map = (self.host_counts.data_ptr(), self.host_map.data_ptr(),
                                                       self.dev_map.data_ptr())
            st.host_blobs = ctypes.cast(self._tables[layer], ctypes.c_void_p)
            st.ffn = a
            tr = self.trace
            st.trace_expert, st.trace_slot, st.trace_hit, st.trace_evicted = (t.ctypes.data for t in tr)
            self._steps[key] = st
        st.logits = logits.data_ptr()
        st.ffn.x = x.data_ptr()
        st.ffn.out = out.data_ptr()
        return st

    def step(self, layer, x, logits, out=None, stream=None):
        """One layer of one decode step: x [T,H] bf16 (int16), logits [T,E] fp32 on the device.
        Returns the output [T,H] (bf16 bits) and the step's trace
        (expert, slot, hit, evicted_key) as host arrays."""
        T = x.shape[0]
        assert T <= self.max_tokens
        out = self.out[:T] if out is None else out
        st = self._step(layer, T, x, logits, out)
        st.trace_expert, st.trace_slot, st.trace_hit, st.trace_evicted = self._trace_ptrs
        self._run_step(st, stream)
        n = st.n_experts
        return out, tuple(t[:n].copy() for t in self.trace)

    def step_fast(self, layer, x, logits, stream_handle, trace=None):
        """step() without copying the trace back (stream_handle: raw hipStream_t
        of the compute stream).  trace: None, or four host addresses (expert,
        slot, hit, evicted-key arrays of capacity E) that receive this step's
        records.  Returns the step's number of distinct experts."""
        T = x.shape[0]
        st = self._step(layer, T, x, logits, self.out[:T])
        st.trace_expert, st.trace_slot, st.trace_hit, st.trace_evicted = trace or self._trace_ptrs
        self._run_step(st, stream_handle)
        return st.n_experts

    def step_raw(self, layer, x_ptr, logits_ptr, stream_handle, trace=None, T=1):
        """step_fast() on raw device addresses (x_ptr: [T,H] bf16, logits_ptr:
        [T,E] fp32), with no tensor work on the host; the output lands in
        self.out[:T].  Returns the step's number of distinct experts."""
        st = self._steps.get((layer, T))
        if st is None:
            st = self._step(layer, T, self.out[:T], self.w[:T], self.out[:T])  # placeholders, replaced below
        st.logits = logits_ptr
        st.ffn.x = x_ptr
        st.trace_expert, st.trace_slot, st.trace_hit, st.trace_evicted = trace or self._trace_ptrs
        if self.hybrid is None:
            r = L.lib().moe_cache_decode_step(self.cache.handle, ctypes.byref(st), self._copy_handle, stream_handle)
        else:
            r = L.lib().moe_cache_decode_step_hybrid(self.cache.handle, ctypes.byref(st), ctypes.byref(self.hybrid),
                                                     self._copy_handle, stream_handle)
        if r != L.MOE_OK:
            raise L.MoeError(r, f"moe_cache_decode_step: {L.moe_last_error()}")
        return st.n_experts

    def _run_step(self, st, stream):
        if self.hybrid is None:
            L.moe_cache_decode_step(self.cache, st, self.copy_stream, stream)
        else:
            L.moe_cache_decode_step_hybrid(self.cache, st, self.hybrid, self.copy_stream, stream)

    def stats(self):
        return L.moe_cache_stats(self.cache)

    def resize(self, num_slots, stream=None):
        """Move the cache to `num_slots` slots between steps (the most recent
        keys kept); the old pool is released once the copies have finished."""
        pool = torch.empty(num_slots * self.stride, dtype=torch.uint8, device=self.dev)
        L.moe_cache_resize(self.cache, num_slots, pool, stream)
        s = torch.cuda.current_stream(self.dev) if stream is None else stream
        s.synchronize()
        self.pool = pool
        for st in self._steps.values():
            st.ffn.slot_pool = pool.data_ptr()

    def reset(self):
        L.moe_cache_reset(self.cache)
        if self.hybrid is not None:
            self.hybrid.cpu_experts = 0

    def close(self):
        self.cache.close()


class CachedPrefill:
    """Prefill through the expert-slot cache, one layer ahead: while layer l
    computes, every expert of layer l + 1 is copied from the pinned host bank
    on a side stream into a cache of `num_slots` slots (default 2E: the layer
    computing and the layer arriving).

    host_blob(layer, e) -> pinned uint8 tensor holding that expert's blob.
    """

    def __init__(self, *, num_layers, num_experts, k, H, I, fmt, max_tokens, host_blob, amode="bf16",
                 num_slots=None, device="cuda", renormalize=True):
        self.L, self.E, self.k, self.H, self.I, self.fmt, self.amode = num_layers, num_experts, k, H, I, fmt, amode
        self.renormalize = 1 if renormalize else 0
        self.dev = torch.device(device)
        self.blob_bytes = L.moe_blob_bytes(fmt, H, I)
        self.stride = (self.blob_bytes + 255) // 256 * 256
        self.num_slots = num_slots or 2 * num_experts
        self.pool = torch.empty(self.num_slots * self.stride, dtype=torch.uint8, device=self.dev)
        self.cache = L.moe_cache_create(self.num_slots, self.stride, self.pool, num_layers, num_experts)
        self.copy_stream = torch.cuda.Stream(device=self.dev)
        E, T = num_experts, max(max_tokens, 1)
        self.max_tokens = T
        self._blobs = [[host_blob(l, e) for e in range(E)] for l in range(num_layers)]
        for row in self._blobs:
            for b in row:
                assert b.is_pinned() and b.numel() >= self.stride
        self._tables = [(ctypes.c_void_p * E)(*[b.data_ptr() for b in row]) for row in self._blobs]
        mb = L.moe_cache_map_bytes(E)
        # one slot map per layer: layer l's step reads its map while layer l + 1's is uploaded
        self.host_maps = [torch.empty(mb, dtype=torch.uint8, pin_memory=True) for _ in range(num_layers)]
        self.dev_maps = [torch.empty(mb, dtype=torch.uint8, device=self.dev) for _ in range(num_layers)]
        self.ids = torch.empty((T, k), dtype=torch.int32, device=self.dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=self.dev)
        self.counts = torch.zeros(E, dtype=torch.int32, device=self.dev)
        self.offsets = torch.zeros(E + 1, dtype=torch.int32, device=self.dev)
        self.perm = torch.zeros(T * k, dtype=torch.int32, device=self.dev)
        self.inv = torch.zeros(T * k, dtype=torch.int32, device=self.dev)
        a = self._args(T, None, None)
        need = L.moe_expert_ffn_workspace_size(a)
        self._ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=self.dev)
        self.trace = (np.empty(E, np.int32), np.empty(E, np.uint8), np.empty(E, np.int32))

    def _args(self, T, x, out):
        a = L.ffn_args(T=T, k=self.k, E=self.E, H=self.H, I=self.I, wfmt=self.fmt, amode=self.amode, x=x,
                       counts=self.counts, offsets=self.offsets, perm=self.perm, topk_w=self.w, inv=self.inv, out=out,
                       slot_stride=self.stride)
        if getattr(self, "_ws", None) is not None:
            a.workspace, a.workspace_bytes = self._ws.data_ptr(), self._ws.numel()
        return a

    def prefetch(self, layer, stream=None):
        """Queue the copies of every expert of `layer` not cached yet; returns
        the lookups (slot, hit, evicted key) of experts 0..E-1."""
        L.moe_cache_prefetch_layer(self.cache, layer, self._tables[layer], self.host_maps[layer],
                                   self.dev_maps[layer], self.trace, self.copy_stream, stream)
        return tuple(t.copy() for t in self.trace)

    def layer_step(self, layer, x, logits, out, stream=None):
        """One prefill step of a prefetched layer: x [T,H] bf16 (int16), logits
        [T,E] fp32, out [T,H] (int16) on the device.  Returns the step's lookups
        (expert, hit, slot, evicted key) of experts 0..E-1."""
        T = x.shape[0]
        assert T <= self.max_tokens
        st = L.CachePrefill()
        st.layer, st.renormalize = layer, self.renormalize
        st.logits, st.topk_ids, st.dev_map = logits.data_ptr(), self.ids.data_ptr(), self.dev_maps[layer].data_ptr()
        st.ffn = self._args(T, x, out)
        slot, hit, ev = self.trace
        st.trace_slot, st.trace_hit, st.trace_evicted = slot.ctypes.data, hit.ctypes.data, ev.ctypes.data
        L.moe_cache_prefill_step(self.cache, st, stream)
        return np.arange(self.E, dtype=np.int32), hit.copy(), slot.copy(), ev.copy()

    def run(self, xs, logits, outs, stream=None):
        """Every layer in order, each layer's experts prefetched while the
        previous layer computes; returns each step's lookups."""
        traces = []
        self.prefetch(0, stream)
        for l in range(self.L):
            traces.append(self.layer_step(l, xs[l], logits[l], outs[l], stream))
            if l + 1 < self.L:
                self.prefetch(l + 1, stream)
        return traces

    def stats(self):
        return L.moe_cache_stats(self.cache)

    def close(self):
        self.cache.close()


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns (uint16 numpy) as an int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def to_numpy_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)
