"""One sparse MoE layer on the GPU: device buffers plus the sequence of C-ABI calls.

    [moe_router_logits] -> moe_route -> moe_permute -> moe_expert_ffn (+ combine)

This module only allocates torch device memory and calls the library; every
step of the computation runs in libmoe's HIP kernels.
"""
from __future__ import annotations

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
                       shared_blob=lay.shared_blob, expert_mask=mask, y=self.y,
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

    def check(self, stream=None):
        """Verify the workspace counters (synchronises the stream)."""
        if self._ws is not None:
            L.moe_workspace_check(self._ws, stream)

    def route(self, T, x=None, w_router=None, logits=None, stream=None):
        lay = self.layer
        if logits is None:
            L.moe_router_logits(x, w_router, T, lay.H, lay.E, self.logits, stream)
            logits = self.logits
        L.moe_route_permute(logits, T, lay.E, lay.k, lay.renormalize, self.ids, self.w, self.counts, self.offsets,
                            self.perm, self.inv, stream)

    def ffn(self, T, x, stream=None, args=None):
        L.moe_expert_ffn(args if args is not None else self.args(T, x), stream)

    def forward(self, x, *, logits=None, w_router=None, stream=None):
        T = x.shape[0]
        assert T <= self.max_tokens
        self.route(T, x=x, w_router=w_router, logits=logits, stream=stream)
        self.ffn(T, x, stream)
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
                    "forward", "check"):
            return getattr(self.__dict__["state"], name)
        raise AttributeError(name)


def bf16_tensor(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns (uint16 numpy) as an int16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def to_numpy_bf16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)
