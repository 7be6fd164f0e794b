"""Helpers shared by the GPU parity tests (inputs from synth, references from oracle)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")

DEV = "cuda:0"


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    """Progress line naming the case, flushed before the GPU step that follows."""
    print(*a, flush=True)
    sys.stdout.flush()


def resident_layer(experts, *, k, T, shared=None, amode="bf16", renormalize=True):
    from fp4_expert_ffn_amd.layer import MoELayer, blob_of
    ex0 = experts[0]
    layer = MoELayer(E=len(experts), k=k, H=ex0.H, I=ex0.I, fmt=ex0.fmt, max_tokens=max(T, 1), device=DEV,
                     shared=shared is not None, amode=amode, renormalize=renormalize)
    for e, ex in enumerate(experts):
        if ex is not None:
            layer.load_expert(e, blob_of(ex))
    if shared is not None:
        layer.load_shared(blob_of(shared))
    return layer


def out_f32(layer, T):
    from fp4_expert_ffn_amd.layer import to_numpy_bf16
    return synth.bf16_bits_to_f32(to_numpy_bf16(layer.out[:T]))


class DequantCache:
    """float64 dequantised weights per expert, generated on demand (oracle side)."""

    def __init__(self, make, cap=48):
        self.make, self.cap, self.d = make, cap, {}

    def __call__(self, e):
        if e not in self.d:
            if len(self.d) >= self.cap:
                self.d.pop(next(iter(self.d)))
            self.d[e] = oracle.moe.dequant_expert(self.make(e))
        return self.d[e]


def sample_tokens(perm, offsets, k, T, n_random, seed):
    """Tokens to check at full size: first/last tokens, random ones, and for several
    experts the token of the expert's last row (the ragged tail of its last tile)."""
    rng = np.random.default_rng(seed)
    toks = {0, T - 1}
    toks.update(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    E = offsets.size - 1
    nonempty = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    for e in rng.choice(nonempty, size=min(6, len(nonempty)), replace=False):
        toks.add(int(perm[offsets[e + 1] - 1] // k))
        toks.add(int(perm[offsets[e]] // k))
    biggest = int(np.argmax(np.diff(offsets)))
    toks.add(int(perm[offsets[biggest + 1] - 1] // k))
    return sorted(toks)
