"""Seeded synthetic inputs for the sparse MoE layer (input generation only).

Both the HIP library's tests/bench and the CPU oracle take their inputs from
here; this package holds none of the layer's arithmetic (no routing, no
dequantisation, no FFN).  Weight draws come from ``gen.c`` (Philox4x32-10 +
Box-Muller, encoded to MXFP4 / NVFP4 / BF16); activations and router logits
from numpy's PCG64 seeded by ``SeedSequence([seed, config, ...])``.

The workloads follow the FreeToken pages' description of where the layer's
inputs come from: a router that picks a few experts per token (page
"FreeToken qwen：ローカルQwen MoEセットアップガイド", second and third
paragraphs) and expert weights in MXFP4 / NVFP4 / BF16 checkpoints (page
"FreeToken量子化：MoE推論のセットアップガイド", third paragraph).  The shapes
are the A3B-like (hidden 2048, 128 experts, top-8, intermediate 768) and
large-expert (hidden 7168, 256 + 1 shared experts, intermediate 2048) shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_gen.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile gen.c into _gen.so with gcc (OpenMP)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               os.path.join(_HERE, "gen.c"), "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_SO)
        u64, f32, i32, i64 = ctypes.c_uint64, ctypes.c_float, ctypes.c_int, ctypes.c_int64
        vp = ctypes.c_void_p
        lib.synth_philox4x32_10.argtypes = [vp, vp, vp]
        lib.synth_normal_f32.argtypes = [u64, u64, f32, vp, i64]
        lib.synth_weight_bf16.argtypes = [u64, u64, f32, i32, i32, vp]
        lib.synth_weight_mxfp4.argtypes = [u64, u64, f32, i32, i32, vp, vp]
        lib.synth_weight_nvfp4.argtypes = [u64, u64, f32, i32, i32, vp, vp, vp]
        lib.synth_weight_fp8.argtypes = [u64, u64, f32, i32, i32, vp, vp]
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    _load().synth_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def normal_f32(seed: int, stream: int, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _load().synth_normal_f32(seed, stream, std, _p(out), n)
    return out


def stream_id(config: int, layer: int, expert: int, tensor: int) -> int:
    """64-bit stream number for one weight tensor: any tensor can be regenerated alone."""
    return ((config & 0xFF) << 56) | ((layer & 0xFFFF) << 40) | ((expert & 0xFFFFFF) << 16) | (tensor & 0xFFFF)


FMTS = ("bf16", "mxfp4", "nvfp4", "fp8")
SHARED_EXPERT = 0xFFFFFF  # expert id used in stream_id() for the always-on shared expert


@dataclass
class Proj:
    """One projection matrix [rows, cols] in canonical (row-major, K-contiguous) layout."""
    rows: int
    cols: int
    w: np.ndarray | None = None   # bf16 bits, uint16 [rows, cols]
    q: np.ndarray | None = None   # packed E2M1 codes, uint8 [rows, cols/2] (FP8: E4M3 codes [rows, cols])
    s: np.ndarray | None = None   # block scales: E8M0 [rows, cols/32] or E4M3 [rows, cols/16]
    g: float = 1.0                # NVFP4 / FP8 per-tensor dequant multiplier


@dataclass
class Expert:
    """A SwiGLU expert: gate, up [I, H] and down [H, I]."""
    fmt: str
    H: int
    I: int
    gate: Proj = field(default=None)
    up: Proj = field(default=None)
    down: Proj = field(default=None)

    def projs(self):
        return (self.gate, self.up, self.down)

    def nbytes(self) -> int:
        n = 0
        for p in self.projs():
            for a in (p.w, p.q, p.s):
                if a is not None:
                    n += a.nbytes
            if self.fmt in ("nvfp4", "fp8"):
                n += 4
        return n


def _proj(fmt, seed, stream, rows, cols, std) -> Proj:
    lib = _load()
    p = Proj(rows, cols)
    if fmt == "bf16":
        p.w = np.empty((rows, cols), np.uint16)
        lib.synth_weight_bf16(seed, stream, std, rows, cols, _p(p.w))
    elif fmt == "mxfp4":
        assert cols % 32 == 0
        p.q = np.empty((rows, cols // 2), np.uint8)
        p.s = np.empty((rows, cols // 32), np.uint8)
        lib.synth_weight_mxfp4(seed, stream, std, rows, cols, _p(p.q), _p(p.s))
    elif fmt == "nvfp4":
        assert cols % 16 == 0
        p.q = np.empty((rows, cols // 2), np.uint8)
        p.s = np.empty((rows, cols // 16), np.uint8)
        g = np.zeros(1, np.float32)
        lib.synth_weight_nvfp4(seed, stream, std, rows, cols, _p(p.q), _p(p.s), _p(g))
        p.g = float(g[0])
    elif fmt == "fp8":
        p.q = np.empty((rows, cols), np.uint8)
        g = np.zeros(1, np.float32)
        lib.synth_weight_fp8(seed, stream, std, rows, cols, _p(p.q), _p(g))
        p.g = float(g[0])
    else:
        raise ValueError(fmt)
    return p


def expert(fmt: str, H: int, I: int, *, seed: int = 0, config: int = 0, layer: int = 0,
           expert_id: int = 0, std: float = 0.02) -> Expert:
    """Weights N(0, std) drawn per (seed, config, layer, expert, tensor) and encoded to fmt."""
    e = Expert(fmt, H, I)
    e.gate = _proj(fmt, seed, stream_id(config, layer, expert_id, 0), I, H, std)
    e.up = _proj(fmt, seed, stream_id(config, layer, expert_id, 1), I, H, std)
    e.down = _proj(fmt, seed, stream_id(config, layer, expert_id, 2), H, I, std)
    return e


# ---------------------------------------------------------------- activations

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = 0x7FFF + ((u >> 16) & 1)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) & 0xFFFFFFFF for k in key]))


def activations(T: int, H: int, *key: int) -> np.ndarray:
    """x [T, H] as bf16 bits, N(0,1) rounded to bf16."""
    return f32_to_bf16_bits(rng(*key).standard_normal((T, H), dtype=np.float32))


def router_weight(E: int, H: int, *key: int, std: float = 0.02) -> np.ndarray:
    return (rng(*key).standard_normal((E, H), dtype=np.float32) * np.float32(std)).astype(np.float32)


def zipf_rank_to_expert(E: int, *key: int) -> np.ndarray:
    """Seeded permutation: rank r (0 = most popular) -> expert id."""
    return rng(*key).permutation(E).astype(np.int64)


def zipf_logits(T: int, E: int, rank_to_expert: np.ndarray, g: np.random.Generator,
                s: float = 1.1) -> np.ndarray:
    """logits[t, e] = log p_rank(e) + Gumbel(0,1), p_r proportional to r^-s (r = 1..E).

    The top-k of such a row is a draw of k experts without replacement with
    probabilities p (the Gumbel-top-k construction), so expert popularity
    follows Zipf(s)."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    logp = np.empty(E, np.float64)
    logp[rank_to_expert] = np.log(p)
    u = g.random((T, E))
    u = np.clip(u, 1e-300, 1.0 - 1e-16)
    gumbel = -np.log(-np.log(u))
    return (logp[None, :] + gumbel).astype(np.float32)


# ---------------------------------------------------------------- the five workloads

SEED = 0

TINY = dict(H=256, E=8, k=2, I=128, T=16, fmt="mxfp4")
A3B = dict(H=2048, E=128, k=8, I=768)
LARGE = dict(H=7168, E=256, k=8, I=2048)
STREAM = dict(layers=48, slots=2048, tokens=512, repeat_p=0.6)


def tiny_layer(seed: int = SEED) -> dict:
    """Tiny layer: hidden 256, 8 experts, top-2, intermediate 128, 16 tokens, MXFP4, router weight given."""
    c = TINY
    return dict(
        cfg=0, T=c["T"], H=c["H"], E=c["E"], k=c["k"], I=c["I"], fmt=c["fmt"],
        x=activations(c["T"], c["H"], seed, 0, 1),
        w_router=router_weight(c["E"], c["H"], seed, 0, 2),
        experts=[expert(c["fmt"], c["H"], c["I"], seed=seed, config=0, expert_id=e) for e in range(c["E"])],
    )


def decode_batch(T: int, batch_index: int = 0, seed: int = SEED) -> dict:
    """A3B-like decode batch: x [T, 2048] and Zipf(1.1) logits [T, 128]; weights via a3b_experts()."""
    c = A3B
    r2e = zipf_rank_to_expert(c["E"], seed, 1, 7)
    g = rng(seed, 1, 8, T, batch_index)
    return dict(cfg=1, T=T, H=c["H"], E=c["E"], k=c["k"], I=c["I"],
                x=activations(T, c["H"], seed, 1, 9, T, batch_index),
                logits=zipf_logits(T, c["E"], r2e, g))


def a3b_experts(fmt: str, config: int, seed: int = SEED, layer: int = 0, ids=None):
    c = A3B
    ids = range(c["E"]) if ids is None else ids
    return [expert(fmt, c["H"], c["I"], seed=seed, config=config, layer=layer, expert_id=e) for e in ids]


def prefill_batch(T: int = 4096, n_masked: int = 8, seed: int = SEED) -> dict:
    """A3B-like prefill: Zipf logits plus n_masked experts (drawn from the 64 least popular
    ranks) whose logits are set to -1e4 so that they receive no token."""
    c = A3B
    r2e = zipf_rank_to_expert(c["E"], seed, 2, 7)
    g = rng(seed, 2, 8, T)
    logits = zipf_logits(T, c["E"], r2e, g)
    cold = r2e[c["E"] - 64:]
    masked = np.sort(rng(seed, 2, 10).choice(cold, size=n_masked, replace=False))
    logits[:, masked] = np.float32(-1e4)
    return dict(cfg=2, T=T, H=c["H"], E=c["E"], k=c["k"], I=c["I"], masked=masked,
                x=activations(T, c["H"], seed, 2, 9, T), logits=logits)


def large_batch(T: int, seed: int = SEED, batch_index: int = 0) -> dict:
    """Large-expert layer input: x [T, 7168] and router weight [256, 7168] N(0, 0.02).
    batch_index > 0 draws another x (the router weight is the layer's, the same for all)."""
    c = LARGE
    key = (seed, 3, 9, T) if batch_index == 0 else (seed, 3, 9, T, batch_index)
    return dict(cfg=3, T=T, H=c["H"], E=c["E"], k=c["k"], I=c["I"],
                x=activations(T, c["H"], *key),
                w_router=router_weight(c["E"], c["H"], seed, 3, 2))


def large_expert(e: int, seed: int = SEED) -> Expert:
    """Routed expert e (0..255) or the shared expert (e = SHARED_EXPERT), MXFP4."""
    c = LARGE
    return expert("mxfp4", c["H"], c["I"], seed=seed, config=3, expert_id=e)


def stream_routing(tokens: int = 512, layers: int = 48, E: int = 128, repeat_p: float = 0.6,
                   seed: int = SEED) -> np.ndarray:
    """Cached-decode-stream logits [tokens, layers, E].

    Per layer a seeded Zipf(1.1) rank permutation; for t > 0, independently per
    (t, layer), with probability repeat_p the previous token's row is reused,
    otherwise a fresh Zipf-Gumbel row is drawn."""
    out = np.empty((tokens, layers, E), np.float32)
    g = rng(seed, 4, 8)
    r2e = [zipf_rank_to_expert(E, seed, 4, 7, l) for l in range(layers)]
    rep = g.random((tokens, layers)) < repeat_p
    for l in range(layers):
        fresh = zipf_logits(tokens, E, r2e[l], rng(seed, 4, 11, l))
        for t in range(tokens):
            out[t, l] = out[t - 1, l] if (t > 0 and rep[t, l]) else fresh[t]
    return out


def stream_activations(t: int, layer: int, H: int = 2048, seed: int = SEED) -> np.ndarray:
    """Fresh x [1, H] per (token, layer) for the cached stream (not chained)."""
    return activations(1, H, seed, 4, 9, t, layer)
