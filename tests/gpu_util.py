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


def grouped_reference(x_bits, ids, w, E, make_expert, *, shared=None, amode="bf16", h_codes=None, workers=None):
    """Whole-output reference of one layer call: oracle.moe.layer_outputs with
    each active expert's weights generated and dequantised ahead of use in a
    thread pool (at most `workers` experts held at once)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    workers = workers or min(16, len(os.sched_getaffinity(0)))
    order = sorted(set(int(e) for e in np.asarray(ids).ravel()))
    pos = {e: i for i, e in enumerate(order)}
    futs = {}
    with ThreadPoolExecutor(workers) as ex:
        def submit(i):
            if i < len(order):
                futs[order[i]] = ex.submit(lambda e=order[i]: oracle.moe.dequant_expert(make_expert(e)))
        for i in range(workers):
            submit(i)

        def weights(e):
            W = futs.pop(e).result()
            submit(pos[e] + workers)
            return W
        sw = oracle.moe.dequant_expert(shared) if shared is not None else None
        return oracle.moe.layer_outputs(x_bits, np.asarray(ids), np.asarray(w), E, weights, shared_weights=sw,
                                        amode=amode, h_codes=h_codes)


def gpu_fp4_codes(layer, T, x, which):
    """The MXFP4 encoding of x (which 0) or h (1) the layer's last FP4 call left
    in its workspace: (E2M1 codes [R, K], E8M0 [R, K/32]) in permutation order."""
    from fp4_expert_ffn_amd import moe_debug_fp4_codes
    a = layer.args(T, x)
    R = T * layer.k + (T if layer.shared_blob is not None else 0)
    K = layer.H if which == 0 else layer.I
    q = torch.empty((R, K // 2), dtype=torch.uint8, device=DEV)
    s = torch.empty((R, K // 32), dtype=torch.uint8, device=DEV)
    moe_debug_fp4_codes(a, which, q, s)
    torch.cuda.synchronize()
    return oracle.formats.unpack_e2m1(q.cpu().numpy()), s.cpu().numpy()


def fp4_code_report(layer, T, x_dev, x_bits, perm, k, h_ref, shared=False):
    """R15 checks of the FP4 path: x's encoding bit-exact (per permuted row,
    the token's row); the fraction of SwiGLU-output values whose encoding
    (code and block scale) differs from the oracle's.  Returns that fraction."""
    xc, xs = gpu_fp4_codes(layer, T, x_dev, 0)
    rows = np.concatenate([np.asarray(perm) // k, np.arange(T)]) if shared else np.asarray(perm) // k
    oc, os_ = oracle.quant.quantize_mxfp4_rows(synth.bf16_bits_to_f32(x_bits)[rows])
    assert np.array_equal(xs, os_), "x block scales differ from the oracle's"
    assert np.array_equal(xc, oc), "x codes differ from the oracle's"
    hc, hs = gpu_fp4_codes(layer, T, x_dev, 1)
    assert hc.shape == h_ref["codes"].shape and hs.shape == h_ref["scales"].shape
    gv = oracle.quant.dequantize_mxfp4_codes(hc, hs)
    ov = oracle.quant.dequantize_mxfp4_codes(h_ref["codes"], h_ref["scales"])
    frac = float(np.mean(gv != ov))
    blk = float(np.mean(hs != h_ref["scales"]))
    say(f"    h encodings differing from the oracle's: {frac:.2e} of values, {blk:.2e} of block scales")
    return frac
