"""Pins for the expert FFN, the combine and the whole layer.

Independent references: torch (float64 matmul and torch.nn.functional.silu),
scalar triple loops in pure Python on tiny shapes, and the dense formulas."""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as M
from oracle import quant as Q


def _torch_swiglu(Wg, Wu, Wd, X):
    Xt = torch.from_numpy(X)
    g = Xt @ torch.from_numpy(Wg).T
    u = Xt @ torch.from_numpy(Wu).T
    return ((torch.nn.functional.silu(g) * u) @ torch.from_numpy(Wd).T).numpy()


@pytest.mark.parametrize("fmt", synth.FMTS)
def test_one_expert_top1_is_dense_swiglu(fmt):
    H, I, T = 128, 64, 5
    ex = synth.expert(fmt, H, I, seed=5, config=99, expert_id=0)
    x = synth.activations(T, H, 5, 99, 1)
    res = M.layer(x, [ex], 1, logits=np.zeros((T, 1), np.float32))
    assert np.all(res["ids"] == 0) and np.all(res["w"] == 1.0)
    Wg, Wu, Wd = (F.dequant(p, fmt) for p in ex.projs())
    ref = _torch_swiglu(Wg, Wu, Wd, F.bf16_to_f64(x))
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-15)


def test_k_equals_E_is_softmax_weighted_sum():
    H, I, T, E = 64, 32, 4, 3
    exs = [synth.expert("mxfp4", H, I, seed=6, config=98, expert_id=e) for e in range(E)]
    x = synth.activations(T, H, 6, 98, 1)
    logits = np.random.default_rng(0).standard_normal((T, E)).astype(np.float32)
    res = M.layer(x, exs, E, logits=logits)
    p = torch.softmax(torch.from_numpy(logits).double(), 1).numpy()
    X = F.bf16_to_f64(x)
    dense = sum(p[:, [e]] * _torch_swiglu(*(F.dequant(q, "mxfp4") for q in exs[e].projs()), X) for e in range(E))
    # the routing weights are float32 (relative rounding 2^-24 each)
    np.testing.assert_allclose(res["out"], dense, rtol=0, atol=1e-6 * np.abs(dense).max())


def _scalar_layer(x, exs, k, logits, amode):
    """Pure-Python loops: dense per-token formula, no numpy linear algebra."""
    T, H = x.shape
    E = len(exs)
    Ws = [[F.dequant(p, exs[e].fmt).tolist() for p in exs[e].projs()] for e in range(E)]
    X = F.bf16_to_f64(x)
    out = []
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))[:k]
        m = row[order[0]]
        ex = [math.exp(row[e] - m) for e in order]
        ws = [v / sum(ex) for v in ex]
        xr = X[t].tolist()
        if amode == "mxfp4":
            xr = Q.quant_dequant(np.array([xr], np.float32))[0].tolist()
        acc = [0.0] * H
        for j, e in enumerate(order):
            Wg, Wu, Wd = Ws[e]
            I = len(Wg)
            h = []
            for i in range(I):
                g = sum(Wg[i][c] * xr[c] for c in range(H))
                u = sum(Wu[i][c] * xr[c] for c in range(H))
                h.append(g / (1 + math.exp(-g)) * u)
            if amode == "mxfp4":
                h = Q.quant_dequant(np.array([h], np.float32))[0].tolist()
            for o in range(H):
                acc[o] += float(np.float32(ws[j])) * sum(Wd[o][i] * h[i] for i in range(I))
        out.append(acc)
    return np.array(out)


@pytest.mark.parametrize("fmt,amode", [("bf16", "bf16"), ("mxfp4", "bf16"), ("nvfp4", "bf16"), ("mxfp4", "mxfp4")])
def test_tiny_layer_brute_force(fmt, amode):
    T, E, k, H, I = 3, 4, 2, 64, 32
    exs = [synth.expert(fmt, H, I, seed=7, config=97, expert_id=e) for e in range(E)]
    x = synth.activations(T, H, 7, 97, 1)
    logits = np.random.default_rng(4).standard_normal((T, E)).astype(np.float32)
    res = M.layer(x, exs, k, logits=logits, amode=amode)
    ref = _scalar_layer(x, exs, k, logits, amode)
    np.testing.assert_allclose(res["out"], ref, rtol=1e-9, atol=1e-14)


def test_combine_dense_formula_and_shared():
    rng = np.random.default_rng(9)
    T, k, H = 5, 3, 7
    y = rng.standard_normal((T * k, H))
    perm = rng.permutation(T * k).astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(T * k)
    w = rng.random((T, k)).astype(np.float32)
    sh = rng.standard_normal((T, H))
    out, bits = M.combine(y, inv, w, sh)
    for t in range(T):
        want = sum(float(w[t, j]) * y[inv[t * k + j]] for j in range(k)) + sh[t]
        np.testing.assert_allclose(out[t], want, rtol=1e-15)
    assert np.array_equal(bits, F.round_f32_to_bf16(out))


def test_token_output_matches_layer():
    L = synth.tiny_layer()
    res = M.layer(L["x"], L["experts"], L["k"], w_router=L["w_router"])
    Ws = {}

    def wts(e):
        if e not in Ws:
            Ws[e] = M.dequant_expert(L["experts"][e])
        return Ws[e]
    for t in (0, 7, 15):
        o = M.token_output(t, L["x"], res["ids"][t], res["w"][t], wts)
        np.testing.assert_allclose(o, res["out"][t], rtol=1e-12, atol=1e-16)


def test_router_logits_fp64():
    L = synth.tiny_layer()
    lg = M.router_logits(L["x"], L["w_router"])
    ref = (torch.from_numpy(F.bf16_to_f64(L["x"])) @ torch.from_numpy(L["w_router"]).double().T).numpy()
    np.testing.assert_allclose(lg, ref, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- batched evaluation

@pytest.mark.parametrize("fmt", synth.FMTS)
@pytest.mark.parametrize("amode", ["bf16", "mxfp4"])
def test_rows_together_equal_rows_one_by_one(fmt, amode):
    """expert_forward_rows (three matrix products over all rows) equals the
    per-row loop of expert_forward, which the dense-SwiGLU and scalar-loop
    pins above fix.  float64 products in a different summation order agree to
    rounding; in amode mxfp4 the float32 h they encode is identical here
    except where a product lands within that rounding of an E2M1 boundary."""
    if amode == "mxfp4" and fmt != "mxfp4":
        pytest.skip("MXFP4 activations go with MXFP4 weights")
    H, I, n = 256, 128, 23
    ex = synth.expert(fmt, H, I, seed=7, config=97, expert_id=0)
    x = synth.activations(n, H, 7, 97, 1)
    W = M.dequant_expert(ex)
    a = M.expert_forward(ex, x, amode)
    b = M.expert_forward_rows(x, W, amode)
    assert a.shape == b.shape == (n, H)
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12 * np.abs(a).max())


@pytest.mark.parametrize("fmt,amode,shared", [("nvfp4", "bf16", False), ("mxfp4", "mxfp4", True),
                                              ("bf16", "bf16", True)])
def test_grouped_layer_equals_the_per_token_layer(fmt, amode, shared):
    """layer_outputs (each expert's rows together, given the routing) equals
    layer() (the per-row loop) on the same routing, with a ragged row mix,
    an expert with no rows and a shared expert."""
    H, I, T, E, k = 128, 128, 19, 6, 2
    exs = [synth.expert(fmt, H, I, seed=8, config=96, expert_id=e) for e in range(E)]
    sh = synth.expert(fmt, H, I, seed=8, config=96, expert_id=synth.SHARED_EXPERT) if shared else None
    x = synth.activations(T, H, 8, 96, 1)
    logits = np.random.default_rng(3).standard_normal((T, E)).astype(np.float32)
    logits[:, 4] = -1e4
    ref = M.layer(x, exs, k, logits=logits, shared=sh, amode=amode)
    got = M.layer_outputs(x, ref["ids"], ref["w"], E, lambda e: M.dequant_expert(exs[e]),
                          shared_weights=M.dequant_expert(sh) if shared else None, amode=amode)
    np.testing.assert_allclose(got, ref["out"], rtol=0, atol=1e-12 * np.abs(ref["out"]).max())


# ---------------------------------------------------------------- the tolerance metric

def test_relative_error_hand_cases():
    """max |gpu - ref| / max |ref|, on values built by hand."""
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    # a known ratio: the largest difference 0.04 over the largest |ref| 4
    assert M.relative_error(ref + np.array([[0.0, 0.04], [-0.01, 0.0]]), ref) == pytest.approx(0.01, rel=1e-12)
    # the denominator is max |ref|, not max |gpu|: 18 / 2, not 18 / 20
    assert M.relative_error(np.array([1.0, 20.0]), np.array([1.0, 2.0])) == pytest.approx(9.0)
    # ... and not the signed maximum of ref (which is 1 here): 0.5 / 10
    assert M.relative_error(np.array([-10.0, 1.5]), np.array([-10.0, 1.0])) == pytest.approx(0.05)
    # the numerator is the largest absolute difference, whatever its sign
    assert M.relative_error(np.array([3.0, -1.0]), np.array([3.0, 2.0])) == pytest.approx(1.0)
    # identical arrays, and an all-zero reference
    assert M.relative_error(ref, ref) == 0.0
    assert M.relative_error(np.zeros(3), np.zeros(3)) == 0.0
    assert M.relative_error(np.array([0.0, 1e-3, 0.0]), np.zeros(3)) == math.inf
    # a NaN or inf anywhere in the GPU output fails any tolerance
    for bad in (math.nan, math.inf, -math.inf):
        assert not M.relative_error(np.array([1.0, bad]), np.array([1.0, 1.0])) <= 1e-2


def test_relative_error_refuses_broadcasting():
    ref = np.ones((3, 4))
    for shape in ((4,), (1, 4), (3, 1), (4, 3)):
        with pytest.raises(ValueError):
            M.relative_error(np.ones(shape), ref)
