"""The sparse MoE layer, step by step, as a plain CPU computation.

Pages: a routing network chooses a subset of the experts for every token at
every inference step (page "FreeToken qwen：ローカルQwen MoEセットアップガイド",
third paragraph); each token passes through only a few experts (page
"FreeToken量子化：MoE推論のセットアップガイド", second paragraph).  The pages
give no formula for the router or the expert; the steps below are the plain
definitions used by Qwen/DeepSeek-style MoE layers with a SwiGLU expert:

  logits  = x W_r^T                                   (router_logits)
  ids     = the k largest logits of each row           (route)
  w       = softmax over the k selected logits          (route)
  perm    = (t, j) pairs sorted stably by expert id     (permute)
  y       = W_down (silu(W_gate x) * (W_up x))          (expert_forward)
  out[t]  = sum_j w[t,j] y[t,j] (+ shared expert(x_t))  (combine)

Readings of what the pages leave open (each is listed with its reason in the
design notes): selection on the float32 logit with ties to the lower expert
id and NaN below -inf; ids of a row ordered by descending logit; softmax
restricted to the selected logits (equal to the full softmax renormalised);
within an expert, rows in ascending flat index t*k + j; the shared expert has
weight 1 and is added after the routed sum; the output is rounded to bf16.
"""
from __future__ import annotations

import math

import numpy as np

from .formats import bf16_to_f64, dequant, round_f32_to_bf16
from .quant import dequantize_mxfp4_codes, quant_dequant, quantize_mxfp4_rows


def router_logits(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * W_r[e, h], float64 (x bf16, W_r float32)."""
    return bf16_to_f64(x_bits) @ np.asarray(w_router, dtype=np.float32).astype(np.float64).T


def _rank_key(v: float, e: int):
    # larger logit first; NaN below everything (including -inf); ties -> lower id
    return (1, 0.0, e) if math.isnan(v) else (0, -v, e)


def topk_ids(logits: np.ndarray, k: int) -> np.ndarray:
    """Per row, the ids of the k largest float32 logits, in rank order."""
    lf = np.asarray(logits, dtype=np.float32)
    T, E = lf.shape
    ids = np.empty((T, k), np.int32)
    for t in range(T):
        row = [float(v) for v in lf[t]]
        order = sorted(range(E), key=lambda e: _rank_key(row[e], e))
        ids[t] = order[:k]
    return ids


def _unnormalised(vals, m):
    # exp(v - m) with the conventions: v == m -> 1 (covers +-inf maxima), NaN -> 0
    out = []
    for v in vals:
        if math.isnan(v):
            out.append(0.0)
        elif v == m:
            out.append(1.0)
        else:
            out.append(math.exp(v - m))
    return out


def route(logits: np.ndarray, k: int, renormalize: bool = True):
    """Top-k routing.  Returns (ids int32 [T,k], weights float32 [T,k]).

    renormalize=True: w_j = exp(l_j - m) / sum_{i in top-k} exp(l_i - m), which
    equals softmax over all experts renormalised over the selected ones.
    renormalize=False: w_j = softmax over all E experts, evaluated at the
    selected ids.  A row whose selected logits are all NaN gets weights 1/k."""
    lf = np.asarray(logits, dtype=np.float32)
    ids = topk_ids(lf, k)
    T, E = lf.shape
    w = np.empty((T, k), np.float32)
    for t in range(T):
        row = [float(v) for v in lf[t]]
        sel = [row[e] for e in ids[t]]
        m = sel[0]
        num = _unnormalised(sel, m)
        den = sum(num) if renormalize else sum(_unnormalised(row, m))
        if den == 0.0:
            w[t] = 1.0 / k
        else:
            w[t] = [n / den for n in num]
    return ids, w


def permute(ids: np.ndarray, E: int):
    """Stable counting sort of the flat pairs f = t*k + j by expert id.

    Returns counts [E], offsets [E+1] (exclusive scan), perm [T*k] (perm[p] =
    flat index at sorted position p) and inv [T*k] (inv[perm[p]] = p)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    n = flat.size
    perm = np.array(sorted(range(n), key=lambda f: (int(flat[f]), f)), dtype=np.int32).reshape(n)
    counts = np.zeros(E, np.int32)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    inv = np.empty(n, np.int32)
    inv[perm] = np.arange(n, dtype=np.int32)
    return counts, offsets, perm, inv


def silu(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def dequant_expert(ex):
    """(W_gate [I,H], W_up [I,H], W_down [H,I]) in float64."""
    return dequant(ex.gate, ex.fmt), dequant(ex.up, ex.fmt), dequant(ex.down, ex.fmt)


def expert_forward(ex, x_rows_bits: np.ndarray, amode: str = "bf16", weights=None) -> np.ndarray:
    """SwiGLU expert applied to each row of x (bf16 bits [n, H]); returns y [n, H] float64.

    amode "bf16": x is used as given and h stays float64.
    amode "mxfp4": x is MXFP4-encoded per row (blocks of 32 along H) and h,
    rounded to float32, is MXFP4-encoded per row (blocks of 32 along I) before
    the down projection — the activation precision of the FP4 x FP4 MFMA path."""
    Wg, Wu, Wd = weights if weights is not None else dequant_expert(ex)
    X = bf16_to_f64(np.asarray(x_rows_bits).reshape(-1, Wg.shape[1]))
    if amode == "mxfp4":
        X = quant_dequant(X.astype(np.float32))
    Y = np.empty((X.shape[0], Wd.shape[0]), np.float64)
    for r in range(X.shape[0]):
        x = X[r]
        h = silu(Wg @ x) * (Wu @ x)
        if amode == "mxfp4":
            h = quant_dequant(h.astype(np.float32)[None, :])[0]
        Y[r] = Wd @ h
    return Y


def combine(y_perm: np.ndarray, inv: np.ndarray, w: np.ndarray, y_shared=None):
    """out[t] = sum_{j ascending} w[t,j] * y_perm[inv[t*k+j]] (+ y_shared[t]).

    Returns (float64 [T,H], bf16 bits [T,H])."""
    T, k = w.shape
    H = y_perm.shape[1]
    out = np.zeros((T, H), np.float64)
    for t in range(T):
        for j in range(k):
            out[t] += float(w[t, j]) * y_perm[inv[t * k + j]]
        if y_shared is not None:
            out[t] += y_shared[t]
    return out, round_f32_to_bf16(out)


def layer(x_bits: np.ndarray, experts, k: int, *, logits=None, w_router=None, renormalize=True,
          shared=None, amode="bf16"):
    """One full MoE layer call.  Exactly one of logits / w_router is given.

    Returns a dict with logits, ids, w, counts, offsets, perm, inv, y_perm,
    y_shared, out (float64) and out_bf16."""
    T = x_bits.shape[0]
    E = len(experts)
    if logits is None:
        logits = router_logits(x_bits, w_router).astype(np.float32)
    ids, w = route(logits, k, renormalize)
    counts, offsets, perm, inv = permute(ids, E)
    H = x_bits.shape[1]
    y_perm = np.zeros((T * k, H), np.float64)
    for e in range(E):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        toks = perm[lo:hi] // k
        y_perm[lo:hi] = expert_forward(experts[e], x_bits[toks], amode)
    y_shared = expert_forward(shared, x_bits, amode) if shared is not None else None
    out, out_bf16 = combine(y_perm, inv, w, y_shared)
    return dict(logits=np.asarray(logits, np.float32), ids=ids, w=w, counts=counts, offsets=offsets,
                perm=perm, inv=inv, y_perm=y_perm, y_shared=y_shared, out=out, out_bf16=out_bf16)


def expert_forward_rows(x_rows_bits: np.ndarray, weights, amode: str = "bf16", h_codes=None) -> np.ndarray:
    """The SwiGLU expert of ``expert_forward`` with its n rows stacked into one
    matrix: Y = (silu(X W_gate^T) * (X W_up^T)) W_down^T in float64, X [n, H]
    (bf16 bits), the same definition evaluated as three matrix products.
    amode "mxfp4" encodes X, and H rounded to float32, per row as
    ``expert_forward`` does; then, if h_codes is a list, the encoding of H
    (E2M1 codes [n, I], E8M0 codes [n, I/32]) is appended to it."""
    Wg, Wu, Wd = weights
    X = bf16_to_f64(np.asarray(x_rows_bits).reshape(-1, Wg.shape[1]))
    if amode == "mxfp4":
        X = quant_dequant(X.astype(np.float32))
    Hm = silu(X @ Wg.T) * (X @ Wu.T)
    if amode == "mxfp4":
        codes, scales = quantize_mxfp4_rows(Hm.astype(np.float32))
        if h_codes is not None:
            h_codes.append((codes, scales))
        Hm = dequantize_mxfp4_codes(codes, scales)
    return Hm @ Wd.T


def layer_outputs(x_bits: np.ndarray, ids: np.ndarray, w: np.ndarray, E: int, expert_weights, *,
                  shared_weights=None, amode: str = "bf16", h_codes=None) -> np.ndarray:
    """out (float64 [T, H]) of one layer call given its routing (ids, w [T, k]):
    the rows of each expert (the permutation of ``permute``) evaluated together
    by ``expert_forward_rows``, then ``combine``.  expert_weights(e) returns the
    dequantised (W_gate, W_up, W_down) of expert e; each is asked for once, in
    ascending e.  With amode "mxfp4" and h_codes a dict, h_codes["codes"] and
    h_codes["scales"] receive the encoding of every row's SwiGLU output in
    permutation order (shared expert's token rows last)."""
    T, k = ids.shape
    H = x_bits.shape[1]
    counts, offsets, perm, inv = permute(ids, E)
    y_perm = np.zeros((T * k, H), np.float64)
    hc = [] if (h_codes is not None and amode == "mxfp4") else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_perm[lo:hi] = expert_forward_rows(x_bits[perm[lo:hi] // k], expert_weights(e), amode, hc)
    y_shared = None
    if shared_weights is not None:
        y_shared = expert_forward_rows(x_bits, shared_weights, amode, hc)
    if hc is not None:
        h_codes["codes"] = np.concatenate([c for c, _ in hc])
        h_codes["scales"] = np.concatenate([sc for _, sc in hc])
    return combine(y_perm, inv, w, y_shared)[0]


def token_output(t: int, x_bits: np.ndarray, ids_row, w_row, expert_weights, *, shared_weights=None,
                 amode="bf16") -> np.ndarray:
    """out[t] alone (float64 [H]): for sampled-output checks at full size.

    expert_weights(e) returns the dequantised (W_gate, W_up, W_down) of expert e."""
    x = x_bits[t:t + 1]
    acc = np.zeros(x_bits.shape[1], np.float64)
    for j, e in enumerate(ids_row):
        acc += float(w_row[j]) * expert_forward(None, x, amode, weights=expert_weights(int(e)))[0]
    if shared_weights is not None:
        acc += expert_forward(None, x, amode, weights=shared_weights)[0]
    return acc


def relative_error(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| over the whole output, in float64.

    The two arrays must have the same shape (no broadcasting).  A non-finite
    value in gpu gives inf; a reference that is all zeros gives 0 when gpu is
    all zeros too, else inf."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape {g.shape} != reference shape {r.shape}")
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return math.inf
    num = float(np.max(np.abs(g - r)))
    den = float(np.max(np.abs(r)))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den
