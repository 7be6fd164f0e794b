"""Pins for routing (top-k + softmax) and the permutation."""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import moe as M


def _parse(tok):
    return float(tok)  # handles inf / -inf / nan


def test_hand_built_tie_rows(golden):
    for r in golden("route_ties.txt"):
        k, vals, want = [p.strip() for p in r.split("|")]
        row = np.array([[_parse(v) for v in vals.split(",")]], np.float32)
        ids, w = M.route(row, int(k))
        assert ids[0].tolist() == [int(v) for v in want.split(",")], r
        assert abs(float(w[0].sum()) - 1.0) < 1e-6


def _key(v, e):
    # larger key = ranks higher: (not NaN, value, -id)
    return (0, 0.0, -e) if math.isnan(v) else (1, v, -e)


def _brute_topk(row, k):
    E = len(row)
    valid = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if not rest or min(_key(row[e], e) for e in S) > max(_key(row[e], e) for e in rest):
            valid.append(S)
    assert len(valid) == 1
    return sorted(valid[0], key=lambda e: _key(row[e], e), reverse=True)


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (8, 2), (8, 4), (8, 8)])
def test_topk_brute_force_over_all_subsets(E, k):
    rng = np.random.default_rng(E * 10 + k)
    for trial in range(40):
        # few distinct values so that ties are common
        row = rng.integers(-2, 3, E).astype(np.float32) / 2
        if trial % 5 == 0:
            row[rng.integers(0, E)] = np.nan
        if trial % 7 == 0:
            row[rng.integers(0, E)] = -np.inf
        ids, _ = M.route(row[None, :], k)
        assert ids[0].tolist() == _brute_topk([float(v) for v in row], k)


def test_weights_equal_renormalised_full_softmax():
    rng = np.random.default_rng(1)
    logits = (rng.standard_normal((50, 16)) * 3).astype(np.float32)
    ids, w = M.route(logits, 4)
    full = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    for t in range(50):
        p = full[t, ids[t]]
        np.testing.assert_allclose(w[t], p / p.sum(), rtol=2e-7, atol=0)
        assert abs(float(w[t].astype(np.float64).sum()) - 1) <= 4 * 2 ** -24
        assert np.all(np.diff(logits[t, ids[t]]) <= 0)  # descending
    # k = E: weights are the full softmax
    ids, w = M.route(logits, 16)
    np.testing.assert_allclose(np.take_along_axis(full, ids, 1), w, rtol=2e-7)
    # renormalize = False: the full softmax at the selected ids
    ids, w = M.route(logits, 4, renormalize=False)
    np.testing.assert_allclose(np.take_along_axis(full, ids, 1), w, rtol=2e-7)


def _brute_permute(ids, E):
    flat = ids.ravel().tolist()
    pairs = sorted((e, f) for f, e in enumerate(flat))
    perm = [f for _, f in pairs]
    counts = [flat.count(e) for e in range(E)]
    return counts, perm


def test_permute_brute_force_and_invariants():
    rng = np.random.default_rng(2)
    for T, k, E in [(1, 1, 1), (3, 2, 4), (16, 2, 8), (7, 8, 128), (40, 8, 16)]:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        counts, offsets, perm, inv = M.permute(ids, E)
        bc, bp = _brute_permute(ids, E)
        assert counts.tolist() == bc and perm.tolist() == bp
        assert offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(perm[inv], np.arange(T * k)) and np.array_equal(inv[perm], np.arange(T * k))
        # gather rows by perm, then unpermute by inv: identity (bit-exact copies)
        rows = rng.standard_normal((T * k, 5)).astype(np.float32)
        assert np.array_equal(rows[perm][inv], rows)
        # each expert's rows are consecutive and in ascending flat index
        flat = ids.ravel()
        for e in range(E):
            seg = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
