"""Planted mistakes in the oracle (on the CPU) must each fail one of its pins.

Each case swaps one oracle piece for a plausible wrong version, runs the pin
that should catch it, and expects that pin to fail."""
import math
from collections import OrderedDict

import numpy as np
import pytest

import oracle.formats as F
import oracle.lru as LRU
import oracle.moe as M
import oracle.quant as Q
import tests.test_oracle_ffn as tffn
import tests.test_oracle_formats as tfmt
import tests.test_oracle_lru as tlru
import tests.test_oracle_quant as tq
import tests.test_oracle_route as troute
from tests.conftest import golden_rows


def _fails(fn, *a):
    with pytest.raises(AssertionError):
        fn(*a)


def test_swapped_nibbles_caught(monkeypatch):
    def bad(q):
        q = np.asarray(q, np.uint8)
        c = np.empty((q.shape[0], q.shape[1] * 2), np.uint8)
        c[:, 0::2], c[:, 1::2] = q >> 4, q & 15
        return c
    monkeypatch.setattr(F, "unpack_e2m1", bad)
    _fails(tfmt.test_nibble_order_low_first)


def test_e8m0_bias_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(F, "E8M0", np.array([2.0 ** (c - 128) for c in range(255)] + [math.nan]))
    _fails(tfmt.test_e8m0_matches_torch_exhaustive)


def test_wrong_silu_sign_caught(monkeypatch):
    monkeypatch.setattr(M, "silu", lambda z: z / (1.0 + np.exp(z)))
    _fails(tffn.test_one_expert_top1_is_dense_swiglu, "mxfp4")


def test_gate_up_swapped_caught(monkeypatch):
    orig = M.dequant_expert
    monkeypatch.setattr(M, "dequant_expert", lambda ex: (lambda g, u, d: (u, g, d))(*orig(ex)))
    _fails(tffn.test_one_expert_top1_is_dense_swiglu, "bf16")


def test_ties_to_higher_id_caught(monkeypatch):
    monkeypatch.setattr(M, "_rank_key", lambda v, e: (1, 0.0, -e) if math.isnan(v) else (0, -v, -e))
    _fails(troute.test_hand_built_tie_rows, golden_rows)


def test_softmax_without_max_shift_but_over_all_experts_caught(monkeypatch):
    orig = M.route

    def bad(logits, k, renormalize=True):
        return orig(logits, k, renormalize=False)
    monkeypatch.setattr(M, "route", bad)
    _fails(troute.test_weights_equal_renormalised_full_softmax)


def test_unstable_permute_caught(monkeypatch):
    def bad(ids, E):
        flat = np.asarray(ids).ravel()
        perm = np.array(sorted(range(flat.size), key=lambda f: (int(flat[f]), -f)), np.int32)
        counts = np.bincount(flat, minlength=E).astype(np.int32)
        off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        inv = np.empty_like(perm)
        inv[perm] = np.arange(flat.size)
        return counts, off, perm, inv
    monkeypatch.setattr(M, "permute", bad)
    _fails(troute.test_permute_brute_force_and_invariants)


def test_combine_with_perm_instead_of_inv_caught(monkeypatch):
    orig = M.combine

    def bad(y, inv, w, sh=None):
        perm = np.empty_like(inv)
        perm[inv] = np.arange(inv.size)
        return orig(y, perm, w, sh)
    monkeypatch.setattr(M, "combine", bad)
    _fails(tffn.test_combine_dense_formula_and_shared)


def test_quantiser_ties_away_from_zero_caught(monkeypatch):
    def bad(q):
        sign = 8 if math.copysign(1.0, q) < 0 else 0
        d = np.abs(Q._GRID - abs(q))
        cands = [c for c in range(8) if d[c] == d.min()]
        return sign | cands[-1]
    monkeypatch.setattr(Q, "_nearest_e2m1", bad)
    _fails(tq.test_hand_built_rounding_cases, golden_rows)


def test_lru_evicting_most_recent_caught(monkeypatch):
    def bad_lookup(self, layer, ids):
        out = []
        for e in ids:
            key = (layer, e)
            if key in self._lru:
                self._lru.move_to_end(key)
                out.append((e, True, self._lru[key], None))
                continue
            if self._free:
                slot, victim = self._free.pop(0), None
            else:
                victim, slot = self._lru.popitem(last=True)
            self._lru[key] = slot
            out.append((e, False, slot, victim))
        return out
    monkeypatch.setattr(LRU.SlotLRU, "lookup", bad_lookup)
    _fails(tlru.test_textbook_trace, golden_rows)


def test_metric_dividing_by_max_gpu_caught(monkeypatch):
    def bad(gpu, ref):
        g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
        return float(np.max(np.abs(g - r)) / np.max(np.abs(g)))
    monkeypatch.setattr(M, "relative_error", bad)
    _fails(tffn.test_relative_error_hand_cases)


def test_metric_dividing_by_signed_max_caught(monkeypatch):
    def bad(gpu, ref):
        g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
        return float(np.max(np.abs(g - r)) / np.max(r))
    monkeypatch.setattr(M, "relative_error", bad)
    _fails(tffn.test_relative_error_hand_cases)


def test_metric_broadcasting_caught(monkeypatch):
    def bad(gpu, ref):
        g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
        return float(np.max(np.abs(g - r)) / np.max(np.abs(r)))
    monkeypatch.setattr(M, "relative_error", bad)
    with pytest.raises(pytest.fail.Exception, match="DID NOT RAISE"):
        tffn.test_relative_error_refuses_broadcasting()


def test_batched_expert_with_gate_and_up_swapped_caught(monkeypatch):
    orig = M.expert_forward_rows
    monkeypatch.setattr(M, "expert_forward_rows", lambda x, w, amode="bf16": orig(x, (w[1], w[0], w[2]), amode))
    _fails(tffn.test_rows_together_equal_rows_one_by_one, "mxfp4", "bf16")


def test_grouped_layer_with_rows_off_by_one_expert_caught(monkeypatch):
    orig_perm = M.permute

    def bad(ids, E):
        counts, offsets, perm, inv = orig_perm(ids, E)
        return counts, offsets, np.roll(perm, 1), inv
    orig_layer_outputs = M.layer_outputs

    def layer_outputs(*a, **kw):
        monkeypatch.setattr(M, "permute", bad)
        try:
            return orig_layer_outputs(*a, **kw)
        finally:
            monkeypatch.setattr(M, "permute", orig_perm)
    monkeypatch.setattr(M, "layer_outputs", layer_outputs)
    _fails(tffn.test_grouped_layer_equals_the_per_token_layer, "nvfp4", "bf16", False)
