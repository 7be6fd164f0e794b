"""Pins for the LRU expert-slot cache simulation."""
import numpy as np
import pytest

from oracle.lru import CacheTooSmall, SlotLRU


def test_textbook_trace(golden):
    c = SlotLRU(2)
    names = {}
    for r in golden("lru_textbook.txt"):
        step, key, hit, ev, slot = r.split()
        e = ord(key) - ord("A")
        names[e] = key
        (rec,) = c.lookup(0, [e])
        assert rec[1] == bool(int(hit)) and rec[2] == int(slot)
        assert (rec[3] is None and ev == "-") or (rec[3] == (0, ord(ev) - ord("A")))


class TimestampLRU:
    """Independent formulation: last-use timestamps, victim = argmin timestamp."""

    def __init__(self, C):
        self.C = C
        self.slot = {}
        self.ts = {}
        self.clock = 0

    def lookup(self, layer, ids):
        out = []
        for e in ids:
            key = (layer, e)
            self.clock += 1
            if key in self.slot:
                self.ts[key] = self.clock
                out.append((e, True, self.slot[key], None))
                continue
            used = set(self.slot.values())
            free = [s for s in range(self.C) if s not in used]
            if free:
                s, victim = free[0], None
            else:
                victim = min(self.ts, key=lambda q: self.ts[q])
                s = self.slot.pop(victim)
                del self.ts[victim]
            self.slot[key] = s
            self.ts[key] = self.clock
            out.append((e, False, s, victim))
        return out


def _random_steps(n, layers, E, per, seed):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=float) ** -1.1
    p /= p.sum()
    steps = []
    for _ in range(n):
        for l in range(layers):
            ids = sorted(set(rng.choice(E, per, replace=False, p=p).tolist()))
            steps.append((l, ids))
    return steps


@pytest.mark.parametrize("C", [4, 8, 13, 40])
def test_matches_timestamp_lru(C):
    steps = _random_steps(60, 3, 24, 4, C)
    a, b = SlotLRU(C), TimestampLRU(C)
    for l, ids in steps:
        assert a.lookup(l, ids) == b.lookup(l, ids)


def test_inclusion_property_and_compulsory_misses():
    steps = _random_steps(80, 2, 20, 3, 1)
    misses = []
    for C in range(3, 45):
        c = SlotLRU(C)
        misses.append(sum(not r[1] for l, ids in steps for r in c.lookup(l, ids)))
    assert all(a >= b for a, b in zip(misses, misses[1:]))
    distinct = len({(l, e) for l, ids in steps for e in ids})
    assert misses[-1] == distinct  # C >= #keys: only first touches miss


def test_step_larger_than_cache_rejected_and_state_unchanged():
    c = SlotLRU(2)
    c.lookup(0, [1])
    with pytest.raises(CacheTooSmall):
        c.lookup(0, [2, 3, 4])
    assert c.lookup(0, [1])[0][1] is True


def test_never_evicts_key_of_same_step():
    c = SlotLRU(3)
    c.lookup(0, [0, 1, 2])
    recs = c.lookup(1, [0, 1, 2])
    assert [r[3] for r in recs] == [(0, 0), (0, 1), (0, 2)]
    recs = c.lookup(0, [5, 6])  # victims must be (1,0),(1,1), never a key of this step
    assert [r[3] for r in recs] == [(1, 0), (1, 1)]


@pytest.mark.parametrize("C,n", [(12, 5), (5, 12), (9, 9), (20, 4)])
def test_resize_keeps_what_an_lru_of_the_new_size_would_hold(C, n):
    """Stack property of LRU: a cache of n slots that saw the whole history
    holds exactly the n most recent keys, in recency order.  So after
    resize(n) it holds what a fresh min(C, n)-slot cache run over the same
    history holds, and when shrinking (n <= C) the hit / miss sequence of
    later steps equals that of a fresh n-slot cache run over the whole
    history."""
    steps = _random_steps(90, 3, 16, 4, 2)
    first, second = steps[:50], steps[50:]
    a, b = SlotLRU(C), SlotLRU(min(C, n))
    for l, ids in first:
        a.lookup(l, ids)
        b.lookup(l, ids)
    before = [k for k in a._lru]
    moves, dropped = a.resize(n)
    assert dropped + [m[0] for m in moves] == before
    assert [m[0] for m in moves] == list(b._lru)          # same keys, same recency order
    assert [m[2] for m in moves] == list(range(len(moves)))
    for l, ids in second:
        ra, rb = a.lookup(l, ids), b.lookup(l, ids)
        if n <= C:
            assert [(r[0], r[1], r[3]) for r in ra] == [(r[0], r[1], r[3]) for r in rb]
        slots = list(a._lru.values())
        assert len(set(slots)) == len(slots) and all(0 <= s < n for s in slots)


def test_resize_then_misses_take_the_slots_above_the_kept_keys():
    c = SlotLRU(4)
    c.lookup(0, [1, 2, 3])       # slots 0, 1, 2
    c.lookup(1, [7])             # slot 3
    moves, dropped = c.resize(6)
    assert dropped == [] and [(m[0], m[2]) for m in moves] == [((0, 1), 0), ((0, 2), 1), ((0, 3), 2), ((1, 7), 3)]
    assert [r[2] for r in c.lookup(2, [0, 1])] == [4, 5]
    moves, dropped = c.resize(2)
    assert dropped == [(0, 1), (0, 2), (0, 3), (1, 7)] and [m[0] for m in moves] == [(2, 0), (2, 1)]


def test_stream_trace_golden_is_current():
    """The stored oracle trace of the real-size cached stream (used by the
    stream benchmark's trace verdict) equals the oracle's trace today."""
    import importlib.util
    import os
    from tests.conftest import GOLDEN
    spec = importlib.util.spec_from_file_location("mk", os.path.join(GOLDEN, "make_stream_trace.py"))
    mk = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mk)
    digest, hits, misses = mk.oracle_trace()
    with open(os.path.join(GOLDEN, "stream_trace_a3b_48x2048x512.txt")) as f:
        ref = dict(ln.split() for ln in f if ln.strip() and not ln.startswith("#"))
    assert ref["sha256"] == digest and int(ref["hits"]) == hits and int(ref["misses"]) == misses


def test_bench_trace_verdict_reads_the_oracle_encoding():
    """bench.py's stream trace verdict, fed the oracle's own records in the
    layout the library writes them (per step: expert, slot, hit, evicted-key
    rows), reports a match; one changed slot makes it report a mismatch."""
    import numpy as np
    import bench
    import oracle
    import synth
    L_, E, K, S, T = 48, 128, 8, 2048, 512
    logits = synth.stream_routing(T, L_, E)
    lru = oracle.lru.SlotLRU(S)
    NS = T * L_
    e, s, v = (np.zeros((NS, E), np.int32) for _ in range(3))
    h = np.zeros((NS, E), np.uint8)
    n = np.zeros(NS, np.int32)
    for t in range(T):
        ids, _ = oracle.moe.route(logits[t], K)
        for l in range(L_):
            i = t * L_ + l
            recs = lru.lookup(l, sorted(set(ids[l].tolist())))
            n[i] = len(recs)
            for j, (ex, hit, slot, ev) in enumerate(recs):
                e[i, j], h[i, j], s[i, j], v[i, j] = ex, int(hit), slot, -1 if ev is None else ev[0] * E + ev[1]
    assert bench.stream_trace_verdict(n, e, h, s, v, E, T, L_, S)["matches_oracle"] is True
    s[NS // 2, 0] += 1
    assert bench.stream_trace_verdict(n, e, h, s, v, E, T, L_, S)["matches_oracle"] is False
