"""Writes stream_trace_a3b_48x2048x512.txt: the oracle's expert-cache trace of
the cached decode stream at its real size (48 A3B-like layers of 128 experts,
top-8, 2048 slots shared under LRU, 512 single-token steps from a cold cache,
the stream's seeded routing), as a SHA-256 over its records plus totals.

Calls only the oracle (routing and LRU) and the seeded input generator.

Record encoding, per step in order (token t, then layer l): the int32 count
n of the step's distinct experts, then n records of four int32 (expert, hit
0/1, slot, evicted key or -1; key = layer * 128 + expert), little endian."""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

LAYERS, E, K, SLOTS, TOKENS = 48, 128, 8, 2048, 512
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stream_trace_a3b_48x2048x512.txt")


def oracle_trace():
    logits = synth.stream_routing(TOKENS, LAYERS, E)
    lru = oracle.lru.SlotLRU(SLOTS)
    h = hashlib.sha256()
    hits = misses = 0
    for t in range(TOKENS):
        ids, _ = oracle.moe.route(logits[t], K)          # [LAYERS, K]
        for l in range(LAYERS):
            recs = lru.lookup(l, sorted(set(ids[l].tolist())))
            arr = np.array([[e, int(hit), slot, -1 if ev is None else ev[0] * E + ev[1]]
                            for e, hit, slot, ev in recs], dtype="<i4")
            h.update(np.array([len(recs)], dtype="<i4").tobytes())
            h.update(arr.tobytes())
            hits += int(arr[:, 1].sum())
            misses += len(recs) - int(arr[:, 1].sum())
    return h.hexdigest(), hits, misses


def main():
    digest, hits, misses = oracle_trace()
    with open(OUT, "w") as f:
        f.write("# Expert-cache trace of the cached decode stream at its real size, computed by the oracle\n"
                "# (written by make_stream_trace.py; record encoding in its docstring).\n"
                "# 48 layers x 128 experts, top-8, 2048 LRU slots, 512 tokens, seed 0, cold start.\n")
        f.write(f"sha256 {digest}\nhits {hits}\nmisses {misses}\n")
    print(f"wrote {OUT}: {hits} hits, {misses} misses")


if __name__ == "__main__":
    main()
