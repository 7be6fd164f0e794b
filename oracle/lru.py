"""LRU expert-slot cache shared across MoE layers (plain simulation).

Pages: "FreeToken量子化：MoE推論のセットアップガイド", the paragraphs on the
two-tier expert memory hierarchy (host RAM holds every routed expert; free
VRAM is one variable expert cache shared by all MoE layers) and on decode (a
shared LRU over recently selected experts: a hit runs on the GPU, a miss is
brought in over PCIe); page on the bhrtaym blog, section "MoEバックエンドは
4種類から選べる", Table of backends, row ``offload`` (experts in host RAM, LRU
slots on the GPU, misses streamed over PCIe).

Readings where the pages are silent:
  * the key is (layer, expert);
  * per (token, layer) step the step's distinct experts are looked up in
    ascending id; every access (hit or miss) makes its key most recent;
  * a miss takes the lowest-numbered free slot, otherwise it evicts the least
    recently used key and reuses that key's slot;
  * a step may not look up more distinct experts than there are slots.

Resizing (page "FreeToken量子化：MoE推論のセットアップガイド", the paragraph
on resizing the expert cache at runtime at scheduler safe points; the pages
give no placement rule, so this is a reading):
  * the cache keeps the min(n, cached) most recently used keys and drops the
    rest, least recent first;
  * the kept keys move to a new set of n slots, packed from slot 0 in
    recency order (least recent in slot 0), their relative recency unchanged;
  * the slots above them are free, taken lowest first as before.
"""
from __future__ import annotations

from collections import OrderedDict


class CacheTooSmall(Exception):
    pass


class SlotLRU:
    def __init__(self, num_slots: int):
        self.num_slots = num_slots
        self._lru = OrderedDict()            # key -> slot, least recent first
        self._free = list(range(num_slots))  # ascending

    def __contains__(self, key):
        return key in self._lru

    def slot_of(self, key):
        return self._lru.get(key)

    def lookup(self, layer: int, ids):
        """Look up the distinct, ascending expert ids of one step of one layer.

        Returns one record per id: (expert, hit, slot, evicted_key or None)."""
        ids = list(ids)
        assert ids == sorted(set(ids)), "ids must be distinct and ascending"
        if len(ids) > self.num_slots:
            raise CacheTooSmall(f"{len(ids)} experts > {self.num_slots} slots")
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
                victim, slot = self._lru.popitem(last=False)
            self._lru[key] = slot
            out.append((e, False, slot, victim))
        return out

    def resize(self, num_slots: int):
        """Change the slot count; returns (moves, dropped): moves lists
        (key, old_slot, new_slot) in recency order, least recent first;
        dropped lists the keys no longer cached, least recent first."""
        assert num_slots > 0
        keys = list(self._lru.items())          # least recent first
        ndrop = max(0, len(keys) - num_slots)
        dropped = [k for k, _ in keys[:ndrop]]
        kept = keys[ndrop:]
        moves = [(k, old, new) for new, (k, old) in enumerate(kept)]
        self._lru = OrderedDict((k, new) for k, _, new in moves)
        self._free = list(range(len(kept), num_slots))
        self.num_slots = num_slots
        return moves, dropped
