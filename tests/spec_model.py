"""A second, independently written model of the cache policy, used to pin the oracle.

The oracle keeps integer recency stamps (2t+1 for a miss fetched at step t,
2t+2 for a hit).  This model keeps no stamps at all: it keeps the slots in
an ordered list of recency groups, oldest group first.  Initially there is
one group holding every (empty) slot.  After each resolve, the slots that
received a miss form a new group, and the slots that hit form a newer group
after it -- "hits promoted above newly fetched misses" (pith review, "What
carries the argument").  Victims are taken from the oldest groups; inside a
group the lowest slot goes first.  If the stamp encoding in the oracle were
wrong (signs, offsets, or a swapped hit/miss order), the two models would
diverge on some short sequence, which the brute-force test enumerates.
"""
from __future__ import annotations


class RecencyListModel:
    def __init__(self, B: int):
        self.B = B
        self.slots = [None] * B          # position held by each slot
        self.groups = [set(range(B))]    # recency groups, oldest first

    def resident(self):
        return {p for p in self.slots if p is not None}

    def resolve(self, S):
        k = len(S)
        if k > self.B or len(set(S)) != k:
            raise ValueError("bad selection")
        where = {p: j for j, p in enumerate(S)}
        slot_idx = [None] * k
        hit_slots = set()
        for s, p in enumerate(self.slots):
            if p is not None and p in where:
                slot_idx[where[p]] = s
                hit_slots.add(s)
        misses = [j for j in range(k) if slot_idx[j] is None]
        victims = []
        for g in self.groups:
            if len(victims) == len(misses):
                break
            free = sorted(s for s in g if s not in hit_slots)
            victims.extend(free[: len(misses) - len(victims)])
        assert len(victims) == len(misses)
        victims.sort()
        plan = []
        for j, v in zip(misses, victims):
            plan.append((j, v, -1 if self.slots[v] is None else self.slots[v], S[j]))
            self.slots[v] = S[j]
            slot_idx[j] = v
        touched = set(victims) | hit_slots
        self.groups = [g - touched for g in self.groups]
        self.groups = [g for g in self.groups if g]
        if victims:
            self.groups.append(set(victims))
        if hit_slots:
            self.groups.append(set(hit_slots))
        hit_mask = [1 if j not in misses else 0 for j in range(k)]
        return slot_idx, hit_mask, plan
