"""Pins for the oracle's expert-cache simulation (no GPU).

The oracle keeps per-slot recency stamps.  Two independently written models
check it: a textbook OrderedDict LRU (for calls whose unique set fits), and a
recency-list simulator (slots kept in least-to-most-recent order, empty slots
first by index) that realises the pin/bypass rule a different way.
"""
import itertools
from collections import OrderedDict

import numpy as np
import pytest

from oracle.cache import SlotCache


class RecencyListCache:
    """Second model: an explicit list of slots from least to most recent."""

    def __init__(self, C, E):
        self.E = E
        self.owner = [None] * C          # key held by each slot
        self.order = list(range(C))      # empty slots first, ascending index

    def lookup(self, layer, experts):
        keys = [layer * self.E + e for e in experts]
        where = {k: s for s, k in enumerate(self.owner) if k is not None}
        hit_slots = [where[k] for k in keys if k in where]
        miss_keys = [k for k in keys if k not in where]
        free = [s for s in self.order if s not in hit_slots]
        res = {}
        filled = []
        for r, k in enumerate(miss_keys):
            if r < len(free):
                s = free[r]
                self.owner[s] = k
                filled.append(s)
                res[k] = s
            else:
                res[k] = -1 - (r - len(free))
        for k in keys:
            if k in where:
                res[k] = where[k]
        touched = set(hit_slots) | set(filled)
        self.order = [s for s in self.order if s not in touched] + hit_slots + filled
        return [res[k] for k in keys]


def _state_keys(c):
    return {k: s for s, k in enumerate(c.key) if k >= 0}


def _check_invariants(c: SlotCache, n_call, before_hits, before_fills, before_byp):
    occ = [k for k in c.key if k >= 0]
    assert len(occ) == len(set(occ))            # key <-> slot bijection
    assert len(occ) <= c.capacity
    stamps = [c.stamp[s] for s in range(c.capacity) if c.key[s] >= 0]
    assert len(stamps) == len(set(stamps)) and all(st > 0 for st in stamps)
    assert all(c.stamp[s] == 0 for s in range(c.capacity) if c.key[s] < 0)
    assert (c.hits - before_hits) + (c.fills - before_fills) + (c.bypasses - before_byp) == n_call


def test_matches_textbook_lru_when_unique_set_fits():
    rng = np.random.default_rng(0)
    for trial in range(40):
        E, L = 16, 2
        C = int(rng.integers(1, 12))
        c = SlotCache(C, E)
        lru = OrderedDict()
        for _ in range(60):
            layer = int(rng.integers(0, L))
            n = int(rng.integers(1, C + 1))
            U = sorted(rng.choice(E, n, replace=False).tolist())
            slots, fills, bypass = c.lookup(layer, U)
            assert not bypass
            # textbook LRU on the same access sequence: hits first, then misses,
            # each in ascending expert order
            keys = [layer * E + e for e in U]
            hits = [k for k in keys if k in lru]
            misses = [k for k in keys if k not in lru]
            for k in hits:
                lru.move_to_end(k)
            for k in misses:
                if len(lru) >= C:
                    lru.popitem(last=False)
                lru[k] = True
            assert set(_state_keys(c)) == set(lru)
            by_recency = sorted(_state_keys(c), key=lambda k: c.stamp[_state_keys(c)[k]])
            assert by_recency == list(lru)
            for i, k in enumerate(keys):
                assert c.key[slots[i]] == k


@pytest.mark.parametrize("E,L,C,calls", [(3, 1, 0, 5), (3, 1, 1, 5), (3, 1, 2, 5), (3, 1, 3, 5),
                                         (2, 2, 2, 4), (2, 2, 3, 4), (4, 1, 2, 3), (4, 1, 3, 3)])
def test_brute_force_against_recency_list(E, L, C, calls):
    subsets = [s for r in range(1, E + 1) for s in itertools.combinations(range(E), r)]
    calls_space = [(l, s) for l in range(L) for s in subsets]
    for trace in itertools.product(calls_space, repeat=calls):
        a = SlotCache(C, E)
        b = RecencyListCache(C, E)
        for layer, U in trace:
            h0, f0, b0 = a.hits, a.fills, a.bypasses
            before = dict(_state_keys(a))
            sa, fills, byp = a.lookup(layer, list(U))
            sb = b.lookup(layer, list(U))
            assert sa == sb, (trace, layer, U)
            assert [k for k in a.key] == [k if k is not None else -1 for k in b.owner]
            _check_invariants(a, len(U), h0, f0, b0)
            # hits keep their slots; nothing hit in this call is evicted
            for e, s in zip(U, sa):
                k = layer * E + e
                if k in before:
                    assert s == before[k]
            # fills land in distinct slots; bypass only when no victim is left
            assert len({f[0] for f in fills}) == len(fills)
            if byp:
                assert len(fills) + (len(U) - len(fills) - len(byp)) == C


def test_bypass_when_unique_set_exceeds_capacity():
    c = SlotCache(2, 8)
    slots, fills, byp = c.lookup(0, [1, 3, 5, 7])
    assert slots == [0, 1, -1, -2] and len(fills) == 2 and len(byp) == 2
    # a second call pins its hit (expert 3) and takes the other slot for 6
    slots, fills, byp = c.lookup(0, [3, 6])
    assert slots == [1, 0] and fills == [(0, 0, 6)]


def test_resize_invariants():
    rng = np.random.default_rng(5)
    E = 32
    for trial in range(30):
        C = int(rng.integers(2, 20))
        c = SlotCache(C, E)
        for _ in range(int(rng.integers(1, 30))):
            U = sorted(rng.choice(E, int(rng.integers(1, C + 1)), replace=False).tolist())
            c.lookup(int(rng.integers(0, 2)), U)
        key0, stamp0, clock0 = c.snapshot()
        occ = {k: st for k, st in zip(key0, stamp0) if k >= 0}
        newC = int(rng.integers(0, C + 5))
        moves, evicted = c.resize(newC)
        key1, stamp1, clock1 = c.snapshot()
        assert clock1 == clock0 and len(key1) == newC
        after = {k: st for k, st in zip(key1, stamp1) if k >= 0}
        if newC >= len(occ):
            assert after == occ and not evicted           # only slot numbers change
        else:
            assert len(after) == newC
            keep = sorted(occ, key=lambda k: occ[k])[len(occ) - newC:]
            assert set(after) == set(keep)                 # the most recent survive
            assert all(after[k] == occ[k] for k in after)
        if newC >= C:
            assert key1[:C] == key0 and not moves          # grow: state unchanged
        for s, d in moves:
            assert s >= newC and d < newC


def test_resize_to_zero_empties():
    c = SlotCache(4, 8)
    c.lookup(0, [1, 2, 3])
    moves, evicted = c.resize(0)
    assert c.capacity == 0 and sorted(evicted) == [1, 2, 3] and not moves
    slots, fills, byp = c.lookup(0, [4])
    assert slots == [-1] and not fills
