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


def _with_state(C, E, key, stamp, clock):
    c = SlotCache(C, E)
    c.key, c.stamp, c.clock = list(key), list(stamp), clock
    return c


def test_resize_hand_computed_slot_numbering():
    """Six slots holding keys in slots 1, 3, 4, 5 (stamps 4, 2, 9, 7), shrunk
    to three: the least recent key (13, stamp 2) is evicted, the survivors
    in slots 4 and 5 move to the free slots 0 and 2 in that order, and slot
    1 keeps its key.  Worked out by hand from the rule."""
    c = _with_state(6, 10, [-1, 11, -1, 13, 14, 15], [0, 4, 0, 2, 9, 7], 9)
    moves, evicted = c.resize(3)
    assert c.key == [14, 11, 15] and c.stamp == [9, 4, 7] and c.clock == 9
    assert moves == [(4, 0), (5, 2)] and evicted == [13]
    # no eviction, survivors fill the holes in ascending order
    c = _with_state(5, 10, [7, -1, -1, 8, 9], [3, 0, 0, 1, 2], 3)
    moves, evicted = c.resize(3)
    assert c.key == [7, 8, 9] and c.stamp == [3, 1, 2] and not evicted
    assert moves == [(3, 1), (4, 2)]
    # several evictions, all among the tail; the head is left alone
    c = _with_state(6, 10, [1, 2, 3, 4, 5, 6], [6, 5, 4, 3, 2, 1], 6)
    moves, evicted = c.resize(2)
    assert c.key == [1, 2] and c.stamp == [6, 5] and not moves
    assert evicted == [6, 5, 4, 3]


def _resize_by_ranks(key, stamp, new_C):
    """A second resize model: rank the occupied slots by recency, keep the
    new_C most recent, then pair the kept slots at or past new_C (ascending)
    with the empty slots below new_C (ascending) by position."""
    occupied = [s for s in range(len(key)) if key[s] >= 0]
    keep = set(sorted(occupied, key=lambda s: -stamp[s])[:new_C])
    out_key = [key[s] if s in keep else -1 for s in range(new_C)]
    out_stamp = [stamp[s] if s in keep else 0 for s in range(new_C)]
    movers = sorted(s for s in keep if s >= new_C)
    holes = [d for d in range(new_C) if out_key[d] < 0]
    for s, d in zip(movers, holes):
        out_key[d], out_stamp[d] = key[s], stamp[s]
    return out_key, out_stamp, list(zip(movers, holes))


@pytest.mark.parametrize("E,C,calls", [(4, 3, 3), (3, 4, 3), (5, 4, 2)])
def test_resize_brute_force_against_rank_model(E, C, calls):
    """Every trace of lookups over all subsets, then every shrink and grow
    target: the oracle's resize equals the rank model, and later lookups
    keep agreeing with the recency-list simulator (recency is preserved)."""
    subsets = [s for r in range(1, E + 1) for s in itertools.combinations(range(E), r)]
    for trace in itertools.product(subsets, repeat=calls):
        base = SlotCache(C, E)
        for U in trace:
            base.lookup(0, list(U))
        for new_C in range(0, C + 2):
            c = _with_state(C, E, base.key, base.stamp, base.clock)
            want_key, want_stamp, want_moves = _resize_by_ranks(base.key, base.stamp, new_C)
            moves, evicted = c.resize(new_C)
            if new_C >= C:
                want_key = base.key + [-1] * (new_C - C)
                want_stamp = base.stamp + [0] * (new_C - C)
                want_moves = []
            assert c.key == want_key and c.stamp == want_stamp, (trace, new_C)
            assert moves == want_moves and c.clock == base.clock
            # a lookup after the resize: the recency-list model rebuilt from
            # the resized state (empty slots by index, then by stamp) agrees
            r = RecencyListCache(new_C, E)
            r.owner = [k if k >= 0 else None for k in c.key]
            r.order = sorted(range(new_C), key=lambda s: (c.key[s] >= 0, c.stamp[s], s))
            for U in subsets[:: max(1, len(subsets) // 4)]:
                assert c.lookup(0, list(U))[0] == r.lookup(0, list(U))


def test_reset_is_a_fresh_cache_at_the_same_clock():
    """After reset the state equals a new cache whose clock was advanced to
    the old clock, and every later lookup sequence behaves the same in both
    (brute force over short traces of a tiny cache)."""
    import itertools
    from oracle import SlotCache
    E, C = 4, 3
    traces = list(itertools.product([(0,), (1,), (0, 2), (1, 3), (0, 1, 2, 3)], repeat=3))
    for pre in traces[:40]:
        for post in traces[::7]:
            a = SlotCache(C, E)
            for u in pre:
                a.lookup(0, list(u))
            clock = a.clock
            n_res = sum(1 for k in a.key if k >= 0)
            assert a.reset() == n_res
            b = SlotCache(C, E)
            b.clock = clock
            assert a.snapshot() == b.snapshot()
            for u in post:
                assert a.lookup(0, list(u)) == b.lookup(0, list(u))
                assert a.snapshot() == b.snapshot()


# ------------------------------------------------------------------ prefetch
def test_prefetch_hand_computed():
    """C=6, E=8, two layers.  Layer 0 takes slots 0-2, layer 1 slots 3-4;
    the issuing call (layer 0, experts 2 and 3) starts at clock 5, hits slot
    2 and fills slot 5.  Its prefetch of layer 1's experts 1, 4, 5, 6, 7:
    expert 1 hits (slot 4, stamp 8); only slots 0, 1, 3 hold stamps <= 5, so
    4, 5, 6 take them in that (stamp) order and 7 is skipped -- slots 2 and 5,
    which the issuing call uses, are never victims."""
    c = SlotCache(6, 8, 2)
    c.lookup(0, [0, 1, 2])
    c.lookup(1, [0, 1])
    pinned = c.clock
    assert pinned == 5
    c.lookup(0, [2, 3])
    fills = c.prefetch(1, [1, 4, 5, 6, 7], pinned)
    assert fills == [(0, 1, 4), (1, 1, 5), (3, 1, 6)]
    assert c.key == [12, 13, 2, 14, 9, 3]
    assert c.stamp == [9, 10, 6, 11, 8, 7]
    assert c.clock == 11
    assert (c.pf_lookups, c.pf_hits, c.pf_fills) == (5, 1, 3)
    assert c.evictions == 3 and (c.hits, c.fills, c.bypasses) == (1, 6, 0)
    # the prefetched experts are hits for the next layer's lookup
    slots, f2, byp = c.lookup(1, [4, 6])
    assert slots == [0, 3] and not f2 and not byp


def test_prefetch_into_empty_slots_ascending():
    c = SlotCache(5, 4, 2)
    c.lookup(0, [3])                      # slot 0
    pinned = c.clock
    c.lookup(0, [1])                      # slot 1
    assert c.prefetch(1, [0, 2], pinned) == [(2, 1, 0), (3, 1, 2)]
    assert c.key == [3, 1, 4, 6, -1] and c.stamp == [1, 2, 3, 4, 0]


def _prefetch_brute(key, stamp, clock, E, layer, experts, pinned):
    """Independent statement: hits restamped in ascending expert order;
    eligible = slots not holding a listed key with (empty or stamp <= pinned),
    taken in (stamp, index) order by the misses in ascending expert order."""
    key, stamp = list(key), list(stamp)
    listed = {layer * E + e for e in experts}
    for e in experts:
        kk = layer * E + e
        if kk in key:
            clock += 1
            stamp[key.index(kk)] = clock
    eligible = sorted((s for s in range(len(key))
                       if key[s] not in listed and (key[s] < 0 or stamp[s] <= pinned)),
                      key=lambda s: (stamp[s], s))
    misses = [e for e in experts if layer * E + e not in key]
    for e, s in zip(misses, eligible):
        key[s] = layer * E + e
        clock += 1
        stamp[s] = clock
    return key, stamp, clock


@pytest.mark.parametrize("seed", range(40))
def test_prefetch_matches_brute_force(seed):
    """Random traces of lookups, each followed by a prefetch of a random set
    of another layer, against the brute-force statement; and the slots the
    issuing call used keep their keys."""
    rng = np.random.default_rng(seed)
    C, E, L = int(rng.integers(1, 12)), int(rng.integers(2, 10)), 3
    c = SlotCache(C, E, L)
    for _ in range(30):
        layer = int(rng.integers(L))
        U = sorted(set(rng.integers(0, E, int(rng.integers(1, E + 1))).tolist()))
        pinned = c.clock
        slots, _, _ = c.lookup(layer, U)
        used = {s for s in slots if s >= 0}
        nxt = (layer + 1) % L
        P = sorted(set(rng.integers(0, E, int(rng.integers(0, E + 1))).tolist()))
        before = (list(c.key), list(c.stamp), c.clock)
        want = _prefetch_brute(*before, E, nxt, P, pinned)
        fills = c.prefetch(nxt, P, pinned)
        assert (c.key, c.stamp, c.clock) == want
        assert all(c.key[s] == before[0][s] for s in used)
        assert len(fills) == sum(1 for kk in {nxt * E + e for e in P}
                                 if kk in c.key and kk not in before[0])


def test_prefetch_with_nothing_pinned_is_a_lookup():
    """With pinned equal to the current clock (no issuing call) and enough
    room, a prefetch leaves the state a lookup of the same set leaves."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        a, b = SlotCache(8, 6, 2), SlotCache(8, 6, 2)
        for _ in range(6):
            layer = int(rng.integers(2))
            U = sorted(set(rng.integers(0, 6, 3).tolist()))
            a.lookup(layer, U)
            b.lookup(layer, U)
        P = sorted(set(rng.integers(0, 6, 3).tolist()))
        a.prefetch(1, P, a.clock)
        _, _, byp = b.lookup(1, P)
        assert not byp
        assert (a.key, a.stamp, a.clock) == (b.key, b.stamp, b.clock)
