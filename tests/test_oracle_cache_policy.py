"""Pins for the oracle's alternative placement policies (no GPU).

"per_layer" must behave as one independent LRU per layer over that layer's
share of the slots, and "static" must never change the placement a fill made.
Each is checked against a separately written model: textbook OrderedDict
LRUs (one per layer) for calls whose unique set fits the layer's share, an
explicit per-layer recency list by brute force over small traces, and the
plain set arithmetic of a fixed placement.
"""
import itertools
from collections import OrderedDict

import numpy as np
import pytest

from oracle.cache import SlotCache


def _share(layer, C, L):
    return list(range(layer * C // L, (layer + 1) * C // L))


class PerLayerRecency:
    """Second model: one least-to-most-recent list per layer over its slots."""

    def __init__(self, C, E, L):
        self.E = E
        self.owner = [None] * C
        self.order = [_share(l, C, L) for l in range(L)]  # empty slots first, ascending

    def lookup(self, layer, experts):
        keys = [layer * self.E + e for e in experts]
        where = {k: s for s, k in enumerate(self.owner) if k is not None}
        hit = [where[k] for k in keys if k in where]
        miss = [k for k in keys if k not in where]
        free = [s for s in self.order[layer] if s not in hit]
        res, filled = {}, []
        for r, k in enumerate(miss):
            if r < len(free):
                self.owner[free[r]] = k
                filled.append(free[r])
                res[k] = free[r]
            else:
                res[k] = -1 - (r - len(free))
        for k in keys:
            if k in where:
                res[k] = where[k]
        touched = set(hit) | set(filled)
        self.order[layer] = [s for s in self.order[layer] if s not in touched] + hit + filled
        return [res[k] for k in keys]


def test_per_layer_is_one_textbook_lru_per_layer():
    rng = np.random.default_rng(3)
    for trial in range(30):
        E, L = 12, 3
        C = int(rng.integers(L, 16))
        c = SlotCache(C, E, n_layers=L, policy="per_layer")
        lrus = [OrderedDict() for _ in range(L)]
        for _ in range(50):
            layer = int(rng.integers(0, L))
            cap = len(_share(layer, C, L))
            n = int(rng.integers(1, cap + 1))
            U = sorted(rng.choice(E, n, replace=False).tolist())
            slots, fills, byp = c.lookup(layer, U)
            assert not byp
            assert all(s in _share(layer, C, L) for s in slots)
            lru = lrus[layer]
            keys = [layer * E + e for e in U]
            for k in [k for k in keys if k in lru]:
                lru.move_to_end(k)
            for k in [k for k in keys if k not in lru]:
                if len(lru) >= cap:
                    lru.popitem(last=False)
                lru[k] = True
            for l in range(L):
                held = {c.key[s]: c.stamp[s] for s in _share(l, C, L) if c.key[s] >= 0}
                assert sorted(held, key=held.get) == list(lrus[l])


@pytest.mark.parametrize("E,L,C,calls", [(2, 2, 2, 4), (2, 2, 3, 4), (3, 2, 3, 3), (3, 2, 1, 4),
                                         (2, 3, 4, 3)])
def test_per_layer_brute_force(E, L, C, calls):
    subsets = [s for r in range(1, E + 1) for s in itertools.combinations(range(E), r)]
    space = [(l, s) for l in range(L) for s in subsets]
    for trace in itertools.product(space, repeat=calls):
        a = SlotCache(C, E, n_layers=L, policy="per_layer")
        b = PerLayerRecency(C, E, L)
        for layer, U in trace:
            n0 = a.hits + a.fills + a.bypasses
            sa, _, _ = a.lookup(layer, list(U))
            assert sa == b.lookup(layer, list(U)), (trace, layer, U)
            assert a.key == [k if k is not None else -1 for k in b.owner]
            assert a.hits + a.fills + a.bypasses - n0 == len(U)


def test_per_layer_empty_share_bypasses_everything():
    c = SlotCache(2, 8, n_layers=4, policy="per_layer")  # layers 0 and 2 own no slot
    assert _share(0, 2, 4) == [] and _share(1, 2, 4) == [0]
    slots, fills, byp = c.lookup(0, [1, 2])
    assert slots == [-1, -2] and not fills and len(byp) == 2
    slots, fills, byp = c.lookup(1, [1, 2])
    assert slots == [0, -1] and fills == [(0, 1, 1)]


def test_static_keeps_the_filled_set():
    rng = np.random.default_rng(5)
    E, L, C = 10, 2, 6
    c = SlotCache(C, E, n_layers=L, policy="static")
    pinned = {0: [1, 4, 7], 1: [0, 2, 9]}
    for l, es in pinned.items():
        _, fills, byp = c.fill(l, es)
        assert len(fills) == 3 and not byp
    placed = list(c.key)
    slot_of = {k: s for s, k in enumerate(placed)}
    for _ in range(40):
        layer = int(rng.integers(0, L))
        U = sorted(rng.choice(E, int(rng.integers(1, E + 1)), replace=False).tolist())
        clock0, hits0 = c.clock, c.hits
        slots, fills, byp = c.lookup(layer, U)
        assert not fills and c.key == placed
        held = [e for e in U if e in pinned[layer]]
        assert [slots[U.index(e)] for e in held] == [slot_of[layer * E + e] for e in held]
        missing = [e for e in U if e not in pinned[layer]]
        assert [b[2] for b in byp] == missing
        assert [slots[U.index(e)] for e in missing] == [-1 - i for i in range(len(missing))]
        assert c.hits - hits0 == len(held) and c.clock - clock0 == len(held)
        for i, e in enumerate(held):
            assert c.stamp[slot_of[layer * E + e]] == clock0 + 1 + i


def test_resize_is_global_only():
    for policy in ("per_layer", "static"):
        with pytest.raises(AssertionError):
            SlotCache(4, 8, n_layers=2, policy=policy).resize(2)
