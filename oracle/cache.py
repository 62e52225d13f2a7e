"""State of the HBM expert cache: fixed slots, one global LRU over layers.

Test infrastructure (see the package docstring).

The pages describe one global LRU cache across the MoE layers, used during
decode instead of pinning chosen experts at start-up (jansverre.net FreeToken
article, section "Hvorfor er båndbredden viktigere enn antall kjerner?"), that
exploits expert overlap between adjacent tokens (aipolix.com FreeToken
article, fifth paragraph), whose size can change without restarting or
reloading the host-resident expert pool (same article, sixth paragraph).
They give no algorithm; the readings below are this implementation's.

State: ``key[C]`` (layer*E + expert, -1 = empty), ``stamp[C]`` (0 = empty,
otherwise a unique recency number), ``clock``.

lookup(layer, U) for the ascending unique experts U of one call:
  1. start = clock;
  2. hits, in ascending expert: clock += 1, stamp the slot with clock;
  3. victims = empty slots in ascending index, then occupied slots whose
     stamp <= start in ascending stamp (this call's hits are pinned);
  4. the i-th miss (ascending expert) takes victims[i] when it exists
     (evicting its key; clock += 1; stamp; a fill of that slot is issued);
     otherwise it bypasses the cache through staging slot b (the b-th
     bypass), encoded -1-b, and the state is unchanged.
prefetch(layer, U, pinned) for ascending unique experts U (global policy):
  the same as a lookup except that
  - a miss may take only empty slots (ascending index) and occupied slots
    whose stamp <= pinned (ascending stamp), where pinned is the clock
    before the lookup of the call that issues the prefetch, so that nothing
    that call uses is displaced while its kernels read it;
  - a miss with no such slot is skipped: no staging copy, state unchanged.
  Hits are stamped and the clock advances as in a lookup.  Its counts are
  kept apart (pf_lookups, pf_hits, pf_fills); its evictions add to
  evictions.  This build's reading of a cross-layer prefetch of likely
  misses: the pages carry the layer-ahead upload into prefill (aipolix.com
  FreeToken article, fourth paragraph) and mention preloading experts that
  activation patterns mark as likely (world.tibi.club FreeToken article,
  section "Cum reușește FreeToken să ruleze 753B pe un singur GPU?", third
  technique) without a rule.
resize(C'): grow appends empty slots; shrink evicts occupied slots in
  ascending stamp while occupancy > C', then moves every survivor in a slot
  >= C' (ascending) to the lowest empty slot < C' (ascending), keeping key
  and stamp.  clock is unchanged.

Placement policies.  The pages set the global LRU against placements that
lock chosen experts into GPU memory at start-up, and quote the miss rates of
the global cache and of two other engines at equal capacity (jansverre.net
FreeToken article, section "Hvorfor er båndbredden viktigere enn antall
kjerner?").  Two alternatives to the global LRU are modelled with the same
rule, for that comparison:
  - "per_layer": layer l owns the slots floor(l C / L) .. floor((l+1) C / L) - 1
    and a lookup of layer l takes its victims from those slots only (empty
    ones ascending, then its occupied ones whose stamp <= start, ascending);
  - "static": lookups never insert, so every miss bypasses; only fill()
    places experts (with the global rule), e.g. a set chosen beforehand.
Hits, stamps and the clock follow the same rule under every policy.  resize
is defined for the global policy only.
"""


POLICIES = ("global", "per_layer", "static")


class SlotCache:
    def __init__(self, capacity: int, n_experts: int, n_layers: int = 1, policy: str = "global"):
        assert policy in POLICIES
        self.E = n_experts
        self.L = n_layers
        self.policy = policy
        self.key = [-1] * capacity
        self.stamp = [0] * capacity
        self.clock = 0
        self.hits = self.fills = self.bypasses = self.evictions = 0
        self.pf_lookups = self.pf_hits = self.pf_fills = 0

    @property
    def capacity(self):
        return len(self.key)

    def slot_of(self, key):
        for s, k in enumerate(self.key):
            if k == key:
                return s
        return None

    def victim_range(self, layer: int):
        """The slots a lookup of `layer` may fill."""
        if self.policy == "per_layer":
            C, L = self.capacity, self.L
            return range(layer * C // L, (layer + 1) * C // L)
        return range(self.capacity)

    def lookup(self, layer: int, experts, insert=None):
        """Returns (slots, fills, bypass).

        slots[i] >= 0: the cache slot of experts[i]; < 0: -1 - staging index.
        fills: [(slot, layer, expert)] in issue order; bypass: [(staging,
        layer, expert)].  insert (default: every policy but "static") lets
        misses take victims.
        """
        if insert is None:
            insert = self.policy != "static"
        experts = [int(e) for e in experts]
        assert experts == sorted(set(experts)), "experts must be ascending unique"
        start = self.clock
        keys = [layer * self.E + e for e in experts]
        slots = [None] * len(keys)
        misses = []
        for i, kk in enumerate(keys):
            s = self.slot_of(kk)
            if s is None:
                misses.append(i)
            else:
                self.clock += 1
                self.stamp[s] = self.clock
                slots[i] = s
                self.hits += 1
        rng = self.victim_range(layer)
        empty = [s for s in rng if self.key[s] < 0]
        old = sorted((self.stamp[s], s) for s in rng
                     if self.key[s] >= 0 and self.stamp[s] <= start)
        victims = empty + [s for _, s in old] if insert else []
        fills, bypass = [], []
        for r, i in enumerate(misses):
            e = experts[i]
            if r < len(victims):
                s = victims[r]
                if self.key[s] >= 0:
                    self.evictions += 1
                self.key[s] = keys[i]
                self.clock += 1
                self.stamp[s] = self.clock
                slots[i] = s
                fills.append((s, layer, e))
                self.fills += 1
            else:
                b = r - len(victims)
                slots[i] = -1 - b
                bypass.append((b, layer, e))
                self.bypasses += 1
        return slots, fills, bypass

    def prefetch(self, layer: int, experts, pinned: int):
        """Insert-only lookup of a predicted set (see the module docstring).
        Returns the fills [(slot, layer, expert)] in issue order."""
        assert self.policy == "global", "prefetch is defined for the global policy only"
        experts = [int(e) for e in experts]
        assert experts == sorted(set(experts)), "experts must be ascending unique"
        keys = [layer * self.E + e for e in experts]
        misses = []
        for kk, e in zip(keys, experts):
            s = self.slot_of(kk)
            self.pf_lookups += 1
            if s is None:
                misses.append((kk, e))
            else:
                self.clock += 1
                self.stamp[s] = self.clock
                self.pf_hits += 1
        empty = [s for s in range(self.capacity) if self.key[s] < 0]
        old = sorted((self.stamp[s], s) for s in range(self.capacity)
                     if self.key[s] >= 0 and self.stamp[s] <= pinned)
        victims = empty + [s for _, s in old]
        fills = []
        for (kk, e), s in zip(misses, victims):
            if self.key[s] >= 0:
                self.evictions += 1
            self.key[s] = kk
            self.clock += 1
            self.stamp[s] = self.clock
            fills.append((s, layer, e))
            self.pf_fills += 1
        return fills

    def fill(self, layer: int, experts):
        """Explicit preload: the same rule as a lookup, inserting under every
        policy (it is how the "static" set is placed)."""
        return self.lookup(layer, experts, insert=True)

    def resize(self, new_capacity: int):
        """Returns (moves [(src, dst)], evicted keys)."""
        assert new_capacity >= 0
        assert self.policy == "global", "resize is defined for the global policy only"
        C = self.capacity
        if new_capacity >= C:
            self.key += [-1] * (new_capacity - C)
            self.stamp += [0] * (new_capacity - C)
            return [], []
        evicted = []
        occupied = sorted((self.stamp[s], s) for s in range(C) if self.key[s] >= 0)
        n_occ = len(occupied)
        for _, s in occupied:
            if n_occ <= new_capacity:
                break
            evicted.append(self.key[s])
            self.key[s] = -1
            self.stamp[s] = 0
            n_occ -= 1
            self.evictions += 1
        moves = []
        free = [s for s in range(new_capacity) if self.key[s] < 0]
        for s in range(new_capacity, C):
            if self.key[s] >= 0:
                d = free.pop(0)
                self.key[d], self.stamp[d] = self.key[s], self.stamp[s]
                self.key[s], self.stamp[s] = -1, 0
                moves.append((s, d))
        del self.key[new_capacity:]
        del self.stamp[new_capacity:]
        return moves, evicted

    def reset(self):
        """Every slot empty, every key absent; the clock and the counters are
        kept.  A cold restart of the cache without recreating it or reloading
        the host pool: the recovery after a failed copy, so that no entry
        whose bytes may not have landed stays resident.  (This build's rule;
        the pages report only that a cold server could hang.)  Returns the
        number of entries dropped."""
        n = sum(1 for k in self.key if k >= 0)
        self.key = [-1] * self.capacity
        self.stamp = [0] * self.capacity
        return n

    def snapshot(self):
        return list(self.key), list(self.stamp), self.clock
