"""Pins of the oracle's slot pool (the page's LRU struct) against a textbook
timestamp LRU written independently, and against invariants that hold for any
LRU swap-in."""
import numpy as np
import pytest

import oracle


W = 128


class TimestampLRU:
    """Least-recently-used by last-use time: each use stamps a clock; the
    victim is the occupied slot with the oldest stamp.  Hits are used first,
    then misses, each in ascending ID order; unused slots go lowest first."""

    def __init__(self, S):
        self.S = S
        self.owner = [None] * S
        self.stamp = [0] * S
        self.clock = 0
        self.hits = self.misses = 0

    def step(self, sel):
        slot_of = {l: s for s, l in enumerate(self.owner) if l is not None}
        hits = [l for l in sel if l in slot_of]
        misses = [l for l in sel if l not in slot_of]
        for l in hits:
            self.clock += 1
            self.stamp[slot_of[l]] = self.clock
            self.hits += 1
        moved = []
        for l in misses:
            unused = [s for s in range(self.S) if self.owner[s] is None]
            if unused:
                s = unused[0]
            else:
                s = min(range(self.S), key=lambda x: self.stamp[x])
            self.owner[s] = l
            self.clock += 1
            self.stamp[s] = self.clock
            slot_of = {l2: s2 for s2, l2 in enumerate(self.owner) if l2 is not None}
            moved.append((l, s))
            self.misses += 1
        slot_of = {l: s for s, l in enumerate(self.owner) if l is not None}
        phys = list(range(W)) + [W + slot_of[l] for l in sel]
        lru = sorted([s for s in range(self.S) if self.owner[s] is not None], key=lambda s: -self.stamp[s])
        return phys, moved, lru


def random_selections(rng, cap, S, steps, overlap=0.7):
    cur = sorted(rng.choice(cap, size=min(S, cap), replace=False)[: rng.integers(1, S + 1)].tolist())
    out = [cur]
    for _ in range(steps - 1):
        keep = [l for l in cur if rng.random() < overlap]
        n_new = int(rng.integers(0, S - len(keep) + 1))
        pool = np.setdiff1d(np.arange(cap), keep)
        new = rng.choice(pool, size=min(n_new, pool.size), replace=False).tolist()
        cur = sorted(set(keep) | set(new))
        out.append(cur)
    return out


@pytest.mark.parametrize("seed", range(8))
def test_matches_timestamp_lru(seed):
    rng = np.random.default_rng(seed)
    cap, S = int(rng.integers(20, 200)), int(rng.integers(4, 19))
    pool = oracle.Pool(cap, S, W, 2048)
    pool.store(0, cap)
    ref = TimestampLRU(S)
    total = 0
    for sel in random_selections(rng, cap, S, 40):
        st, phys, moved = pool.stage(np.array(sel, np.int32))
        assert st == 0
        r_phys, r_moved, r_lru = ref.step(sel)
        assert phys.tolist() == r_phys
        assert moved == r_moved
        sl, lru = pool.state()
        assert lru.tolist() == r_lru
        assert [sl[s] for s in range(S)] == [(-1 if o is None else o) for o in ref.owner]
        total += len(sel)
        s = pool.stats()
        assert s["hits"] == ref.hits and s["misses"] == ref.misses
        assert s["hits"] + s["misses"] == total
        assert s["h2d_bytes"] == 2048 * s["misses"]


def test_invariants_and_repeat():
    rng = np.random.default_rng(99)
    cap, S = 500, 64
    pool = oracle.Pool(cap, S, W, 2048)
    pool.store(0, cap)
    for sel in random_selections(rng, cap, S, 60, overlap=0.8):
        st, phys, _ = pool.stage(np.array(sel, np.int32))
        slots = phys[W:] - W
        assert len(set(slots.tolist())) == len(sel)          # one slot per selected chunk
        assert np.all((slots >= 0) & (slots < S))
        sl, _ = pool.state()
        assert set(sel) <= set(sl.tolist())                   # resident after the step
        assert all(sl[s] == l for s, l in zip(slots, sel))
    m0 = pool.stats()["misses"]
    st, _, moved = pool.stage(np.array(sel, np.int32))      # same selection again: all hits
    assert moved == [] and pool.stats()["misses"] == m0


def test_large_pool_misses_once_per_distinct_id():
    rng = np.random.default_rng(5)
    cap, S = 300, 300
    pool = oracle.Pool(cap, S - 1, W, 4)   # cap > gpu_chunks keeps swapping on
    pool.store(0, cap)
    seen = set()
    for _ in range(30):
        sel = sorted(rng.choice(150, size=40, replace=False).tolist())
        pool.stage(np.array(sel, np.int32))
        seen |= set(sel)
    assert pool.stats()["misses"] == len(seen)


def test_first_fill_uses_lowest_slots():
    pool = oracle.Pool(100, 8, W, 8)
    pool.store(0, 100)
    st, phys, moved = pool.stage(np.array([10, 20, 30], np.int32))
    assert moved == [(10, 0), (20, 1), (30, 2)]
    assert phys[W:].tolist() == [W, W + 1, W + 2]


def test_hits_before_misses_never_evicts_selected():
    # 3 slots, [1,2,3] resident with LRU order 3,2,1 (1 least recent).  Selecting
    # [0, 1] must evict 2 (the LRU among unselected), not 1.
    pool = oracle.Pool(10, 3, W, 8)
    pool.store(0, 10)
    pool.stage(np.array([1, 2, 3], np.int32))
    st, phys, moved = pool.stage(np.array([0, 1], np.int32))
    assert moved == [(0, 1)]                 # slot 1 held ID 2
    assert phys[W:].tolist() == [W + 1, W + 0]


def test_not_stored_is_an_error_and_changes_nothing():
    pool = oracle.Pool(100, 8, W, 8)
    pool.store(0, 50)
    pool.stage(np.array([1, 2], np.int32))
    before = pool.state()
    st, _, _ = pool.stage(np.array([3, 60], np.int32))
    assert st == oracle.ST_NOT_STORED
    after = pool.state()
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    assert pool.stats()["d2h_bytes"] == 50 * 8


def test_swap_disabled_is_identity():
    pool = oracle.Pool(16, 16, W, 8)      # cap <= gpu_chunks
    pool.store(0, 16)
    st, phys, moved = pool.stage(np.array([0, 5, 15], np.int32))
    assert st == 0 and moved == []
    assert phys.tolist() == list(range(W)) + [W + 0, W + 5, W + 15]
    assert pool.stats()["hits"] == 0 and pool.stats()["misses"] == 0


class CapacityLRU(TimestampLRU):
    """The timestamp LRU with a usable-slot capacity: misses take unused slots
    below it; shrinking drops the oldest stamps until the capacity holds the
    rest, then relocates entries above it, lowest first, to the freed slots
    below it, lowest first (stamps move with their entries)."""

    def __init__(self, S):
        super().__init__(S)
        self.C = S

    def step(self, sel):
        full = self.S
        self.S = self.C          # unused slots and victims only below the capacity
        try:
            return super().step(sel)
        finally:
            self.S = full

    def set_capacity(self, C):
        self.C = C
        used = [s for s in range(self.S) if self.owner[s] is not None]
        for s in sorted(used, key=lambda x: self.stamp[x])[:max(0, len(used) - C)]:
            self.owner[s] = None
        high = [s for s in range(C, self.S) if self.owner[s] is not None]
        free = [s for s in range(C) if self.owner[s] is None]
        for a, b in zip(high, free):
            self.owner[b], self.stamp[b] = self.owner[a], self.stamp[a]
            self.owner[a] = None


@pytest.mark.parametrize("seed", range(8))
def test_capacity_changes_match_the_timestamp_model(seed):
    rng = np.random.default_rng(100 + seed)
    cap, S = int(rng.integers(60, 300)), int(rng.integers(12, 40))
    pool = oracle.Pool(cap, S, W, 2048)
    pool.store(0, cap)
    ref = CapacityLRU(S)
    c_min = 4
    for t, sel in enumerate(random_selections(rng, cap, c_min, 60)):
        if t % 5 == 4:
            C = int(rng.integers(c_min, S + 1))
            pool.set_capacity(C)
            ref.set_capacity(C)
            sl, lru = pool.state()
            # shrinking keeps exactly the C most recent entries, in slots 0..n-1
            assert sorted(s for s in range(S) if sl[s] >= 0) == list(range(min(C, len(lru))))
        st, phys, moved = pool.stage(np.array(sel, np.int32))
        assert st == 0
        r_phys, r_moved, r_lru = ref.step(sel)
        assert phys.tolist() == r_phys and moved == r_moved
        sl, lru = pool.state()
        assert lru.tolist() == r_lru
        assert [sl[s] for s in range(S)] == [(-1 if o is None else o) for o in ref.owner]
        assert all(s < pool.capacity() for s in lru)


def test_shrink_keeps_most_recent_and_grow_reuses_lowest_slots():
    pool = oracle.Pool(100, 8, W, 2048)
    pool.store(0, 100)
    pool.stage(np.arange(0, 8, dtype=np.int32))          # slots 0..7 hold 0..7
    pool.stage(np.array([6, 7], np.int32))                # most recent: 7, 6
    pool.stage(np.array([1], np.int32))                   # then 1
    pool.set_capacity(3)                                  # keep 1, 7, 6; 6 and 7 move to slots 0 and 2
    sl, lru = pool.state()
    assert sl.tolist() == [6, 1, 7, -1, -1, -1, -1, -1]
    assert lru.tolist() == [1, 2, 0]                      # LRU order of 1, 7, 6 kept
    st, phys, moved = pool.stage(np.array([50], np.int32))
    assert moved == [(50, 0)]                             # full at 3: the LRU back (6, slot 0) goes
    pool.set_capacity(5)
    st, phys, moved = pool.stage(np.array([60, 61], np.int32))
    assert moved == [(60, 3), (61, 4)]                    # grown: the lowest unused slots first


def test_adapt_policy_decisions():
    pool = oracle.Pool(1000, 64, W, 2048)
    pool.store(0, 1000)
    pool.set_capacity(16)
    pool.stage(np.arange(0, 16, dtype=np.int32))          # 16 misses: miss rate 1
    assert pool.adapt(0.5, 10e6, 0.1, 8, 16, 64, 1) == 24
    pool.stage(np.arange(0, 16, dtype=np.int32))          # all hits: miss rate 0 -> shrink
    assert pool.adapt(0.5, 10e6, 0.1, 8, 16, 64, 1) == 16
    pool.stage(np.arange(0, 16, dtype=np.int32))
    assert pool.adapt(0.5, 10e6, 0.1, 8, 16, 64, 1) == 16  # floor
    assert pool.adapt(0.5, 10e6, 0.1, 8, 16, 64, 1) == 16  # no lookups, no change
    pool.stage(np.arange(8, 24, dtype=np.int32))          # 8 hits, 8 misses: 0.5 is not above 0.5
    assert pool.adapt(0.5, 10e6, 0.1, 8, 16, 64, 1) == 16
    pool.stage(np.arange(100, 116, dtype=np.int32))       # 16 misses = 32 KB of H2D in 4 steps
    assert pool.adapt(1.1, 4096, 0.0, 8, 16, 64, 4) == 24  # the H2D rule alone grows
    for _ in range(6):
        pool.stage(np.arange(200 + 16 * _, 216 + 16 * _, dtype=np.int32))
        pool.adapt(0.5, 10e6, 0.1, 32, 16, 64, 1)
    assert pool.capacity() == 64                          # ceiling


class WeightedTimestampLRU:
    """An independent model of the [P4] §3.2 reading: recency from last-use
    stamps; the step's candidates (resident, not selected) ranked by recency a and
    importance c, evicted in ascending w*a + (100-w)*c (ties: less recent first);
    misses take the lowest free slot below the capacity first; then the
    high-water mark frees slots down to max(h*C/100, |sel|)."""

    def __init__(self, S, C=None):
        self.S, self.C = S, S if C is None else C
        self.owner = [None] * S
        self.stamp = [0] * S
        self.clock = 0

    def step(self, sel, imp, w, h):
        chosen = set(sel)
        cand = sorted((s for s in range(self.S) if self.owner[s] is not None and self.owner[s] not in chosen),
                      key=lambda s: self.stamp[s])
        a = {s: i for i, s in enumerate(cand)}
        c = {s: i for i, s in enumerate(sorted(cand, key=lambda s: (imp[self.owner[s]], a[s])))}
        order = sorted(cand, key=lambda s: (w * a[s] + (100 - w) * c[s], a[s]))
        slot_of = {l: s for s, l in enumerate(self.owner) if l is not None}
        for l in sel:
            if l in slot_of:
                self.clock += 1
                self.stamp[slot_of[l]] = self.clock
        nxt = 0
        moved = []
        for l in sel:
            if l in slot_of:
                continue
            free = [s for s in range(self.C) if self.owner[s] is None]
            if free:
                s = free[0]
            else:
                s = order[nxt]
                nxt += 1
            self.owner[s] = l
            self.clock += 1
            self.stamp[s] = self.clock
            moved.append((l, s))
        limit = max(h * self.C // 100, len(sel))
        while sum(o is not None for o in self.owner) > limit and nxt < len(order):
            self.owner[order[nxt]] = None
            nxt += 1
        slot_of = {l: s for s, l in enumerate(self.owner) if l is not None}
        lru = sorted(slot_of.values(), key=lambda s: -self.stamp[s])
        return [W + slot_of[l] for l in sel], moved, lru


@pytest.mark.parametrize("w,h", [(100, 100), (50, 100), (0, 100), (100, 70), (50, 70), (20, 40)])
def test_weighted_replacement_matches_independent_model(w, h):
    rng = np.random.default_rng(w * 7 + h)
    for run in range(4):
        cap, S = int(rng.integers(30, 120)), int(rng.integers(6, 20))
        pool = oracle.Pool(cap, S, W, 2048)
        pool.store(0, cap)
        pool.set_replacement(w, h)
        ref = WeightedTimestampLRU(S)
        for sel in random_selections(rng, cap, S, 25, overlap=0.6):
            imp = L_grid(rng, cap)
            st, phys, moved = pool.stage(np.array(sel, np.int32), imp)
            want_phys, want_moved, want_lru = ref.step(sel, imp, w, h)
            assert st == 0
            assert phys[W:].tolist() == want_phys, (run, sel)
            assert moved == want_moved
            sl, lru = pool.state()
            assert lru.tolist() == want_lru
            assert sl.tolist() == [o if o is not None else -1 for o in ref.owner]


def L_grid(rng, n):
    """Importance scores with many ties (1/8 grid in [0, 1])."""
    return (rng.integers(0, 9, size=n) / 8).astype(np.float32)


def test_importance_only_evicts_the_least_important():
    """w = 0: the evicted entries are the candidates of lowest importance (ties to
    the less recent), whatever their recency."""
    pool = oracle.Pool(100, 4, W, 8)
    pool.store(0, 100)
    pool.set_replacement(0, 100)
    imp = np.zeros(100, np.float32)
    imp[[10, 11, 12, 13]] = [0.9, 0.1, 0.5, 0.3]
    pool.stage(np.array([10, 11, 12, 13], np.int32), imp)     # fills slots 0..3
    # touch 11 last so that it is the most recent, yet the least important
    pool.stage(np.array([11], np.int32), imp)
    st, phys, moved = pool.stage(np.array([50, 51], np.int32), imp)
    assert st == 0 and moved == [(50, 1), (51, 3)]             # 11 (0.1) then 13 (0.3) leave


def test_high_water_keeps_room_for_the_next_misses():
    """h = 50 with 8 slots: after every step at most max(4, |sel|) slots are in
    use, and every selected entry is resident."""
    pool = oracle.Pool(1000, 8, W, 8)
    pool.store(0, 1000)
    pool.set_replacement(100, 50)
    rng = np.random.default_rng(3)
    for _ in range(20):
        sel = np.sort(rng.choice(1000, size=int(rng.integers(1, 7)), replace=False)).astype(np.int32)
        st, _, _ = pool.stage(sel)
        sl, lru = pool.state()
        assert st == 0 and len(lru) <= max(4, sel.size)
        assert set(sel.tolist()) <= set(sl.tolist())
