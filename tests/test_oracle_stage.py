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
