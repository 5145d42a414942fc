"""Pins of the oracle's decode-step chain (oracle.DecodeState) for the parts the
per-function pins do not cover: a periodic indexer whose prediction serves a
window of steps, chunks stored while decoding, and a step that selects a chunk
never stored.  Expected values come from scipy's softmax, hand-worked slot
tables and closed forms, not from the oracle's own routines."""
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np
import pytest
from scipy.special import softmax

import lsa_inputs as L
import oracle


@dataclass
class TinyWL:
    """A hand-sized workload: one ratio-4 layer, 1 sequence, dk 4, one indexer head."""
    n_src: int = 24
    kv_dim: int = 8
    window: int = 2
    gpu_chunks: int = 3
    k: int = 2
    hq: int = 2
    batch: int = 1
    n_layers: int = 1
    src_ratio: int = 4
    layer_ratios: Tuple[int, ...] = (4,)
    key_dtype: str = "f32"
    kv_dtype: str = "f32"
    ensemble: str = "max"
    mode: str = "topk"
    tau: Optional[float] = None
    scale: float = 0.5

    def layer_cap(self, l):
        return self.n_src * self.src_ratio // self.layer_ratios[l]


def one_hot_keys(n, dk):
    """key j points along axis j % dk with length j // dk + 1: the score of a
    one-hot query on axis a is largest for the highest j with j % dk == a."""
    keys = np.zeros((n, dk), np.float32)
    for j in range(n):
        keys[j, j % dk] = j // dk + 1
    return keys


def query(axes, dk=4):
    q = np.zeros((1, 1, 1, dk), np.float32)
    for a in axes:
        q[0, 0, 0, a] = 1.0
    return q


def dense(q, rows, scale):
    """scipy softmax attention of every head over the given rows (K = V = rows)."""
    z = scale * (q.astype(np.float64) @ rows.astype(np.float64).T)
    return (softmax(z, axis=-1) @ rows.astype(np.float64)).astype(np.float32)


def make_state(wl, stored=None, seed=0):
    rng = np.random.default_rng(seed)
    win = [[L.grid_uniform(rng, (wl.window, wl.kv_dim))]]
    store = [[L.grid_uniform(rng, (wl.layer_cap(0), wl.kv_dim))]]
    st = oracle.DecodeState(wl, win, store, stored=None if stored is None else [[stored]])
    return st, win[0][0], store[0][0]


def test_periodic_indexer_window_of_two_steps():
    """Period 2: the prediction of step 0 serves steps 0 and 1, that of step 2
    serves steps 2 and 3.  Non-predicting steps stage nothing (counters and the
    slot table stay) and attend over the held rows; the slot table after each
    prediction is the hand-worked LRU state."""
    wl = TinyWL()
    st, win, store = make_state(wl)
    keys = [one_hot_keys(wl.n_src, 4)]
    w = np.ones((1, 1, 1), np.float32)
    rng = np.random.default_rng(5)
    qa = [L.grid_uniform(rng, (1, 1, wl.hq, wl.kv_dim)) for _ in range(4)]
    # step 0: query on axes 0 and 1 -> top-2 = entries 20 (axis 0) and 21 (axis 1)
    r0 = st.step(keys, query([0, 1]), w, qa[0])
    assert r0["sel"][0].tolist() == [20, 21]
    assert r0["misses"][0][0] == [(20, 0), (21, 1)]
    r1 = st.step(keys, query([2]), w, qa[1], predict=False)   # its indexer query is not used
    assert r1["layer_sel"][0][0].tolist() == [20, 21] and r1["misses"][0][0] == []
    assert st.pools[0][0].stats()["hits"] == 0 and st.pools[0][0].stats()["misses"] == 2
    for r, q in ((r0, qa[0]), (r1, qa[1])):
        want = dense(q[0, 0], np.concatenate([win, store[[20, 21]]]), wl.scale)
        assert np.allclose(r["out"][0][0], want, rtol=0, atol=1e-6)
    # step 2: axes 1 and 2 -> entries 21 (hit) and 22 (miss into the free slot 2)
    r2 = st.step(keys, query([1, 2]), w, qa[2])
    assert r2["sel"][0].tolist() == [21, 22]
    assert r2["misses"][0][0] == [(22, 2)]
    sl, lru = st.pools[0][0].state()
    assert sl.tolist() == [20, 21, 22] and lru.tolist() == [2, 1, 0]
    r3 = st.step(keys, query([3]), w, qa[3], predict=False)
    want = dense(qa[3][0, 0], np.concatenate([win, store[[21, 22]]]), wl.scale)
    assert np.allclose(r3["out"][0][0], want, rtol=0, atol=1e-6)
    s = st.pools[0][0].stats()
    assert (s["hits"], s["misses"]) == (1, 3)


def test_period_one_is_every_step_predicting():
    """predict=True on every step is the plain synchronous chain: the same
    selections and outputs as a fresh state driven step by step."""
    wl = TinyWL()
    a, _, _ = make_state(wl)
    b, _, _ = make_state(wl)
    keys = [one_hot_keys(wl.n_src, 4)]
    w = np.ones((1, 1, 1), np.float32)
    rng = np.random.default_rng(6)
    for t, axes in enumerate(([0, 1], [1, 2], [3, 0], [2, 3])):
        qa = L.grid_uniform(rng, (1, 1, wl.hq, wl.kv_dim))
        ra = a.step(keys, query(axes), w, qa)
        rb = b.step(keys, query(axes), w, qa, predict=True)
        assert ra["sel"][0].tolist() == rb["sel"][0].tolist()
        assert np.array_equal(ra["out"][0][0], rb["out"][0][0])


def test_store_during_decoding_and_not_stored():
    """Entries stored while decoding become selectable; a prediction that
    selects an entry never stored changes nothing of the pool and gives zero
    output (also on the window steps it serves), and the next good prediction
    proceeds from the unchanged slot table."""
    wl = TinyWL()
    st, win, store = make_state(wl, stored=20)       # entries 20..23 not stored yet
    keys = [one_hot_keys(wl.n_src, 4)]
    w = np.ones((1, 1, 1), np.float32)
    qa = np.ones((1, 1, wl.hq, wl.kv_dim), np.float32) / 8
    r = st.step(keys, query([0, 1]), w, qa, n_valid=[20])           # entries 16, 17
    assert r["sel"][0].tolist() == [16, 17] and r["status"][0][0] == 0
    before = (st.pools[0][0].state(), st.pools[0][0].stats())
    r = st.step(keys, query([0, 1]), w, qa, n_valid=[24])           # 20, 21: never stored
    assert r["sel"][0].tolist() == [20, 21] and r["status"][0][0] == oracle.ST_NOT_STORED
    assert np.array_equal(r["out"][0][0], np.zeros((wl.hq, wl.kv_dim), np.float32))
    r = st.step(keys, query([0, 1]), w, qa, predict=False)
    assert np.array_equal(r["out"][0][0], np.zeros((wl.hq, wl.kv_dim), np.float32))
    after = (st.pools[0][0].state(), st.pools[0][0].stats())
    assert np.array_equal(before[0][0], after[0][0]) and np.array_equal(before[0][1], after[0][1])
    assert before[1] == after[1]
    new_rows = np.full((4, wl.kv_dim), 0.25, np.float32)
    st.store(0, 0, 20, new_rows)
    r = st.step(keys, query([0, 1]), w, qa, n_valid=[24])
    assert r["status"][0][0] == 0 and r["misses"][0][0] == [(20, 2), (21, 0)]
    want = dense(qa[0, 0], np.concatenate([win, new_rows[:2]]), wl.scale)
    assert np.allclose(r["out"][0][0], want, rtol=0, atol=1e-6)
    assert st.pools[0][0].stats()["d2h_bytes"] == 24 * wl.kv_dim * 4


def test_restore_of_a_staged_entry_keeps_it_staged_with_new_content():
    """[P1] store flow: storing an entry that is staged keeps it in its slot (no
    eviction, LRU order unchanged); attention then reads the new content."""
    wl = TinyWL()
    st, win, store = make_state(wl)
    keys = [one_hot_keys(wl.n_src, 4)]
    w = np.ones((1, 1, 1), np.float32)
    qa = np.ones((1, 1, wl.hq, wl.kv_dim), np.float32) / 8
    st.step(keys, query([0, 1]), w, qa)
    sl0, lru0 = st.pools[0][0].state()
    fresh = np.full((1, wl.kv_dim), -0.5, np.float32)
    st.store(0, 0, 21, fresh)
    sl1, lru1 = st.pools[0][0].state()
    assert np.array_equal(sl0, sl1) and np.array_equal(lru0, lru1)
    r = st.step(keys, query([0, 1]), w, qa, predict=False)
    want = dense(qa[0, 0], np.concatenate([win, store[[20]], fresh]), wl.scale)
    assert np.allclose(r["out"][0][0], want, rtol=0, atol=1e-6)


def test_ratio128_layer_skips_the_incomplete_chunk():
    """With 33 valid source entries (132 tokens) a ratio-128 layer has one
    complete chunk; a selection of source entry 32 maps to the incomplete chunk
    1, which is left out (its tokens lie in the window), so no error 4 although
    chunk 1 is not stored."""
    wl = TinyWL(n_src=64, layer_ratios=(128,), gpu_chunks=4)
    st, win, store = make_state(wl, stored=1)
    keys = [one_hot_keys(64, 4)]
    w = np.ones((1, 1, 1), np.float32)
    qa = np.ones((1, 1, wl.hq, wl.kv_dim), np.float32) / 8
    r = st.step(keys, query([0]), w, qa, n_valid=[33], k=2)       # entries 32 and 28
    assert r["sel"][0].tolist() == [28, 32]
    assert r["layer_sel"][0][0].tolist() == [0] and r["status"][0][0] == 0
