"""Pins of the KVSwap step oracle (KVSwap article, sections 2.2-2.3 and 3.2)
against computations that do not share its code path."""
import numpy as np
import pytest
from scipy.special import softmax

import lsa_inputs as L
import oracle

pytestmark = pytest.mark.filterwarnings("ignore")


def _tiny(**kw):
    base = dict(name="kv_tiny", base_seed=77, ctx=96, batch=1, layers=1, groups=1, k=12, slots=12,
                group_heads=2, head_dim=64, rank=16, steps=3, drift=0.25)
    base.update(kw)
    return L.KVSwapWorkload(**base)


def _inputs(wl, step=0, prev=None):
    U = L.lowrank_U(wl, 0, 0, 0)
    S = L.lowrank_S(wl, 0, 0, 0)
    V = L.lowrank_V(wl, 0, 0, 0)
    q = L.kvswap_query(wl, 0, 0, 0, step, prev)
    cold = L.kvswap_cold(wl, 0, 0)
    return U, S, V, q, cold


def _enc(*xs):
    return [L.f32_to_f16_bits(x) for x in xs]


def test_selecting_every_position_is_dense_attention_per_head():
    # k = T: the step must reduce to plain softmax attention of every head over all positions
    wl = _tiny(k=96, slots=96)
    U, S, V, q, cold = _inputs(wl)
    st = oracle.KVSwapState(wl, [0])
    Ub, Vb, cb = _enc(U, V, cold)
    res = st.step(0, Ub, S, Vb, q, cb)
    assert np.array_equal(res["sel"], np.arange(96))
    H, dh, C = wl.group_heads, wl.head_dim, wl.C
    for h in range(H):
        K = cold[:, h * dh:(h + 1) * dh].astype(np.float64)
        Vv = cold[:, C + h * dh:C + (h + 1) * dh].astype(np.float64)
        p = softmax(K @ q[h * dh:(h + 1) * dh].astype(np.float64) * wl.scale)
        np.testing.assert_allclose(res["out"][h], p @ Vv, rtol=1e-6, atol=1e-7)


def test_selection_is_top_k_of_factored_numpy_scores():
    # scores from a different order (p = S V^T q first, then U p) are exact on the grid; the
    # selection is the k largest with ties to the lowest position, ascending
    wl = _tiny()
    U, S, V, q, cold = _inputs(wl)
    p = S.astype(np.float64) * (V.astype(np.float64).T @ q.astype(np.float64))
    e = U.astype(np.float64) @ p
    order = sorted(range(wl.ctx), key=lambda t: (-e[t], t))
    want = np.sort(np.array(order[:wl.k]))
    st = oracle.KVSwapState(wl, [0])
    Ub, Vb, cb = _enc(U, V, cold)
    res = st.step(0, Ub, S, Vb, q, cb)
    assert np.array_equal(res["score"], e.astype(np.float32))
    assert np.array_equal(res["sel"], want)
    # the grid keeps every score exact in fp32 (the bound the inputs are drawn for)
    assert np.all(np.abs(e) * 4096 == np.round(np.abs(e) * 4096))


def test_slots_over_steps_follow_lru_and_attention_ignores_placement():
    wl = _tiny(slots=12)
    st = oracle.KVSwapState(wl, [0])
    prev = None
    seen = set()
    for t in range(wl.steps):
        U, S, V, q, cold = _inputs(wl, t, prev)
        prev = q
        Ub, Vb, cb = _enc(U, V, cold)
        res = st.step(0, Ub, S, Vb, q, cb)
        sel = set(res["sel"].tolist())
        # misses are exactly the positions not staged in the previous step
        assert {m for m, _ in res["misses"]} == sel - seen
        seen = sel
        # slots are distinct and inside the pool
        assert len(set(res["phys"].tolist())) == len(sel) and res["phys"].max() < wl.slots
        # same output from a fresh pool (different placement)
        fresh = oracle.KVSwapState(wl, [0]).step(0, Ub, S, Vb, q, cb)
        assert np.array_equal(fresh["out"], res["out"])
