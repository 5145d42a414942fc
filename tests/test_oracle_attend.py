"""Pins of oracle.attend and the KVSwap functions: dense attention as a
library softmax, exact special cases, and the low-rank reconstruction."""
import numpy as np
import pytest
from scipy.special import softmax

import lsa_inputs as L
import oracle


def dense_attention(q, rows, scale):
    """softmax(scale * q K^T) V with K = V = rows, in float64 via scipy."""
    z = scale * (q.astype(np.float64) @ rows.astype(np.float64).T)
    return softmax(z, axis=-1) @ rows.astype(np.float64)


@pytest.mark.parametrize("seed", range(4))
def test_all_chunks_selected_is_dense_attention(seed):
    rng = np.random.default_rng(seed)
    Hq, D, W, cap = 4, 64, 16, 40
    q = L.grid_uniform(rng, (Hq, D))
    win = L.grid_uniform(rng, (W, D))
    store = L.grid_uniform(rng, (cap, D))
    scale = 1 / np.sqrt(D)
    got = oracle.attend(q, win, store, "f32", np.arange(cap), scale)
    want = dense_attention(q, np.concatenate([win, store]), scale)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-7)


def test_selection_picks_the_named_rows():
    rng = np.random.default_rng(1)
    Hq, D, W, cap = 3, 32, 8, 50
    q = L.grid_uniform(rng, (Hq, D))
    win = L.grid_uniform(rng, (W, D))
    store = L.grid_uniform(rng, (cap, D))
    sel = np.array([2, 7, 30, 49])
    got = oracle.attend(q, win, store, "f32", sel, 0.3)
    want = dense_attention(q, np.concatenate([win, store[sel]]), 0.3)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-7)


def test_single_row_returns_it_exactly():
    rng = np.random.default_rng(2)
    row = L.grid_uniform(rng, (1, 48))
    q = L.grid_uniform(rng, (5, 48))
    out = oracle.attend(q, np.zeros((0, 48), np.float32), row, "f32", np.array([0]), 0.7)
    assert np.array_equal(out, np.repeat(row, 5, 0))


def test_zero_query_is_row_mean():
    rng = np.random.default_rng(3)
    rows = L.grid_uniform(rng, (24, 16))
    out = oracle.attend(np.zeros((2, 16), np.float32), rows[:8], rows[8:], "f32", np.arange(16), 0.5)
    np.testing.assert_allclose(out, np.repeat(rows.astype(np.float64).mean(0, keepdims=True), 2, 0),
                               rtol=0, atol=1e-7)


def test_no_rows_gives_zero():
    out = oracle.attend(np.ones((2, 8), np.float32), np.zeros((0, 8), np.float32),
                        np.zeros((4, 8), np.float32), "f32", np.array([], np.int32), 1.0)
    assert np.array_equal(out, np.zeros((2, 8), np.float32))


def test_bf16_storage_matches_f32():
    rng = np.random.default_rng(4)
    q = L.grid_uniform(rng, (4, 64))
    win = L.grid_uniform(rng, (8, 64))
    store = L.grid_uniform(rng, (30, 64))
    sel = np.array([1, 5, 6, 29])
    a = oracle.attend(q, win, store, "f32", sel, 0.125)
    b = oracle.attend(q, L.f32_to_bf16_bits(win), L.f32_to_bf16_bits(store), "bf16", sel, 0.125)
    assert np.array_equal(a, b)


def test_lowrank_score_is_q_times_reconstructed_k():
    # KVSwap article §2.3.2: reconstruct_K = U diag(S) V^T; §2.2.1: scores = q K^T
    rng = np.random.default_rng(5)
    T, r, C = 200, 8, 24
    U = L.grid_uniform(rng, (T, r), lo=-0.5, hi=0.5)
    S = L.grid_uniform(rng, (r,), lo=0, hi=0.5)
    V = L.grid_uniform(rng, (C, r), lo=-0.5, hi=0.5)
    q = L.grid_uniform(rng, (C,), lo=-0.5, hi=0.5)
    K = U.astype(np.float64) @ np.diag(S.astype(np.float64)) @ V.astype(np.float64).T
    want = (K @ q.astype(np.float64)).astype(np.float32)
    got = oracle.lowrank_score(L.f32_to_f16_bits(U), S, L.f32_to_f16_bits(V), q)
    assert np.array_equal(got, want)


def test_attend_kv_is_dense_attention_one_head():
    rng = np.random.default_rng(6)
    T, H, dh = 64, 4, 16
    K = L.grid_uniform(rng, (T, H, dh), lo=-0.5, hi=0.5)
    V = L.grid_uniform(rng, (T, H, dh), lo=-0.5, hi=0.5)
    q = L.grid_uniform(rng, (dh,), lo=-0.5, hi=0.5)
    pos = np.array([0, 3, 9, 33, 63])
    h = 2
    got = oracle.attend_kv(q, L.f32_to_f16_bits(K[:, h].copy()).reshape(-1),
                           L.f32_to_f16_bits(V[:, h].copy()).reshape(-1), "f16", dh, pos, 0.25)
    z = 0.25 * (K[pos, h].astype(np.float64) @ q.astype(np.float64))
    want = softmax(z) @ V[pos, h].astype(np.float64)
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-7)
    # a row stride over all heads picks the same head
    got2 = oracle.attend_kv(q, L.f32_to_f16_bits(K[:, h:].copy()).reshape(-1),
                            L.f32_to_f16_bits(V[:, h:].copy()).reshape(-1), "f16", (H - h) * dh, pos, 0.25)
    assert np.array_equal(got, got2)
