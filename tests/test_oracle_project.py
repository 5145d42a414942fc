"""Pins of oracle.project (the indexers' query/weight projection of the hidden
state) against exact rational brute force, one-hot weights, linearity and a
float64 library matrix product."""
from fractions import Fraction

import numpy as np
import pytest

import lsa_inputs as L
import oracle


def round_f32(x: Fraction) -> np.float32:
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def brute(hidden, wq, ww):
    B, d = hidden.shape
    n_idx, H, dk, _ = wq.shape
    q = np.zeros((B, n_idx, H, dk), np.float32)
    w = np.zeros((B, n_idx, H), np.float32)
    for b in range(B):
        x = [Fraction(float(v)) for v in hidden[b]]
        for i in range(n_idx):
            for h in range(H):
                for t in range(dk):
                    q[b, i, h, t] = round_f32(sum(Fraction(float(wq[i, h, t, c])) * x[c] for c in range(d)))
                w[b, i, h] = round_f32(sum(Fraction(float(ww[i, h, c])) * x[c] for c in range(d)))
    return q, w


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_grid(seed):
    rng = np.random.default_rng(seed)
    B, d, n_idx, H, dk = (int(v) for v in (rng.integers(1, 4), rng.integers(1, 20), rng.integers(1, 4),
                                           rng.integers(1, 4), rng.integers(1, 6)))
    hidden = L.grid_uniform(rng, (B, d))
    wq = L.grid_uniform(rng, (n_idx, H, dk, d), lo=-L.PROJ_MAX, hi=L.PROJ_MAX, step=L.PROJ_STEP)
    ww = L.grid_uniform(rng, (n_idx, H, d), lo=-L.PROJ_MAX, hi=L.PROJ_MAX, step=L.PROJ_STEP)
    q, w = oracle.project(hidden, wq, ww)
    bq, bw = brute(hidden, wq, ww)
    assert np.array_equal(q, bq) and np.array_equal(w, bw)


def test_brute_force_general_floats():
    rng = np.random.default_rng(11)
    hidden = rng.standard_normal((2, 9)).astype(np.float32)
    wq = rng.standard_normal((2, 2, 3, 9)).astype(np.float32)
    ww = rng.standard_normal((2, 2, 9)).astype(np.float32)
    q, w = oracle.project(hidden, wq, ww)
    bq, bw = brute(hidden, wq, ww)
    # double accumulation of 9 exact products, one rounding to float: within an ulp
    assert np.allclose(q, bq, rtol=2 ** -23, atol=0) and np.allclose(w, bw, rtol=2 ** -23, atol=0)


def test_one_hot_weights_pick_hidden_elements():
    rng = np.random.default_rng(12)
    d, n_idx, H, dk = 64, 2, 3, 5
    hidden = L.grid_uniform(rng, (3, d))
    pick = rng.integers(0, d, size=(n_idx, H, dk))
    wq = np.zeros((n_idx, H, dk, d), np.float32)
    for i in range(n_idx):
        for h in range(H):
            for t in range(dk):
                wq[i, h, t, pick[i, h, t]] = 1.0
    pw = rng.integers(0, d, size=(n_idx, H))
    ww = np.zeros((n_idx, H, d), np.float32)
    for i in range(n_idx):
        for h in range(H):
            ww[i, h, pw[i, h]] = -2.0
    q, w = oracle.project(hidden, wq, ww)
    assert np.array_equal(q, hidden[:, pick])
    assert np.array_equal(w, -2.0 * hidden[:, pw])


def test_linear_in_the_hidden_state():
    rng = np.random.default_rng(13)
    wl = L.WORKLOADS["ens_8k"]
    wq, ww = L.projection_weights(wl, d_model=256)
    h1 = L.grid_uniform(rng, (2, 256))
    h2 = L.grid_uniform(rng, (2, 256))
    q1, w1 = oracle.project(h1, wq, ww)
    q2, w2 = oracle.project(h2, wq, ww)
    q3, w3 = oracle.project(h1 + 2.0 * h2, wq, ww)
    assert np.array_equal(q3, q1 + 2.0 * q2) and np.array_equal(w3, w1 + 2.0 * w2)


def test_float64_matrix_product_and_row_layout():
    # a library product in float64 over the flattened weight rows gives the same floats
    rng = np.random.default_rng(14)
    wl = L.WORKLOADS["swap_1m"]
    wq, ww = L.projection_weights(wl, d_model=512)
    hidden = L.grid_uniform(rng, (3, 512))
    q, w = oracle.project(hidden, wq, ww)
    mq = (wq.reshape(-1, 512).astype(np.float64) @ hidden.T.astype(np.float64)).T.astype(np.float32)
    mw = (ww.reshape(-1, 512).astype(np.float64) @ hidden.T.astype(np.float64)).T.astype(np.float32)
    assert np.array_equal(q.reshape(3, -1), mq) and np.array_equal(w.reshape(3, -1), mw)


def test_bf16_weights_decode_and_sequences_independent():
    rng = np.random.default_rng(15)
    wl = L.WORKLOADS["tiny_8k"]
    wq, ww = L.projection_weights(wl, d_model=128)
    hidden = L.grid_uniform(rng, (4, 128))
    q, w = oracle.project(hidden, wq, ww)
    qb, wb = oracle.project(hidden, L.f32_to_bf16_bits(wq), L.f32_to_bf16_bits(ww), "bf16")
    assert np.array_equal(q, qb) and np.array_equal(w, wb)
    for b in range(4):
        q1, w1 = oracle.project(hidden[b:b + 1], wq, ww)
        assert np.array_equal(q1[0], q[b]) and np.array_equal(w1[0], w[b])
