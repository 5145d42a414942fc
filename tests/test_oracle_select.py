"""Pins of oracle.select (top-k and sigmoid threshold with cap) and of the
ratio map, against brute-force ordering, the literal sigmoid, OR-mode routing
and hand cases."""
import math

import numpy as np
import pytest

import lsa_inputs as L
import oracle


def brute_topk(e, k):
    order = sorted(range(len(e)), key=lambda j: (-float(e[j]), j))
    return sorted(order[:k])


def sigmoid(x):
    return 1.0 / (1.0 + math.exp(-x)) if x >= 0 else math.exp(x) / (1.0 + math.exp(x))


@pytest.mark.parametrize("seed", range(10))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    # a coarse grid makes many ties
    e = L.grid_uniform(rng, (n,), lo=-2, hi=2, step=0.5)
    for k in (1, 3, 17, 64, n, n + 5):
        assert oracle.select(e, "topk", k).tolist() == brute_topk(e, k)


def test_topk_all_when_k_exceeds_valid():
    e = np.arange(10, dtype=np.float32)
    assert oracle.select(e, "topk", 512).tolist() == list(range(10))
    # only the valid prefix takes part
    assert oracle.select(e, "topk", 512, n_valid=4).tolist() == [0, 1, 2, 3]
    assert oracle.select(e[::-1].copy(), "topk", 2, n_valid=5).tolist() == [0, 1]


def test_signed_zeros_tie():
    e = np.array([0.0, -0.0, 0.0, -1.0, -0.0], np.float32)
    assert oracle.select(e, "topk", 2).tolist() == [0, 1]
    assert oracle.select(e, "topk", 4).tolist() == [0, 1, 2, 4]


def test_threshold_float_brackets_logit():
    for tau in (0.01, 0.3, 0.5, 0.73, 0.9, 0.999, 0.999999, 1 - 1e-12):
        tf = oracle.threshold_float(tau)
        t = math.log(tau / (1 - tau))
        assert float(tf) <= t < float(np.nextafter(tf, np.float32(np.inf)))
    assert oracle.threshold_float(0.5) == 0.0


@pytest.mark.parametrize("seed", range(6))
def test_threshold_is_literal_sigmoid(seed):
    rng = np.random.default_rng(20 + seed)
    e = L.grid_uniform(rng, (500,), lo=-8, hi=8, step=1 / 64)
    # thresholds between grid points: the literal double sigmoid decides unambiguously
    for x in (-3.0078125, -0.0078125, 0.5078125, 2.9921875, 6.0078125):
        tau = sigmoid(x)
        want = [j for j in range(e.size) if sigmoid(float(e[j])) > tau]
        cap = len(want) + 10
        assert oracle.select(e, "threshold", cap, tau).tolist() == want
        # with a binding cap: the first `cap` passing entries of the total order
        if len(want) > 3:
            got = oracle.select(e, "threshold", 3, tau).tolist()
            assert got == brute_topk(np.where(np.isin(np.arange(e.size), want), e, -np.inf), 3)


def test_threshold_half_means_positive():
    e = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0], np.float32)
    assert oracle.select(e, "threshold", 10, 0.5).tolist() == [2, 4]


def test_or_mode_routing_equals_max_threshold():
    # FlashMemory article, "Memory Indexer 放哪里": a chunk is recalled when any one
    # of the indexers deems it important.  Thresholding the max ensemble is that union.
    rng = np.random.default_rng(30)
    keys = L.grid_uniform(rng, (600, 16))
    q = L.grid_uniform(rng, (3, 4, 16))
    w = L.grid_uniform(rng, (3, 4), lo=0, hi=1)
    tau = sigmoid(3.0078125)
    union = set()
    for i in range(3):
        e_i = oracle.score(keys, "f32", q[i:i + 1], w[i:i + 1])
        union |= set(oracle.select(e_i, "threshold", 10 ** 6, tau).tolist())
    e = oracle.score(keys, "f32", q, w, "max")
    assert oracle.select(e, "threshold", 10 ** 6, tau).tolist() == sorted(union)
    assert 0 < len(union) < 600


def test_ratio_map_hand_cases():
    assert oracle.ratio_map(np.arange(128), 4, 128).tolist() == [0, 1, 2, 3]
    assert oracle.ratio_map(np.array([31, 32, 33, 95, 96]), 4, 128).tolist() == [0, 1, 2, 3]
    assert oracle.ratio_map(np.array([0, 5, 9]), 4, 4).tolist() == [0, 5, 9]
    assert oracle.ratio_map(np.array([0, 1, 2, 3, 7]), 4, 8).tolist() == [0, 1, 3]
    assert oracle.ratio_map(np.array([], np.int32), 4, 128).tolist() == []


def test_ratio_map_stays_in_layer_capacity():
    for ctx in (8192, 8191, 1000, 1048576):
        src_cap = oracle.compressed_cap(ctx, 4)
        lay_cap = oracle.compressed_cap(ctx, 128)
        m = oracle.ratio_map(np.array([0, src_cap - 1]), 4, 128)
        assert m[-1] == lay_cap - 1 and m[0] == 0


@pytest.mark.parametrize("seed", range(6))
def test_ratio_map_keeps_only_complete_chunks_by_token_enumeration(seed):
    """Brute force over tokens: a layer chunk is listed iff some selected source
    entry maps to it and every token of the chunk is covered by the valid source
    entries (tokens [0, src_valid * r_src))."""
    rng = np.random.default_rng(300 + seed)
    r_src = 4
    for r_l in (4, 8, 128):
        src_valid = int(rng.integers(0, 200))
        if src_valid == 0:
            sel = np.zeros(0, np.int32)
        else:
            sel = np.sort(rng.choice(src_valid, size=int(rng.integers(1, src_valid + 1)), replace=False))
        tokens = set(range(src_valid * r_src))
        want = []
        for m in sorted({int(j) * r_src // r_l for j in sel}):
            if all(t in tokens for t in range(m * r_l, (m + 1) * r_l)):
                want.append(m)
        got = oracle.ratio_map(sel.astype(np.int32), r_src, r_l, src_valid)
        assert got.tolist() == want, (r_l, src_valid)
    # the hand case of a ratio-128 layer: 33 source entries = 132 tokens: chunk 0
    # (tokens 0..127) exists, chunk 1 (128..255) does not yet
    assert oracle.ratio_map(np.array([0, 31, 32], np.int32), 4, 128, 33).tolist() == [0]
    assert oracle.ratio_map(np.array([0, 31, 32], np.int32), 4, 128, 64).tolist() == [0, 1]
