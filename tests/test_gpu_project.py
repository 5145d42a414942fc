"""GPU parity of the query/weight projection (lsa_project) with oracle.project:
bit-exact on grid inputs (every partial sum is exact in fp32), within an
accumulation bound on general floats."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.workload import to_device

from gpu_util import DEV, bits, say

pytestmark = pytest.mark.gpu


def run(hidden, wq, ww, wd):
    B = hidden.shape[0]
    n_idx, H, dk, _ = wq.shape
    twq = to_device(L.encode(wq, wd), wd, DEV)
    tww = to_device(L.encode(ww, wd), wd, DEV)
    q = torch.full((B, n_idx, H, dk), float("nan"), device=DEV)
    w = torch.full((B, n_idx, H), float("nan"), device=DEV)
    lsa.project(torch.from_numpy(hidden).to(DEV), twq, tww, q, w)
    return q.cpu().numpy(), w.cpu().numpy()


CASES = [
    # (B, d_model, n_idx, H, dk, weight dtype)
    (1, 4096, 3, 8, 128, "bf16"),    # the pages' hidden[4096] -> 3 indexers x 8 heads x 128
    (4, 4096, 3, 8, 128, "f32"),     # batch 4 in one launch, fp32 weights
    (5, 520, 2, 3, 64, "bf16"),      # two launches (4 + 1); 65 chunks per row: a ragged chunk round
    (2, 8, 1, 1, 1, "f32"),          # one chunk per row
    (3, 16384, 1, 2, 32, "bf16"),    # widest rows; the hidden vectors take one launch each
    (64, 1024, 1, 4, 16, "f32"),     # the largest batch
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_project_matches_oracle(case):
    B, d, n_idx, H, dk, wd = case
    say(f"project case {case}")
    rng = np.random.default_rng(hash(case) & 0xFFFF)
    hidden = L.grid_uniform(rng, (B, d))
    wq = L.grid_uniform(rng, (n_idx, H, dk, d), lo=-L.PROJ_MAX, hi=L.PROJ_MAX, step=L.PROJ_STEP)
    ww = L.grid_uniform(rng, (n_idx, H, d), lo=-L.PROJ_MAX, hi=L.PROJ_MAX, step=L.PROJ_STEP)
    q, w = run(hidden, wq, ww, wd)
    wq_o, ww_o = oracle.project(hidden, L.encode(wq, wd), L.encode(ww, wd), wd)
    assert np.array_equal(bits(q), bits(wq_o)), f"q: first diff at {np.argmax(bits(q).ravel() != bits(wq_o).ravel())}"
    assert np.array_equal(bits(w), bits(ww_o))


def test_project_general_floats_within_accumulation_bound():
    rng = np.random.default_rng(21)
    B, d, n_idx, H, dk = 2, 4096, 3, 8, 128
    hidden = rng.standard_normal((B, d)).astype(np.float32)
    wq = (rng.standard_normal((n_idx, H, dk, d)) * 0.02).astype(np.float32)
    ww = (rng.standard_normal((n_idx, H, d)) * 0.02).astype(np.float32)
    q, w = run(hidden, wq, ww, "f32")
    want_q, want_w = oracle.project(hidden, wq, ww)
    abs_q, abs_w = oracle.project(np.abs(hidden), np.abs(wq), np.abs(ww))
    # fp32 sums of d_model products: at most d_model ulps of the absolute sum
    assert np.all(np.abs(q.astype(np.float64) - want_q) <= d * 2.0 ** -24 * abs_q)
    assert np.all(np.abs(w.astype(np.float64) - want_w) <= d * 2.0 ** -24 * abs_w)


def test_projected_queries_feed_the_score():
    # the projection's (q, w) in the layout lsa_score takes: scoring with them on
    # the GPU equals scoring with the oracle's projection (same bits) on the GPU
    wl = L.WORKLOADS["ens_8k"]
    wq, ww = L.projection_weights(wl)
    hidden = np.stack([L.hidden_state(wl, 0, 0)])
    q, w = run(hidden, wq, ww, "bf16")
    oq, ow = oracle.project(hidden, wq, ww)
    assert np.array_equal(bits(q), bits(oq)) and np.array_equal(bits(w), bits(ow))
    keys = torch.from_numpy(L.indexer_keys(wl, 0)[None]).to(DEV)
    s1 = torch.zeros((1, wl.n_src), device=DEV)
    s2 = torch.zeros((1, wl.n_src), device=DEV)
    lsa.score(keys, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s1)
    lsa.score(keys, torch.from_numpy(oq).to(DEV), torch.from_numpy(ow).to(DEV), s2)
    assert torch.equal(s1, s2)
