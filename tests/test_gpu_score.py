"""GPU parity of fm_score (lsa_score) with oracle.score: bit-exact on grid inputs."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.workload import to_device

from gpu_util import DEV, bits, say

pytestmark = pytest.mark.gpu


def run(keys_f32, key_dtype, q, w, ens, n_valid=None):
    B, N, dk = keys_f32.shape
    enc = np.stack([L.encode(keys_f32[b], key_dtype) for b in range(B)])
    kt = to_device(enc, key_dtype, DEV)
    scores = torch.full((B, N), float("nan"), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), scores, ens, n_valid)
    got = scores.cpu().numpy()
    for b in range(B):
        nv = N if n_valid is None else n_valid[b]
        want = oracle.score(enc[b], key_dtype, q[b], w[b], ens, n_valid=nv)
        assert np.array_equal(bits(got[b, :nv]), bits(want)), f"seq {b}: first diff at {np.argmax(bits(got[b,:nv]) != bits(want))}"
        assert np.all(np.isnan(got[b, nv:])), "entries past n_valid must not be written"


CASES = [
    # (B, N, dk, n_idx, H, key dtype, ensemble)
    (1, 2048, 64, 1, 4, "f32", "max"),      # tiny 8K workload shape
    (1, 2048, 128, 3, 8, "f32", "max"),     # 8K ensemble workload shape
    (1, 2048, 128, 3, 8, "f32", "mean"),
    (2, 4133, 128, 3, 8, "bf16", "max"),    # ragged tail, bf16 keys
    (1, 777, 32, 4, 8, "f32", "mean"),      # all 32 MFMA query rows used
    (3, 300, 64, 2, 5, "bf16", "mean"),
    (1, 1, 128, 1, 1, "f32", "max"),
    (1, 129, 128, 3, 8, "f32", "max"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_score_matches_oracle(case):
    B, N, dk, n_idx, H, kd, ens = case
    say(f"score case {case}")
    rng = np.random.default_rng(hash(case) & 0xFFFF)
    keys = L.grid_uniform(rng, (B, N, dk))
    q = L.grid_uniform(rng, (B, n_idx, H, dk))
    w = L.grid_uniform(rng, (B, n_idx, H))
    run(keys, kd, q, w, ens)


def test_ragged_n_valid_per_sequence():
    rng = np.random.default_rng(5)
    B, N, dk = 4, 300, 128
    keys = L.grid_uniform(rng, (B, N, dk))
    q = L.grid_uniform(rng, (B, 3, 8, dk))
    w = L.grid_uniform(rng, (B, 3, 8))
    run(keys, "f32", q, w, "max", n_valid=[0, 1, 129, 300])


def test_all_negative_dots_give_positive_zero():
    rng = np.random.default_rng(6)
    keys = L.grid_uniform(rng, (1, 256, 64), lo=0.125, hi=1.0)
    q = -L.grid_uniform(rng, (1, 2, 3, 64), lo=0.125, hi=1.0)
    w = -np.ones((1, 2, 3), np.float32)
    for ens in ("max", "mean"):
        kt = torch.from_numpy(keys).to(DEV)
        s = torch.full((1, 256), float("nan"), device=DEV)
        lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, ens)
        assert np.all(bits(s.cpu().numpy()) == 0)


@pytest.mark.parametrize("name", ["thresh_256k", "swap_1m"])
def test_full_size_workload_scores(name):
    wl = L.WORKLOADS[name]
    say(f"full-size score {name}: B={wl.batch} N={wl.n_src}")
    B = wl.batch
    keys = [L.indexer_keys(wl, b) for b in range(B)]
    qw = [L.indexer_query(wl, b, 0) for b in range(B)]
    q = np.stack([x[0] for x in qw])
    w = np.stack([x[1] for x in qw])
    kt = to_device(np.stack(keys), wl.key_dtype, DEV)
    s = torch.zeros((B, wl.n_src), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, wl.ensemble)
    got = s.cpu().numpy()
    for b in range(B):
        want = oracle.score(keys[b], wl.key_dtype, q[b], w[b], wl.ensemble)
        assert np.array_equal(bits(got[b]), bits(want)), f"seq {b}"
