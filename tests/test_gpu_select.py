"""GPU parity of fm_select (lsa_select) with oracle.select: identical index sets."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

_CTX = None


def ctx():
    global _CTX
    if _CTX is None:
        _CTX = lsa.Ctx(0)
    return _CTX


def run(e: np.ndarray, k: int, mode="topk", tau=0.5, n_valid=None):
    n_seg, N = e.shape
    st = torch.from_numpy(np.ascontiguousarray(e, np.float32)).to(DEV)
    sel = torch.full((n_seg, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((n_seg,), -7, dtype=torch.int32, device=DEV)
    lsa.select(ctx(), st, k, sel, cnt, mode, tau, n_valid)
    sel, cnt = sel.cpu().numpy(), cnt.cpu().numpy()
    for s in range(n_seg):
        nv = N if n_valid is None else n_valid[s]
        want = oracle.select(e[s], mode, k, tau, n_valid=nv)
        assert cnt[s] == want.size, f"seg {s}: count {cnt[s]} vs {want.size}"
        assert np.array_equal(sel[s, :cnt[s]], want), f"seg {s}: index sets differ"
        assert np.all(sel[s, cnt[s]:] == -1)
    return cnt


SIZES = [1, 100, 1024, 2048, 5000, 32768, 32769, 65536, 262144]


@pytest.mark.parametrize("N", SIZES)
@pytest.mark.parametrize("k", [1, 64, 512])
def test_topk_with_ties(N, k):
    say(f"select topk N={N} k={k}")
    rng = np.random.default_rng(N * 31 + k)
    e = L.grid_uniform(rng, (1, N), lo=-4, hi=4, step=0.25)   # heavy ties
    run(e, k)


@pytest.mark.parametrize("N", [2048, 65536, 262144])
def test_topk_distinct_scores(N):
    rng = np.random.default_rng(N)
    e = rng.permutation(N).astype(np.float32)[None, :] * np.float32(0.5) - np.float32(N / 4)
    run(e, 512)


def test_all_equal_scores_pick_lowest_indices():
    e = np.zeros((2, 70000), np.float32)
    e[1, ::2] = -0.0
    cnt = run(e, 512)
    assert list(cnt) == [512, 512]


def test_multi_segment_ragged():
    rng = np.random.default_rng(3)
    e = L.grid_uniform(rng, (5, 40000), lo=-2, hi=2, step=0.125)
    run(e, 512, n_valid=[0, 1, 511, 33000, 40000])
    run(e[:, :3000], 64, n_valid=[3000, 100, 0, 64, 65])


@pytest.mark.parametrize("N", [2048, 65536, 262144])
def test_threshold_mode(N):
    rng = np.random.default_rng(N + 1)
    e = L.grid_uniform(rng, (3, N), lo=-40, hi=32, step=1 / 64)
    # a few pass, about half pass (the cap binds), none pass
    for t_star in (31.0 - 1 / 128, 1 / 128, 33.0):
        tau = 1.0 / (1.0 + np.exp(-t_star))
        run(e, 512, "threshold", tau)


def test_many_segments_kvswap_shape():
    # 400 of 32768 per segment, as in the grouped KV prediction workload
    rng = np.random.default_rng(9)
    e = L.grid_uniform(rng, (64, 32768), lo=-64, hi=64, step=1 / 16)
    run(e, 400)


@pytest.mark.parametrize("N", [5000, 32768])
def test_single_workgroup_crowded_boundary_bin(N):
    # segments of one workgroup whose K-th largest key shares its top 12 bits with
    # more than 4096 others: the last two radix passes then run over the registers
    rng = np.random.default_rng(N + 7)
    e = np.zeros((4, N), np.float32)
    e[1, ::3] = 1.0                                     # a third equal, the rest below
    # distinct values in [1, 1.125): one 12-bit bin, they differ only in lower bits
    e[2] = (1.0 + rng.permutation(N).astype(np.float64) * 2.0 ** -20).astype(np.float32)
    e[3] = e[2]
    e[3, ::5] = 2.0                                     # some above the crowded bin
    for k in (1, 400, 512):
        say(f"select crowded boundary bin N={N} k={k}")
        run(e, k)
