"""HIP-graph replay of decode steps: every replay, with eager work and
synchronisations in between, gives the same bits and LRU counters as the eager
steps of an identical workload."""
import pytest
import torch

import lsa_inputs as L
from learned_sparse_kv_amd.workload import DeviceWorkload

from gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["ens_8k", "thresh_256k"])
def test_graph_replay_matches_eager(name):
    wl = L.WORKLOADS[name]
    steps = 6
    say(f"graph replay {name}")
    eager = DeviceWorkload(wl)
    eager.make_steps(steps)
    want = []
    for t in range(steps):
        eager.step(t)
        torch.cuda.synchronize()
        want.append((eager.sel.clone(), eager.count.clone(), eager.out.clone(), eager.phys.clone()))
    graphed = DeviceWorkload(wl)
    graphed.make_steps(steps)
    graphed.step(0)                      # sizes the workspace; then start from empty pools
    graphed.reset_pools()
    graphed.capture(range(steps))
    graphed.reset_pools()                # capture does not run the steps, but be explicit
    scratch = torch.zeros(1 << 20, device="cuda:0")
    for t in range(steps):
        graphed.replay(t)
        scratch.add_(1.0)                # eager work between replays
        torch.cuda.synchronize()
        sel, cnt, out, phys = want[t]
        assert torch.equal(graphed.count, cnt)
        assert torch.equal(graphed.sel, sel), f"step {t}: selection"
        assert torch.equal(graphed.phys, phys), f"step {t}: rows"
        assert torch.equal(graphed.out.view(torch.int32), out.view(torch.int32)), f"step {t}: output bits"
    for pe, pg in zip(eager.pools, graphed.pools):
        se, sg = pe.stats(), pg.stats()
        assert (se["hits"], se["misses"]) == (sg["hits"], sg["misses"])
