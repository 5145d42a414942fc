"""The allocation-free decode step (lsa_decode_step_noalloc) against the
regular one (lsa_decode_step): the same kernels on the same inputs, so the
selections, row lists, counters and outputs must be identical, bit for bit.
Two calls in a row on the library's static scratch, the second with a smaller
input, then a step too large for the scratch, which must be refused."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.workload import DeviceWorkload

from gpu_util import bits, say

pytestmark = pytest.mark.gpu


def run_pair(wl, steps, n_valid=None):
    """Two identical workloads, one stepped by each entry point; compare every step."""
    say(f"noalloc vs regular: {wl.name} B={wl.batch} N={wl.n_src} steps={steps}")
    a = DeviceWorkload(wl)
    b = DeviceWorkload(wl)
    a.make_steps(steps)
    b.make_steps(steps)
    a.n_valid = b.n_valid = n_valid
    for t in range(steps):
        a.step(t)
        lsa.decode_step_noalloc(b.ctx, **b._step_args(t))
        torch.cuda.synchronize()
        assert torch.equal(a.count, b.count), f"step {t}: counts"
        assert torch.equal(a.sel, b.sel), f"step {t}: selections"
        assert torch.equal(a.scores.view(torch.int32), b.scores.view(torch.int32)), f"step {t}: scores"
        assert torch.equal(a.n_rows, b.n_rows), f"step {t}: row counts"
        na = a.n_rows.cpu().numpy()
        pa, pb = a.phys.cpu().numpy(), b.phys.cpu().numpy()
        for l in range(wl.n_layers):
            for s in range(wl.batch):
                assert np.array_equal(pa[l, s, :na[l, s]], pb[l, s, :na[l, s]]), f"step {t} layer {l} seq {s}: rows"
        assert np.array_equal(bits(a.out.cpu().numpy()), bits(b.out.cpu().numpy())), f"step {t}: outputs"
    for pa_, pb_ in zip(a.pools, b.pools):
        assert pa_.stats() == pb_.stats()


def test_noalloc_matches_decode_step_then_smaller():
    # first the 256K threshold workload (four 65536-entry sequences: the select's
    # histogram path, whose zero region lives in the static scratch), then a
    # smaller one (2048 entries, one sequence, a swapping pool) on the same array
    run_pair(L.WORKLOADS["thresh_256k"], 3)
    run_pair(L.WORKLOADS["ens_8k"].replace(ensemble="mean"), 4, n_valid=[1900])


def test_noalloc_refuses_a_step_beyond_the_scratch():
    wl = L.WORKLOADS["ens_8k"].replace(batch=8, layer_ratios=(4,) * 16, gpu_chunks=2048)
    dw = DeviceWorkload(wl)
    dw.make_steps(1)
    dw.out.fill_(7.0)
    with pytest.raises(lsa.LsaError) as e:
        lsa.decode_step_noalloc(dw.ctx, **dw._step_args(0))
    assert e.value.status == 7 and "static scratch" in e.value.msg
    torch.cuda.synchronize()
    assert torch.all(dw.out == 7.0)      # nothing was enqueued
