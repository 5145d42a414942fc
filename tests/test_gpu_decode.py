"""GPU parity of whole decode steps (lsa_decode_step) with the oracle's step:
identical selected sets, physical row lists and LRU counters; attention within
1e-5 (fp32) / 2e-2 (bf16) per row.  Covers every workload at full size, in the
launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd.workload import DeviceWorkload

from gpu_util import RTOL, bits, rel_err_rows, say

pytestmark = pytest.mark.gpu


def run_decode(wl, steps, check_scores=True):
    say(f"decode {wl.name}: {steps} steps, B={wl.batch}, N={wl.n_src}, layers={wl.layer_ratios}, cold={wl.cold}")
    dw = DeviceWorkload(wl, keep_host=True)
    dw.make_steps(steps)
    ref = oracle.DecodeState(wl, dw.windows, dw.stores)
    W = wl.window
    outs = []
    for t in range(steps):
        dw.step(t)
        torch.cuda.synchronize()
        want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
        cnt = dw.count.cpu().numpy()
        sel = dw.sel.cpu().numpy()
        phys = dw.phys.cpu().numpy()
        nrows = dw.n_rows.cpu().numpy()
        out = dw.out.cpu().numpy()
        sc = dw.scores.cpu().numpy()
        for b in range(wl.batch):
            if check_scores:
                assert np.array_equal(bits(sc[b]), bits(want["scores"][b])), f"step {t} seq {b}: scores"
            assert cnt[b] == want["sel"][b].size, f"step {t} seq {b}: count"
            assert np.array_equal(sel[b, :cnt[b]], want["sel"][b]), f"step {t} seq {b}: selected set"
            for l in range(wl.n_layers):
                n = W + want["layer_sel"][l][b].size
                assert nrows[l, b] == n
                assert np.array_equal(phys[l, b, :n], want["phys"][l][b]), f"step {t} layer {l} seq {b}: rows"
                err = rel_err_rows(out[l, b], want["out"][l][b])
                assert err <= RTOL[wl.kv_dtype], f"step {t} layer {l} seq {b}: rel err {err}"
        outs.append(out)
    for l, pool in enumerate(dw.pools):
        st = pool.stats()
        want = [ref.pools[l][b].stats() for b in range(wl.batch)]
        assert st["hits"] == sum(x["hits"] for x in want), f"layer {l} hits"
        assert st["misses"] == sum(x["misses"] for x in want), f"layer {l} misses"
    say(f"decode {wl.name}: ok")
    return outs


@pytest.mark.parametrize("name,steps", [("tiny_8k", 16), ("ens_8k", 8)])
def test_decode_small_workloads(name, steps):
    run_decode(L.WORKLOADS[name], steps)


def test_decode_mean_ensemble():
    run_decode(L.WORKLOADS["ens_8k"].replace(ensemble="mean"), 4)


@pytest.mark.parametrize("kd", ["bf16", "fp8", "mxfp4", "mxint8"])
def test_decode_quantized_keys(kd):
    # indexer keys stored as bf16 or OCP fp8 E4M3 (exact for the grid values), or
    # drawn in the OCP MX formats (codes and block scales)
    run_decode(L.WORKLOADS["ens_8k"].replace(key_dtype=kd), 4)


def test_decode_forced_swap_tiny():
    # page 1 troubleshooting: 64-token context, ratio 4 -> 16 entries; 8 slots force swapping
    wl = L.WORKLOADS["tiny_8k"].replace(ctx=64, gpu_chunks=8, k=8)
    run_decode(wl, 6)


def test_decode_256k_threshold_full_size():
    run_decode(L.WORKLOADS["thresh_256k"], 2)


def test_decode_1m_host_swap_full_size():
    run_decode(L.WORKLOADS["swap_1m"], 2)


def test_swap_on_and_off_give_identical_bits():
    # page 1 phase-2: the token sequence with swap equals the baseline; the
    # attention reads the same rows in the same order either way
    wl = L.WORKLOADS["ens_8k"]
    on = DeviceWorkload(wl)
    off = DeviceWorkload(wl.replace(gpu_chunks=2048))
    assert on.pools[0].swap and not off.pools[0].swap
    on.make_steps(6)
    off.make_steps(6)
    for t in range(6):
        on.step(t)
        off.step(t)
        torch.cuda.synchronize()
        assert torch.equal(on.sel, off.sel)
        assert torch.equal(on.out.view(torch.int32), off.out.view(torch.int32)), f"step {t}"
    assert on.pools[0].stats()["misses"] > 0
