"""GPU parity of the lookahead schedule (lsa_lookahead_prime / lsa_lookahead_step):
step t's row copy and attention share launches with the score, selection and
staging of step t+1.  Step t must give exactly the rows and the output of the
synchronous decode step t (same selection, same LRU sequence), match the oracle
within the workload's tolerance, and replay identically from HIP graphs."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.workload import DeviceWorkload

from gpu_util import check_attn, bits, rel_err_rows, say

pytestmark = pytest.mark.gpu
STEPS = 6


@pytest.fixture(scope="module")
def dw1m():
    wl = L.WORKLOADS["swap_1m"]
    say(f"lookahead {wl.name}: building")
    dw = DeviceWorkload(wl, keep_host=True)
    dw.make_steps(STEPS + 2)
    return dw


def test_lookahead_matches_oracle_and_sync_steps(dw1m):
    dw, wl = dw1m, dw1m.wl
    ref = oracle.DecodeState(wl, dw.windows, dw.stores)
    dw.reset_pools()
    dw.lookahead_prime(0)
    outs = []
    for t in range(STEPS):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
        phys = dw.phys2[cur].cpu().numpy()
        nrows = dw.n_rows2[cur].cpu().numpy()
        out = dw.out.cpu().numpy()
        for l in range(wl.n_layers):
            n = wl.window + want["layer_sel"][l][0].size
            assert nrows[l, 0] == n, f"step {t} layer {l}: row count"
            assert np.array_equal(phys[l, 0, :n], want["phys"][l][0]), f"step {t} layer {l}: rows"
            err = rel_err_rows(out[l, 0], want["out"][l][0])
            check_attn(err, wl.kv_dtype, f"step {t} layer {l}")
        outs.append(out.copy())
        say(f"  lookahead step {t} ok")
    # the GPU staged one step ahead: after STEPS + 1 selections the LRU counters agree
    ref.step(dw.keys_np, dw.q_idx_np[STEPS], dw.w_idx_np[STEPS], dw.q_attn_np[STEPS])
    for l, pool in enumerate(dw.pools):
        st, want = pool.stats(), ref.pools[l][0].stats()
        assert (st["hits"], st["misses"]) == (want["hits"], want["misses"]), f"layer {l} counters"
    # the synchronous schedule from the same pool state gives the same bits
    dw.reset_pools()
    for t in range(STEPS):
        dw.step(t)
        torch.cuda.synchronize()
        assert np.array_equal(bits(dw.out.cpu().numpy()), bits(outs[t])), f"step {t}: sync vs lookahead bits"


def test_lookahead_graph_replay_matches_eager(dw1m):
    dw = dw1m
    dw.reset_pools()
    dw.lookahead_prime(0)
    eager = []
    for t in range(STEPS):
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        eager.append(bits(dw.out.cpu().numpy()).copy())
    # capture the same steps, then replay them from the same starting state
    dw.reset_pools()
    dw.lookahead_prime(0)
    torch.cuda.synchronize()
    dw.capture_lookahead(range(STEPS))
    for rep in range(2):
        if rep:
            dw.reset_pools()
            dw.lookahead_prime(0)
            torch.cuda.synchronize()
        for t in range(STEPS):
            dw.replay(t)
            torch.cuda.synchronize()
            assert np.array_equal(bits(dw.out.cpu().numpy()), eager[t]), f"replay {rep} step {t}"
            # eager work between replays
            _ = dw.out.sum().item()
        say(f"  replay {rep} ok")


def test_lookahead_fp8_keys_give_the_f32_bits(dw1m):
    # the same grid keys stored as fp8 E4M3 score to the same bits on the bf16
    # MFMA path, so the schedule stages the same rows and attends identically
    fp8 = DeviceWorkload(L.WORKLOADS["swap_1m_fp8"])
    fp8.make_steps(STEPS + 2)
    runs = []
    for dw in (dw1m, fp8):
        dw.reset_pools()
        dw.lookahead_prime(0)
        res = []
        for t in range(4):
            cur = lsa.lookahead_buffer(dw.ctx)
            dw.lookahead_step(t)
            torch.cuda.synchronize()
            phys, nr = dw.phys2[cur].cpu().numpy(), dw.n_rows2[cur].cpu().numpy()
            # a row list is defined up to its count; entries past it are stale
            rows = [phys[l, 0, :nr[l, 0]].copy() for l in range(phys.shape[0])]
            res.append((rows, nr.copy(), bits(dw.out.cpu().numpy()).copy(), bits(dw.scores.cpu().numpy()).copy()))
        runs.append(res)
    for t in range(4):
        a, b = runs[0][t], runs[1][t]
        assert np.array_equal(a[1], b[1]), f"step {t}: row counts"
        assert all(np.array_equal(x, y) for x, y in zip(a[0], b[0])), f"step {t}: rows"
        assert np.array_equal(a[2], b[2]), f"step {t}: output"
        assert np.array_equal(a[3], b[3]), f"step {t}: scores"
    say("  fp8 lookahead ok")


def _key_policy_runs(dw, n=4):
    """n lookahead steps, then n synchronous steps, with the default and with the
    non-temporal key policy: (rows, output bits, score bits) per call."""
    runs = []
    try:
        for nt in (False, True):
            dw.ctx.set_key_policy(nt)
            res = []
            dw.reset_pools()
            dw.lookahead_prime(0)
            for t in range(n):
                cur = lsa.lookahead_buffer(dw.ctx)
                dw.lookahead_step(t)
                torch.cuda.synchronize()
                phys, nr = dw.phys2[cur].cpu().numpy(), dw.n_rows2[cur].cpu().numpy()
                rows = [phys[l, b, :nr[l, b]].copy() for l in range(phys.shape[0]) for b in range(phys.shape[1])]
                res.append((rows, bits(dw.out.cpu().numpy()).copy(), bits(dw.scores.cpu().numpy()).copy()))
            dw.reset_pools()
            for t in range(n):
                dw.step(t)
                torch.cuda.synchronize()
                res.append(([], bits(dw.out.cpu().numpy()).copy(), bits(dw.scores.cpu().numpy()).copy()))
            runs.append(res)
    finally:
        dw.ctx.set_key_policy(False)
    for i, (a, b) in enumerate(zip(*runs)):
        assert len(a[0]) == len(b[0]) and all(np.array_equal(x, y) for x, y in zip(a[0], b[0])), f"call {i}: rows"
        assert np.array_equal(a[1], b[1]), f"call {i}: output"
        assert np.array_equal(a[2], b[2]), f"call {i}: scores"


def test_key_policy_gives_the_same_bits(dw1m):
    # the non-temporal key loads of the step calls (lsa_ctx_set_key_policy) change
    # only how the keys pass the caches: scores, rows and outputs keep their bits
    # in both schedules (fp32 keys, one sequence, pinned-host cold pools)
    _key_policy_runs(dw1m)
    say("  key policy (swap_1m): same bits in both schedules")


def test_key_policy_gives_the_same_bits_bf16_batched():
    # bf16 keys and rows, four sequences, threshold mode, swapping HBM cold pools
    wl = L.WORKLOADS["thresh_256k"].replace(gpu_chunks=1024)
    dw = DeviceWorkload(wl)
    dw.make_steps(6)
    _key_policy_runs(dw)
    say("  key policy (thresh_256k, 1024 slots): same bits in both schedules")


def test_lookahead_small_workloads_match_oracle():
    # 512 slots for top-512 (the stage of t+1 runs after step t's attention) and the
    # single-workgroup select path; the tiny workload is fully resident
    for wl in (L.WORKLOADS["ens_8k"], L.WORKLOADS["tiny_8k"], L.WORKLOADS["ens_8k"].replace(key_dtype="mxfp4"),
               L.WORKLOADS["ens_8k"].replace(key_dtype="mxint8")):
        name = f"{wl.name}/{wl.key_dtype}"
        dw = DeviceWorkload(wl, keep_host=True)
        dw.make_steps(6)
        ref = oracle.DecodeState(wl, dw.windows, dw.stores)
        dw.lookahead_prime(0)
        for t in range(4):
            dw.lookahead_step(t)
            torch.cuda.synchronize()
            want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
            out = dw.out.cpu().numpy()
            for l in range(wl.n_layers):
                err = rel_err_rows(out[l, 0], want["out"][l][0])
                check_attn(err, wl.kv_dtype, f"{name} step {t} layer {l}")
        say(f"  {name} lookahead ok")


@pytest.mark.parametrize("slots", [None, 1024])
def test_lookahead_batched_threshold_matches_sync(slots):
    # four sequences of 65536 entries: the select histogram built by the score
    # launch for several sequences, threshold mode, bf16 rows, and the batched
    # indexing of the fused launches; with 1024 slots both layers also swap (from
    # HBM cold pools), so the copy has misses
    wl = L.WORKLOADS["thresh_256k"]
    if slots is not None:
        wl = wl.replace(gpu_chunks=slots)
    dw = DeviceWorkload(wl)
    dw.make_steps(6)
    n = 4
    sync_out, sync_phys = [], []
    dw.reset_pools()
    for t in range(n):
        dw.step(t)
        torch.cuda.synchronize()
        sync_out.append(bits(dw.out.cpu().numpy()).copy())
        sync_phys.append((dw.phys.cpu().numpy().copy(), dw.n_rows.cpu().numpy().copy()))
    sync_stats = [p.stats() for p in dw.pools]
    dw.reset_pools()
    dw.lookahead_prime(0)
    for t in range(n):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        phys, nrows = dw.phys2[cur].cpu().numpy(), dw.n_rows2[cur].cpu().numpy()
        want_phys, want_nrows = sync_phys[t]
        assert np.array_equal(nrows, want_nrows), f"step {t}: row counts"
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                m = int(nrows[l, b])
                assert np.array_equal(phys[l, b, :m], want_phys[l, b, :m]), f"step {t} layer {l} seq {b}: rows"
        assert np.array_equal(bits(dw.out.cpu().numpy()), sync_out[t]), f"step {t}: lookahead vs sync bits"
    # the lookahead staged step n as well: its counters are one step ahead
    if slots is not None:
        la_stats = [p.stats() for p in dw.pools]
        assert sum(s["misses"] for s in la_stats) >= sum(s["misses"] for s in sync_stats) > 0
    say(f"  thresh_256k slots={slots}: lookahead = sync over {n} steps")


def test_lookahead_separate_histogram_matches_sync():
    """Four sequences of a 65536-entry key array with only a few dozen valid
    entries each: the score launch has fewer workgroups than sequences, so the
    select histogram runs as its own launch; rows and output bits equal the
    synchronous steps'."""
    wl = L.WORKLOADS["thresh_256k"].replace(mode="topk", k=32)
    dw = DeviceWorkload(wl)
    dw.make_steps(6)
    dw.n_valid = [40, 64, 100, 33]
    sync = []
    for t in range(4):
        dw.step(t)
        torch.cuda.synchronize()
        sync.append((bits(dw.out.cpu().numpy()).copy(), dw.phys.cpu().numpy().copy(), dw.n_rows.cpu().numpy().copy()))
    dw.lookahead_prime(0)
    for t in range(4):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        out, phys, nrows = sync[t]
        got_n = dw.n_rows2[cur].cpu().numpy()
        assert np.array_equal(got_n, nrows), f"step {t}: row counts"
        got_p = dw.phys2[cur].cpu().numpy()
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                m = int(nrows[l, b])
                assert np.array_equal(got_p[l, b, :m], phys[l, b, :m]), f"step {t} layer {l} seq {b}"
        assert np.array_equal(bits(dw.out.cpu().numpy()), out), f"step {t}: lookahead vs sync bits"
    say("  separate-histogram lookahead = sync")


@pytest.mark.parametrize("period", [1, 2, 4])
def test_lookahead_periodic_indexer(period):
    """[P2] periodic indexer in the lookahead schedule: the last step of each
    window attends and predicts the next window (lsa_lookahead_step with the
    next window's indexer query), the other steps only attend
    (lsa_lookahead_attend).  Rows and outputs equal the oracle's periodic chain
    and, bit for bit, the synchronous periodic schedule."""
    wl = L.WORKLOADS["ens_8k"]
    steps = 8
    dw = DeviceWorkload(wl, keep_host=True)
    dw.make_steps(steps + 1)
    ref = oracle.DecodeState(wl, dw.windows, dw.stores)
    la = []
    dw.lookahead_prime(0)
    for t in range(steps):
        want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t], predict=t % period == 0)
        cur = lsa.lookahead_buffer(dw.ctx)
        if (t + 1) % period == 0:
            dw.lookahead_step(t, t_next=t + 1)
        else:
            dw.lookahead_attend(t)
        torch.cuda.synchronize()
        phys, nrows, out = dw.phys2[cur].cpu().numpy(), dw.n_rows2[cur].cpu().numpy(), dw.out.cpu().numpy()
        for l in range(wl.n_layers):
            n = wl.window + want["layer_sel"][l][0].size
            assert nrows[l, 0] == n, f"step {t} layer {l}: row count"
            if want["phys"][l][0] is not None:
                assert np.array_equal(phys[l, 0, :n], want["phys"][l][0]), f"step {t} layer {l}: rows"
            err = rel_err_rows(out[l, 0], want["out"][l][0])
            check_attn(err, wl.kv_dtype, f"step {t} layer {l}")
        la.append(bits(out).copy())
    # the synchronous periodic schedule from fresh pools gives the same bits
    dw.reset_pools()
    for t in range(steps):
        if t % period == 0:
            dw.step(t)
        else:
            dw.attend(t)
        torch.cuda.synchronize()
        assert np.array_equal(bits(dw.out.cpu().numpy()), la[t]), f"step {t}: sync vs lookahead bits"
    say(f"  periodic lookahead, period {period}: ok")


def test_store_while_decoding_lookahead():
    from test_gpu_decode import growing_run
    growing_run("lookahead")


def test_lookahead_weighted_replacement():
    """The rolling-buffer replacement in the lookahead schedule (the stage of step
    t+1 reads the scores that predict it): rows and outputs equal the oracle's."""
    wl = L.WORKLOADS["ens_8k_wr"]
    dw = DeviceWorkload(wl, keep_host=True)
    dw.make_steps(8)
    ref = oracle.DecodeState(wl, dw.windows, dw.stores)
    dw.lookahead_prime(0)
    for t in range(6):
        want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        phys, nrows, out = dw.phys2[cur].cpu().numpy(), dw.n_rows2[cur].cpu().numpy(), dw.out.cpu().numpy()
        for l in range(wl.n_layers):
            n = wl.window + want["layer_sel"][l][0].size
            assert nrows[l, 0] == n and np.array_equal(phys[l, 0, :n], want["phys"][l][0]), f"step {t} layer {l}"
            err = rel_err_rows(out[l, 0], want["out"][l][0])
            check_attn(err, wl.kv_dtype, f"step {t} layer {l}")


def test_lookahead_41_layer_stack_matches_sync():
    """The 41-layer stack in the lookahead schedule (the row copy covers every
    layer, attention and stage run per group of layers): rows and output bits
    equal the synchronous schedule's."""
    wl = L.WORKLOADS["stack_64k_41"]
    dw = DeviceWorkload(wl)
    dw.make_steps(6)
    sync = []
    for t in range(4):
        dw.step(t)
        torch.cuda.synchronize()
        sync.append((bits(dw.out.cpu().numpy()).copy(), dw.phys.cpu().numpy().copy(), dw.n_rows.cpu().numpy().copy()))
    dw.reset_pools()
    dw.lookahead_prime(0)
    for t in range(4):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        out, phys, nrows = sync[t]
        assert np.array_equal(dw.n_rows2[cur].cpu().numpy(), nrows), f"step {t}: row counts"
        got_p = dw.phys2[cur].cpu().numpy()
        for l in range(wl.n_layers):
            m = int(nrows[l, 0])
            assert np.array_equal(got_p[l, 0, :m], phys[l, 0, :m]), f"step {t} layer {l}"
        assert np.array_equal(bits(dw.out.cpu().numpy()), out), f"step {t}: lookahead vs sync bits"


def test_lookahead_batched_topk_matches_sync_over_16_steps():
    """Four sequences of 65536 entries (64 select collect blocks each), top-512,
    over 16 steps: the final selection of every sequence runs beside the
    attention splits; rows and output bits equal the synchronous schedule's."""
    wl = L.WORKLOADS["thresh_256k"].replace(mode="topk", k=512)
    n = 16
    dw = DeviceWorkload(wl)
    dw.make_steps(n + 2)
    sync = []
    for t in range(n):
        dw.step(t)
        torch.cuda.synchronize()
        sync.append((bits(dw.out.cpu().numpy()).copy(), dw.phys.cpu().numpy().copy(), dw.n_rows.cpu().numpy().copy()))
    dw.reset_pools()
    dw.lookahead_prime(0)
    for t in range(n):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        out, phys, nrows = sync[t]
        assert np.array_equal(dw.n_rows2[cur].cpu().numpy(), nrows), f"step {t}: row counts"
        got_p = dw.phys2[cur].cpu().numpy()
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                m = int(nrows[l, b])
                assert np.array_equal(got_p[l, b, :m], phys[l, b, :m]), f"step {t} layer {l} seq {b}"
        assert np.array_equal(bits(dw.out.cpu().numpy()), out), f"step {t}: lookahead vs sync bits"
    say(f"  batched top-512: lookahead = sync over {n} steps")


@pytest.mark.parametrize("mode", ["topk", "threshold"])
def test_lookahead_candidate_guess_fallback(mode):
    """The score launch lists candidates from a bin guessed by the previous
    step's final selection.  Head weights scaled by 1/16 or 16 between steps move
    the boundary bin by 16 bins either way: a guess above the new boundary, or
    one that lists too many entries, must fall back to the exact scan.  Rows
    and output bits equal the synchronous steps' throughout."""
    wl = L.WORKLOADS["thresh_256k"]
    if mode == "topk":
        wl = wl.replace(mode="topk", k=512)
    n = 8
    dw = DeviceWorkload(wl)
    dw.make_steps(n + 2)
    for t, f in enumerate([1.0, 1 / 16, 1.0, 16.0, 16.0, 1 / 16, 1.0, 1.0, 16.0, 1.0]):
        dw.w_idx[t] *= f
    sync = []
    for t in range(n):
        dw.step(t)
        torch.cuda.synchronize()
        sync.append((bits(dw.out.cpu().numpy()).copy(), dw.phys.cpu().numpy().copy(), dw.n_rows.cpu().numpy().copy()))
    dw.reset_pools()
    dw.lookahead_prime(0)
    for t in range(n):
        cur = lsa.lookahead_buffer(dw.ctx)
        dw.lookahead_step(t)
        torch.cuda.synchronize()
        out, phys, nrows = sync[t]
        assert np.array_equal(dw.n_rows2[cur].cpu().numpy(), nrows), f"step {t}: row counts"
        got_p = dw.phys2[cur].cpu().numpy()
        for l in range(wl.n_layers):
            for b in range(wl.batch):
                m = int(nrows[l, b])
                assert np.array_equal(got_p[l, b, :m], phys[l, b, :m]), f"step {t} layer {l} seq {b}"
        assert np.array_equal(bits(dw.out.cpu().numpy()), out), f"step {t}: lookahead vs sync bits"
    say(f"  {mode}: guessed candidate lists with scaled steps = sync over {n} steps")
