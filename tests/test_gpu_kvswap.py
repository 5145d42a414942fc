"""GPU parity of the KVSwap variant (KVSwap article, sections 2.2-2.3 and 3.2)
with the oracle: low-rank scores bit-identical (exact on the grid), identical
top-k sets and slot rows, per-head attention within 1e-5 per row (both sides
read the same f16 values; only fp32 vs double accumulation differs)."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.kvswap_workload import DeviceKVSwap

from gpu_util import DEV, bits, rel_err_rows, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def ctx():
    return lsa.Ctx(0)


def _rand_codes(rng, shape, pts, off):
    return L.codes_to_f32(rng.integers(0, pts, size=shape, dtype=np.uint8), off)


@pytest.mark.parametrize("n_seg,T,rank,C", [(1, 1, 32, 512), (3, 2047, 32, 512), (2, 5000, 16, 256),
                                            (2, 4096, 64, 128), (5, 2048, 32, 8), (2, 300, 64, 600)])
def test_score_lowrank_bit_identical(ctx, n_seg, T, rank, C):
    say(f"score_lowrank n_seg={n_seg} T={T} rank={rank} C={C}")
    rng = np.random.default_rng(T + rank)
    U = _rand_codes(rng, (n_seg, T, rank), 8, 4)
    V = _rand_codes(rng, (n_seg, C, rank), 8, 4)
    S = _rand_codes(rng, (n_seg, rank), 8, 4) + np.float32(0.5)
    q = _rand_codes(rng, (n_seg, C), 8, 4)
    Ub, Vb = L.f32_to_f16_bits(U), L.f32_to_f16_bits(V)
    to16 = lambda a: torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.float16)
    sc = torch.full((n_seg, T), 7.0, device=DEV)
    lsa.score_lowrank(ctx, to16(Ub), torch.from_numpy(S).to(DEV), to16(Vb), torch.from_numpy(q).to(DEV), sc)
    got = sc.cpu().numpy()
    for s in range(n_seg):
        want = oracle.lowrank_score(Ub[s], S[s], Vb[s], q[s])
        assert np.array_equal(bits(got[s]), bits(want)), f"segment {s}"


@pytest.mark.parametrize("heads,dh,dtype", [(4, 128, "f16"), (1, 64, "f16"), (8, 128, "bf16"), (3, 64, "bf16")])
def test_attend_kv_matches_oracle(ctx, heads, dh, dtype):
    say(f"attend_kv heads={heads} dh={dh} {dtype}")
    rng = np.random.default_rng(heads * dh)
    n_seg, rows, stride = 6, 450, 420
    row_elems = 2 * heads * dh
    kv = _rand_codes(rng, (n_seg, rows, row_elems), 16, 8)
    enc = L.f32_to_f16_bits(kv) if dtype == "f16" else L.f32_to_bf16_bits(kv)
    tdt = torch.float16 if dtype == "f16" else torch.bfloat16
    kv_dev = torch.from_numpy(enc.view(np.int16)).to(DEV).view(tdt)
    q = rng.standard_normal((n_seg, heads, dh)).astype(np.float32)
    n_rows = np.array([0, 1, 37, 400, 420, 64], np.int32)
    phys = np.stack([rng.permutation(rows)[:stride] for _ in range(n_seg)]).astype(np.int32)
    phys[5, 3] = rows + 7          # outside the segment: reads as a zero row
    out = torch.full((n_seg, heads, dh), 9.0, device=DEV)
    lsa.attend_kv(ctx, torch.from_numpy(q).to(DEV), kv_dev, torch.from_numpy(phys).to(DEV),
                  torch.from_numpy(n_rows).to(DEV), out, 1.0 / np.sqrt(dh))
    got = out.cpu().numpy()
    zero_row = np.zeros((1, row_elems), enc.dtype)
    for s in range(n_seg):
        n = n_rows[s]
        if n == 0:
            assert np.all(got[s] == 0)
            continue
        store = np.concatenate([enc[s], zero_row])
        pos = np.where(phys[s, :n] < rows, phys[s, :n], rows).astype(np.int32)
        flat = store.reshape(-1)
        for h in range(heads):
            want = oracle.attend_kv(q[s, h], flat[h * dh:], flat[(heads + h) * dh:], dtype, row_elems, pos,
                                    1.0 / np.sqrt(dh))
            err = rel_err_rows(got[s, h], want)
            assert err <= TOL, f"segment {s} head {h}: rel err {err}"


def run_threads(fn, n):
    """fn(i) for i < n on n threads (the oracle's ctypes calls release the GIL)."""
    import threading
    errs = []

    def body(i):
        try:
            fn(i)
        except BaseException as e:
            errs.append(e)
    ths = [threading.Thread(target=body, args=(i,)) for i in range(n)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    if errs:
        raise errs[0]


def run_kvswap(wl, steps, segs=None, fused=False, period=None):
    """fused: the step gets no scores buffer (score and top-k in one launch), so
    everything but the scores is compared.  period: row j of every U is made
    row j % period, on both sides, so that each score repeats and the k-th
    largest is shared by many positions (ties to the lowest position)."""
    say(f"kvswap {wl.name}: {steps} steps, n_seg={wl.n_seg}, T={wl.ctx}, k={wl.k}, slots={wl.slots}"
        f"{', score + top-k fused' if fused else ''}")
    dw = DeviceKVSwap(wl, log=say)
    dw.make_steps(steps)
    segs = list(range(wl.n_seg)) if segs is None else sorted(segs)
    ref = oracle.KVSwapState(wl, segs)
    inputs = {}
    fold = None
    if period is not None:
        fold = np.arange(wl.ctx) % period
        dw.U.copy_(dw.U[:, torch.from_numpy(fold).to(DEV)])

    def load(i):
        U, S, V, q, cold = dw.host_inputs(segs[i], 0)
        inputs[segs[i]] = (U if fold is None else np.ascontiguousarray(U[fold]), S, V, q, cold)
    run_threads(load, len(segs))
    misses = {s: 0 for s in segs}
    hits = {s: 0 for s in segs}
    T_threads = 16
    for t in range(steps):
        dw.step(t, fused=fused)
        torch.cuda.synchronize()
        sc, sel, cnt = dw.scores.cpu().numpy(), dw.sel.cpu().numpy(), dw.count.cpu().numpy()
        phys, nrows, out = dw.phys.cpu().numpy(), dw.n_rows.cpu().numpy(), dw.out.cpu().numpy()
        wants = {}

        def one(i):
            for s in segs[i::T_threads]:
                U, S, V, _, cold = inputs[s]
                wants[s] = ref.step(s, U, S, V, dw.q_np[t, s], cold)
        run_threads(one, min(T_threads, len(segs)))
        for s in segs:
            want = wants[s]
            if not fused:
                assert np.array_equal(bits(sc[s]), bits(want["score"])), f"step {t} seg {s}: scores"
            n = want["sel"].size
            assert cnt[s] == n and np.array_equal(sel[s, :n], want["sel"]), f"step {t} seg {s}: selection"
            assert nrows[s] == n and np.array_equal(phys[s, :n], want["phys"]), f"step {t} seg {s}: slot rows"
            err = rel_err_rows(out[s], want["out"])
            assert err <= TOL, f"step {t} seg {s}: rel err {err}"
            misses[s] += len(want["misses"])
            hits[s] += n - len(want["misses"])
        say(f"  step {t} ok ({len(segs)} segments)")
    B = wl.batch
    full = 0
    for p, pool in enumerate(dw.pools):
        covered = [s for s in range(p * B, (p + 1) * B) if s in misses]
        if len(covered) == B:
            st = pool.stats()
            assert st["misses"] == sum(misses[s] for s in covered), f"pool {p} misses"
            # a pool with a slot for every position never swaps and keeps no hit count
            want_hits = sum(hits[s] for s in covered) if pool.swap else 0
            assert st["hits"] == want_hits, f"pool {p} hits"
            full += 1
    return dw, full


def test_kvswap_small_all_segments():
    _, full = run_kvswap(L.KVSWAP_WORKLOADS["kvswap_small"], 6)
    assert full == L.KVSWAP_WORKLOADS["kvswap_small"].n_pools


def test_kvswap_32k_full_size_sampled_segments():
    """The pages' shape (4096 segments, one stage launch over 256 pools): 16
    segments spread over layers, groups and sequences, plus every sequence of
    pool 171 (layer 21, group 3), whose counters are then compared too; 4 steps."""
    wl = L.KVSWAP_WORKLOADS["kvswap_32k"]
    spread = []
    i = 0
    while len(spread) < 16:
        s_ = wl.seg((i * 7 + 3) % wl.layers, (i * 3 + 1) % wl.groups, (i * 5 + 2) % wl.batch)
        if s_ not in spread:
            spread.append(s_)
        i += 1
    pool = 21 * wl.groups + 3
    segs = sorted(set(spread) | set(range(pool * wl.batch, (pool + 1) * wl.batch)))
    assert max(s // wl.batch for s in spread) > 16
    _, full = run_kvswap(wl, 4, segs)
    assert full >= 1


def test_kvswap_small_all_segments_fused():
    """Without a scores buffer the step scores and selects each segment in one
    workgroup (the scores stay in LDS): selections, slot rows, outputs and
    counters equal the oracle's."""
    _, full = run_kvswap(L.KVSWAP_WORKLOADS["kvswap_small"], 6, fused=True)
    assert full == L.KVSWAP_WORKLOADS["kvswap_small"].n_pools


def test_kvswap_32k_sampled_segments_fused():
    wl = L.KVSWAP_WORKLOADS["kvswap_32k"]
    pool = 37 * 1 + 5
    segs = sorted({wl.seg((i * 13 + 5) % wl.layers, (i * 3 + 2) % wl.groups, (i * 9 + 1) % wl.batch)
                   for i in range(16)} | set(range(pool * wl.batch, (pool + 1) * wl.batch)))
    _, full = run_kvswap(wl, 3, segs, fused=True)
    assert full >= 1


@pytest.mark.parametrize("T,k,rank,period", [(1, 4, 32, None), (301, 400, 32, None), (1023, 512, 32, None),
                                              (1024, 512, 16, None), (4097, 513, 32, None), (3001, 100, 16, None),
                                              (2500, 300, 64, None), (4097, 400, 32, 7), (2048, 512, 32, 3),
                                              (1500, 400, 32, 1), (5000, 513, 32, 11)])
def test_kvswap_fused_edge_shapes(T, k, rank, period):
    """The fused score + top-k at its edges: a single position, fewer positions
    than k (every position chosen, the pools holding every row), odd and
    ragged T, k above 512, ranks 16 and 64, and U rows repeating with a period
    (period 1: every score equal), so that the k-th largest score is shared by
    many positions and the lowest of them must be the ones chosen."""
    import dataclasses
    wl = dataclasses.replace(L.KVSWAP_WORKLOADS["kvswap_small"], name=f"kvswap_edge_{T}_{k}_{rank}",
                             base_seed=7000 + T + k + rank, ctx=T, k=k, slots=k, rank=rank, layers=1, groups=2)
    _, full = run_kvswap(wl, 2, fused=True, period=period)
    assert full == wl.n_pools


@pytest.mark.parametrize("T,k,layers", [(1500, 100, 10), (700, 64, 12), (3001, 200, 9)])
def test_kvswap_fused_more_segments_than_workgroups(T, k, layers):
    """More segments than CUs (the fused launch has one workgroup per CU, each
    taking every grid-th segment and copying the next one's first rows into
    LDS while it selects): 288-384 segments, so most workgroups take two, with
    T below, at and above one batch of rows (the copy then reads past the
    segment's end, which must read as zero and be dropped)."""
    import dataclasses
    wl = dataclasses.replace(L.KVSWAP_WORKLOADS["kvswap_small"], name=f"kvswap_many_{T}_{k}",
                             base_seed=8000 + T + k, ctx=T, k=k, slots=k, layers=layers, groups=8, batch=4)
    assert wl.n_seg > 256
    _, full = run_kvswap(wl, 2, fused=True)
    assert full == wl.n_pools


def test_kvswap_fused_refuses_a_weighted_pool(ctx):
    """A pool that weighs importance reads the step's scores, so a step without a
    scores buffer is refused before anything is enqueued."""
    wl = L.KVSWAP_WORKLOADS["kvswap_small_wr"]
    dw = DeviceKVSwap(wl, log=say)
    dw.make_steps(1)
    with pytest.raises(lsa.LsaError) as e:
        dw.step(0, fused=True)
    assert "scores buffer" in str(e.value)


def test_kvswap_small_weighted_all_segments():
    """KVSwap §3.2 rolling buffer: 400 slots, top 200 per step, replacement by
    recency and importance (the step's low-rank scores) and a 70 % high-water
    mark; every segment, slot rows and counters equal the oracle's."""
    wl = L.KVSWAP_WORKLOADS["kvswap_small_wr"]
    dw, full = run_kvswap(wl, 6)
    assert full == wl.n_pools
    for p in dw.pools:
        assert p.stats()["hits"] > 0


def test_kvswap_32k_weighted_sampled_segments():
    wl = L.KVSWAP_WORKLOADS["kvswap_32k_wr"]
    pool = 9 * wl.groups + 6
    segs = sorted({wl.seg((i * 11 + 2) % wl.layers, (i * 5 + 3) % wl.groups, (i * 7) % wl.batch) for i in range(16)}
                  | set(range(pool * wl.batch, (pool + 1) * wl.batch)))
    _, full = run_kvswap(wl, 3, segs)
    assert full >= 1
