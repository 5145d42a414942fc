"""GPU parity of the adaptive staging capacity (lsa_pool_set_capacity,
lsa_pool_adapt) with the oracle's pool: after every capacity change and every
step the slot table, LRU order, physical rows and counters are identical, and
every used slot holds its entry's cold row (moved rows included)."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa
from learned_sparse_kv_amd.workload import DeviceWorkload

from gpu_util import DEV, check_attn, rel_err_rows, say
from test_gpu_stage import W, make_pool, selections

pytestmark = pytest.mark.gpu


def setup(rng, cold, S, k, B, ctx_len=4096, ratio=4, D=128):
    pool, kv = make_pool(ctx_len, ratio, S, k, B, cold, D)
    assert pool.swap
    stores, refs = [], []
    for b in range(B):
        rows = L.grid_uniform(rng, (pool.cap, D))
        pool.store(b, 0, rows)
        stores.append(rows)
        r = oracle.Pool(pool.cap, S, W, D * 4)
        r.store(0, pool.cap)
        refs.append(r)
    return pool, kv, stores, refs


def check(pool, kv, stores, refs, what):
    kvh = kv.cpu().numpy()
    for b, r in enumerate(refs):
        sl, lru = pool.state(b)
        rsl, rlru = r.state()
        assert np.array_equal(sl, rsl) and np.array_equal(lru, rlru), f"{what}: slot table of seq {b}"
        used = np.nonzero(sl >= 0)[0]
        assert np.array_equal(used, np.arange(used.size)), f"{what}: used slots are not a prefix"
        assert np.array_equal(kvh[b, W + used], stores[b][sl[used]]), f"{what}: a slot row is not its cold row"


def stage_all(pool, refs, seqs, t, k, phys, nrows, sel, cnt):
    B = len(refs)
    sel_np = np.full((B, k), -1, np.int32)
    for b in range(B):
        sel_np[b, :seqs[b][t].size] = seqs[b][t]
    sel.copy_(torch.from_numpy(sel_np))
    cnt.copy_(torch.tensor([seqs[b][t].size for b in range(B)], dtype=torch.int32))
    lsa.stage(pool, sel, cnt, 4, phys, nrows)
    torch.cuda.synchronize()
    ph, nr = phys.cpu().numpy(), nrows.cpu().numpy()
    for b in range(B):
        st, want, _ = refs[b].stage(seqs[b][t])
        assert st == 0 and nr[b] == W + seqs[b][t].size
        assert np.array_equal(ph[b, :nr[b]], want), f"step {t} seq {b}: rows"


@pytest.mark.parametrize("cold", ["hbm", "host"])
def test_capacity_changes_match_oracle(cold):
    say(f"capacity changes, cold={cold}")
    rng = np.random.default_rng(31 + (cold == "host"))
    S, k, B = 96, 24, 2
    pool, kv, stores, refs = setup(rng, cold, S, k, B)
    seqs = [selections(rng, pool.cap, k, 40, overlap=0.6) for _ in range(B)]
    sel = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    phys = torch.zeros((B, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((B,), dtype=torch.int32, device=DEV)
    caps = [96, 40, 24, 60, 25, 96, 30, 31]
    for t in range(40):
        if t % 5 == 4:
            C = caps[(t // 5) % len(caps)]
            pool.set_capacity(C)
            for r in refs:
                r.set_capacity(C)
            torch.cuda.synchronize()
            assert pool.capacity() == C
            check(pool, kv, stores, refs, f"after capacity {C} at step {t}")
        stage_all(pool, refs, seqs, t, k, phys, nrows, sel, cnt)
        check(pool, kv, stores, refs, f"step {t}")
    st = pool.stats()
    want = [r.stats() for r in refs]
    assert st["hits"] == sum(w["hits"] for w in want) and st["misses"] == sum(w["misses"] for w in want)
    with pytest.raises(lsa.LsaError):
        pool.set_capacity(k - 1)          # below index_topk: error 2
    with pytest.raises(lsa.LsaError):
        pool.set_capacity(S + 1)          # beyond the slots the buffer holds


def test_adapt_policy_matches_oracle():
    rng = np.random.default_rng(41)
    S, k = 128, 24
    pool, kv, stores, refs = setup(rng, "hbm", S, k, 1)
    seqs = [selections(rng, pool.cap, k, 60, overlap=0.5)]
    sel = torch.zeros((1, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((1,), dtype=torch.int32, device=DEV)
    phys = torch.zeros((1, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((1,), dtype=torch.int32, device=DEV)
    pool.set_capacity(k)
    refs[0].set_capacity(k)
    seen = set()
    for t in range(60):
        stage_all(pool, refs, seqs, t, k, phys, nrows, sel, cnt)
        if t % 3 == 2:
            # grow above 35 % misses, shrink below 20 %, 16 slots at a time
            c = pool.adapt(3, k, S, 16, grow_miss_rate=0.35, grow_h2d_bytes_per_step=1e12, shrink_miss_rate=0.2)
            rc = refs[0].adapt(0.35, 1e12, 0.2, 16, k, S, 3)
            assert c == rc == pool.capacity(), f"step {t}: capacity {c} vs oracle {rc}"
            seen.add(c)
            check(pool, kv, stores, refs, f"adapt at step {t}")
    assert len(seen) >= 3, f"the policy should move the capacity: {sorted(seen)}"


def test_decode_steps_across_a_shrink():
    # the 8K ensemble workload with 1024 slots: decode steps, a shrink to 600
    # (evicting and moving rows), more steps, then a grow back -- against the oracle
    wl = L.WORKLOADS["ens_8k"].replace(gpu_chunks=1024)
    dw = DeviceWorkload(wl, keep_host=True)
    dw.make_steps(8)
    ref = oracle.DecodeState(wl, dw.windows, dw.stores)
    swap_layers = [l for l, p in enumerate(dw.pools) if p.swap]
    assert swap_layers
    for t in range(8):
        if t in (3, 6):
            C = 600 if t == 3 else 1024
            for l in swap_layers:
                dw.pools[l].set_capacity(C)
                for r in ref.pools[l]:
                    r.set_capacity(C)
        dw.step(t)
        torch.cuda.synchronize()
        want = ref.step(dw.keys_np, dw.q_idx_np[t], dw.w_idx_np[t], dw.q_attn_np[t])
        phys, nrows, out = dw.phys.cpu().numpy(), dw.n_rows.cpu().numpy(), dw.out.cpu().numpy()
        for l in range(wl.n_layers):
            n = wl.window + want["layer_sel"][l][0].size
            assert nrows[l, 0] == n and np.array_equal(phys[l, 0, :n], want["phys"][l][0]), f"step {t} layer {l}"
            check_attn(rel_err_rows(out[l, 0], want["out"][l][0]), wl.kv_dtype, f"step {t} layer {l}")
        say(f"  step {t} ok (capacity {[dw.pools[l].capacity() for l in swap_layers]})")
