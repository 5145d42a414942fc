"""GPU parity of kv_stage (lsa_stage) with the oracle's LRU pool: physical
rows, misses, slot table, LRU order and counters all identical; staged rows
equal their cold rows."""
import numpy as np
import pytest
import torch

import lsa_inputs as L
import oracle
from learned_sparse_kv_amd import lsa

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu
W = 16


def selections(rng, src_cap, k, steps, overlap=0.75):
    cur = np.sort(rng.choice(src_cap, size=k, replace=False))
    out = [cur]
    for _ in range(steps - 1):
        keep = cur[rng.random(cur.size) < overlap]
        n_new = int(rng.integers(0, k - keep.size + 1))
        pool = np.setdiff1d(np.arange(src_cap), keep)
        cur = np.sort(np.concatenate([keep, rng.choice(pool, size=n_new, replace=False)]))
        out.append(cur)
    return out


def make_pool(ctx_len, ratio, S, k, B, cold, D=128, dtype="f32"):
    rows = lsa.Pool.rows_needed(ctx_len, ratio, W, S)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    kv = torch.zeros((B, rows, D), dtype=tdt, device=DEV)
    return lsa.Pool(ctx_len, ratio, kv, W, S, k, D, B, cold=cold), kv


@pytest.mark.parametrize("cold", ["hbm", "host"])
@pytest.mark.parametrize("ratio", [4, 128])
def test_lru_matches_oracle(cold, ratio):
    say(f"stage parity cold={cold} ratio={ratio}")
    rng = np.random.default_rng(ratio * 7 + (cold == "host"))
    src_ratio, ctx_len, S, k, B, D = 4, 4096 if ratio == 4 else 65536, 48, 40, 2, 128
    pool, kv = make_pool(ctx_len, ratio, S, k, B, cold, D)
    assert pool.swap
    src_cap = L.compressed_cap(ctx_len, src_ratio)
    stores = []
    refs = []
    for b in range(B):
        rows = L.grid_uniform(rng, (pool.cap, D))
        pool.store(b, 0, rows)
        stores.append(rows)
        r = oracle.Pool(pool.cap, S, W, D * 4)
        r.store(0, pool.cap)
        refs.append(r)
    seqs = [selections(rng, src_cap if ratio == 4 else src_cap, k, 30) for _ in range(B)]
    sel = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    phys = torch.zeros((B, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((B,), dtype=torch.int32, device=DEV)
    for t in range(30):
        sel_np = np.full((B, k), -1, np.int32)
        for b in range(B):
            sel_np[b, :seqs[b][t].size] = seqs[b][t]
        sel.copy_(torch.from_numpy(sel_np))
        cnt.copy_(torch.tensor([seqs[b][t].size for b in range(B)], dtype=torch.int32))
        lsa.stage(pool, sel, cnt, src_ratio, phys, nrows)
        torch.cuda.synchronize()
        ph, nr = phys.cpu().numpy(), nrows.cpu().numpy()
        kvh = kv.cpu().numpy()
        for b in range(B):
            lsel = oracle.ratio_map(seqs[b][t], src_ratio, ratio)
            st, want_phys, _ = refs[b].stage(lsel)
            assert st == 0
            assert nr[b] == W + lsel.size
            assert np.array_equal(ph[b, :nr[b]], want_phys), f"step {t} seq {b}"
            sl, lru = pool.state(b)
            rsl, rlru = refs[b].state()
            assert np.array_equal(sl, rsl) and np.array_equal(lru, rlru), f"slot table step {t} seq {b}"
            # the page's KV_SWAP_VALIDATE check: every staged row is its cold row
            assert np.array_equal(kvh[b, want_phys[W:]], stores[b][lsel])
    st = pool.stats()
    want = [r.stats() for r in refs]
    assert st["hits"] == sum(x["hits"] for x in want)
    assert st["misses"] == sum(x["misses"] for x in want)
    assert st["h2d_bytes"] == sum(x["h2d_bytes"] for x in want)
    assert st["d2h_bytes"] == B * pool.cap * D * 4
    assert st["resident"] == B * S


def test_swap_disabled_is_identity_and_rows_resident():
    rng = np.random.default_rng(1)
    pool, kv = make_pool(256, 4, 64, 32, 1, "hbm", D=128, dtype="bf16")
    assert not pool.swap and pool.cap == 64
    rows = L.encode(L.grid_uniform(rng, (64, 128)), "bf16")
    pool.store(0, 0, rows)
    sel = torch.tensor([[0, 5, 63] + [-1] * 29], dtype=torch.int32, device=DEV)
    cnt = torch.tensor([3], dtype=torch.int32, device=DEV)
    phys = torch.zeros((1, W + 32), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((1,), dtype=torch.int32, device=DEV)
    lsa.stage(pool, sel, cnt, 4, phys, nrows)
    torch.cuda.synchronize()
    assert phys[0, :W + 3].tolist() == list(range(W)) + [W, W + 5, W + 63]
    assert int(nrows[0]) == W + 3
    assert np.array_equal(kv[0, W:W + 64].view(torch.int16).cpu().numpy().view(np.uint16), rows)
    assert pool.stats()["misses"] == 0


def test_not_stored_leaves_the_pool_as_the_oracle_does():
    """[P1] error 4: a list holding a never-stored entry changes nothing of that
    sequence (slot table, LRU order and counters equal the oracle's, which
    returns status 4 and keeps its state), writes an empty row list, and is
    reported once by the pool's stats; the other sequence of the pool stages as
    usual, and the failing one continues from its unchanged state."""
    B, S, k, D = 2, 16, 8, 128
    pool, kv = make_pool(1024, 4, S, k, B, "hbm", D)
    rng = np.random.default_rng(12)
    rows = [L.grid_uniform(rng, (pool.cap, D)) for _ in range(B)]
    refs = []
    for b in range(B):
        pool.store(b, 0, rows[b][:100])
        r = oracle.Pool(pool.cap, S, W, D * 4)
        r.store(0, 100)
        refs.append(r)
    sel = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    phys = torch.zeros((B, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((B,), dtype=torch.int32, device=DEV)
    steps = [[[3, 7, 9], [1, 2]], [[3, 150], [2, 60, 99]], [[7, 11, 12], [5]], [[150], [3, 4]]]
    for t, lists in enumerate(steps):
        sel_np = np.full((B, k), -1, np.int32)
        for b in range(B):
            sel_np[b, :len(lists[b])] = lists[b]
        sel.copy_(torch.from_numpy(sel_np))
        cnt.copy_(torch.tensor([len(x) for x in lists], dtype=torch.int32))
        lsa.stage(pool, sel, cnt, 4, phys, nrows)
        torch.cuda.synchronize()
        bad = False
        for b in range(B):
            st, want_phys, _ = refs[b].stage(np.array(lists[b], np.int32))
            if st != 0:
                bad = True
                assert st == oracle.ST_NOT_STORED
                assert int(nrows[b]) == 0, f"step {t} seq {b}: a failed stage lists no rows"
            else:
                assert int(nrows[b]) == W + len(lists[b])
                assert np.array_equal(phys[b, :W + len(lists[b])].cpu().numpy(), want_phys)
            sl, lru = pool.state(b)
            rsl, rlru = refs[b].state()
            assert np.array_equal(sl, rsl) and np.array_equal(lru, rlru), f"step {t} seq {b}: slot table"
        if bad:
            with pytest.raises(lsa.LsaError) as e:
                pool.stats()
            assert e.value.status == 4
        st = pool.stats()                               # the flag is cleared once reported
        assert st["hits"] == sum(r.stats()["hits"] for r in refs)
        assert st["misses"] == sum(r.stats()["misses"] for r in refs)
        assert st["h2d_bytes"] == sum(r.stats()["h2d_bytes"] for r in refs)


def test_incomplete_chunks_are_not_staged():
    """A ratio-128 layer only lists chunks whose 128 tokens are all covered by the
    valid source entries (oracle.ratio_map with src_valid); the incomplete last
    chunk is neither staged nor reported as not stored."""
    B, S, k, D = 2, 8, 8, 128
    pool, kv = make_pool(65536, 128, S, k, B, "hbm", D)     # cap 512 > 8 slots: swaps
    rng = np.random.default_rng(13)
    refs = []
    n_valid = [33, 100]                                     # chunks 0 / 0..2 complete
    for b in range(B):
        n_st = n_valid[b] * 4 // 128
        pool.store(b, 0, L.grid_uniform(rng, (n_st, D)))
        r = oracle.Pool(pool.cap, S, W, D * 4)
        r.store(0, n_st)
        refs.append(r)
    lists = [[0, 31, 32], [5, 40, 64, 96, 99]]
    sel_np = np.full((B, k), -1, np.int32)
    for b in range(B):
        sel_np[b, :len(lists[b])] = lists[b]
    sel = torch.from_numpy(sel_np).to(DEV)
    cnt = torch.tensor([len(x) for x in lists], dtype=torch.int32, device=DEV)
    phys = torch.zeros((B, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((B,), dtype=torch.int32, device=DEV)
    lsa.stage(pool, sel, cnt, 4, phys, nrows, n_valid=n_valid)
    torch.cuda.synchronize()
    for b in range(B):
        lsel = oracle.ratio_map(np.array(lists[b], np.int32), 4, 128, n_valid[b])
        st, want_phys, _ = refs[b].stage(lsel)
        assert st == 0
        assert int(nrows[b]) == W + lsel.size
        assert np.array_equal(phys[b, :W + lsel.size].cpu().numpy(), want_phys)
    assert pool.stats()["misses"] == sum(r.stats()["misses"] for r in refs) == 4


def test_topk_reduction_override():
    # page 1: GPU_CHUNKS below index_topk is refused unless the test override is set
    kv = torch.zeros((1, W + 8, 128), device=DEV)
    with pytest.raises(lsa.LsaError) as e:
        lsa.Pool(64, 4, kv, W, 8, 64, 128, 1)
    assert e.value.status == 2
    pool = lsa.Pool(64, 4, kv, W, 8, 64, 128, 1, allow_topk_reduction=True)
    assert pool.swap and pool.cap == 16


@pytest.mark.parametrize("w,h,cold", [(50, 100, "hbm"), (0, 100, "host"), (100, 70, "hbm"), (50, 70, "host"),
                                      (20, 40, "hbm")])
def test_weighted_replacement_matches_oracle(w, h, cold):
    """KVSwap §3.2 reading: eviction order weighing recency against the step's
    importance scores, and the high-water mark; slot tables, LRU order, rows and
    counters equal the oracle's after every step, then a shrink of the capacity
    (free slots in the middle of the range) equals the oracle's too."""
    say(f"weighted replacement w={w} h={h} cold={cold}")
    rng = np.random.default_rng(w * 13 + h + (cold == "host"))
    B, S, k, D, ctx_len = 2, 64, 40, 128, 4096
    pool, kv = make_pool(ctx_len, 4, S, k, B, cold, D)
    pool.set_replacement(w, h)
    stores, refs = [], []
    for b in range(B):
        rows = L.grid_uniform(rng, (pool.cap, D))
        pool.store(b, 0, rows)
        stores.append(rows)
        r = oracle.Pool(pool.cap, S, W, D * 4)
        r.store(0, pool.cap)
        r.set_replacement(w, h)
        refs.append(r)
    seqs = [selections(rng, pool.cap, k, 24, overlap=0.6) for _ in range(B)]
    sel = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    cnt = torch.zeros((B,), dtype=torch.int32, device=DEV)
    phys = torch.zeros((B, W + k), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((B,), dtype=torch.int32, device=DEV)
    imp = torch.zeros((B, pool.cap), dtype=torch.float32, device=DEV)
    for t in range(24):
        sel_np = np.full((B, k), -1, np.int32)
        imp_np = (rng.integers(0, 9, size=(B, pool.cap)) / 8).astype(np.float32)   # many ties
        for b in range(B):
            sel_np[b, :seqs[b][t].size] = seqs[b][t]
        sel.copy_(torch.from_numpy(sel_np))
        cnt.copy_(torch.tensor([seqs[b][t].size for b in range(B)], dtype=torch.int32))
        imp.copy_(torch.from_numpy(imp_np))
        lsa.stage(pool, sel, cnt, 4, phys, nrows, importance=imp if w < 100 else None)
        torch.cuda.synchronize()
        ph = phys.cpu().numpy()
        kvh = kv.cpu().numpy()
        for b in range(B):
            st, want_phys, _ = refs[b].stage(seqs[b][t], imp_np[b])
            assert st == 0
            assert np.array_equal(ph[b, :W + seqs[b][t].size], want_phys), f"step {t} seq {b}: rows"
            sl, lru = pool.state(b)
            rsl, rlru = refs[b].state()
            assert np.array_equal(sl, rsl) and np.array_equal(lru, rlru), f"step {t} seq {b}: slot table"
            assert np.array_equal(kvh[b, want_phys[W:]], stores[b][seqs[b][t]])
    st = pool.stats()
    assert st["misses"] == sum(r.stats()["misses"] for r in refs)
    assert st["hits"] == sum(r.stats()["hits"] for r in refs)
    # shrink below the used count: the oracle's reading, with free slots in the middle
    pool.set_capacity(k)
    torch.cuda.synchronize()
    kvh = kv.cpu().numpy()
    for b in range(B):
        refs[b].set_capacity(k)
        sl, lru = pool.state(b)
        rsl, rlru = refs[b].state()
        assert np.array_equal(sl, rsl) and np.array_equal(lru, rlru), f"shrink seq {b}"
        for slot in np.nonzero(rsl >= 0)[0]:
            assert np.array_equal(kvh[b, W + slot], stores[b][rsl[slot]]), f"shrink seq {b} slot {slot}: row"
