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


def test_not_stored_is_reported():
    pool, kv = make_pool(1024, 4, 16, 8, 1, "hbm")
    pool.store(0, 0, np.zeros((100, 128), np.float32))
    sel = torch.tensor([[3, 150, -1, -1, -1, -1, -1, -1]], dtype=torch.int32, device=DEV)
    cnt = torch.tensor([2], dtype=torch.int32, device=DEV)
    phys = torch.zeros((1, W + 8), dtype=torch.int32, device=DEV)
    nrows = torch.zeros((1,), dtype=torch.int32, device=DEV)
    lsa.stage(pool, sel, cnt, 4, phys, nrows)
    with pytest.raises(lsa.LsaError) as e:
        pool.stats()
    assert e.value.status == 4
    assert pool.stats()["misses"] == 2          # the flag is cleared once reported


def test_topk_reduction_override():
    # page 1: GPU_CHUNKS below index_topk is refused unless the test override is set
    kv = torch.zeros((1, W + 8, 128), device=DEV)
    with pytest.raises(lsa.LsaError) as e:
        lsa.Pool(64, 4, kv, W, 8, 64, 128, 1)
    assert e.value.status == 2
    pool = lsa.Pool(64, 4, kv, W, 8, 64, 128, 1, allow_topk_reduction=True)
    assert pool.swap and pool.cap == 16
