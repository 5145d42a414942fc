"""GPU parity of fm_score (lsa_score) with oracle.score: bit-exact on grid inputs."""
import zlib

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
    (2, 4133, 128, 3, 8, "fp8", "max"),     # fp8 keys, ragged tail
    (3, 300, 64, 2, 5, "fp8", "mean"),
    (1, 777, 32, 4, 8, "fp8", "max"),
    (1, 1, 128, 1, 1, "fp8", "max"),
    (1, 129, 128, 3, 8, "fp8", "mean"),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_score_matches_oracle(case):
    B, N, dk, n_idx, H, kd, ens = case
    say(f"score case {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    keys = L.grid_uniform(rng, (B, N, dk))
    q = L.grid_uniform(rng, (B, n_idx, H, dk))
    w = L.grid_uniform(rng, (B, n_idx, H))
    run(keys, kd, q, w, ens)


@pytest.mark.parametrize("kd", ["f32", "bf16", "fp8"])
def test_ragged_n_valid_per_sequence(kd):
    rng = np.random.default_rng(5)
    B, N, dk = 4, 300, 128
    keys = L.grid_uniform(rng, (B, N, dk))
    q = L.grid_uniform(rng, (B, 3, 8, dk))
    w = L.grid_uniform(rng, (B, 3, 8))
    run(keys, kd, q, w, "max", n_valid=[0, 1, 129, 300])


@pytest.mark.parametrize("dk", [32, 128])
def test_fp8_every_code_in_every_column(dk):
    """Each finite E4M3 code in each key column, alone in its key: with the
    query all ones in two heads of weight +1 and -1 (second query negated),
    score = ReLU(k) - ReLU(-k) = the decoded code, +0 for either zero."""
    import torch as _t
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    n = codes.size * dk
    keys = np.zeros((1, n, dk), np.uint8)
    idx = np.arange(n)
    keys[0, idx, idx % dk] = codes[idx // dk]
    q = np.stack([np.ones(dk, np.float32), -np.ones(dk, np.float32)])[None, None]
    w = np.array([[[1.0, -1.0]]], np.float32)
    kt = torch.from_numpy(keys).to(DEV).view(torch.float8_e4m3fn)
    s = torch.full((1, n), float("nan"), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, "max")
    got = s.cpu().numpy()[0]
    want = oracle.score(keys[0], "fp8", q[0], w[0], "max")
    assert np.array_equal(bits(got), bits(want))
    dec = _t.from_numpy(codes[idx // dk]).view(_t.float8_e4m3fn).float().numpy() + np.float32(0)
    assert np.array_equal(got, dec)


@pytest.mark.parametrize("mix", ["all", "some"])
def test_fp32_keys_beyond_bf16_precision(mix):
    """fp32 keys with full 24-bit significands (all keys, or a few scattered among
    grid keys): within the fp32 accumulation bound of the exact score, and the
    grid keys around them stay bit-exact."""
    rng = np.random.default_rng(9 if mix == "all" else 10)
    B, N, dk, n_idx, H = 1, 3000, 128, 3, 8
    keys = L.grid_uniform(rng, (N, dk))
    if mix == "all":
        keys = rng.standard_normal((N, dk)).astype(np.float32)
    else:
        rows = rng.choice(N, size=40, replace=False)
        keys[rows, rng.integers(0, dk, size=40)] = rng.standard_normal(40).astype(np.float32)
    q = L.grid_uniform(rng, (B, n_idx, H, dk))
    w = L.grid_uniform(rng, (B, n_idx, H))
    s = torch.zeros((B, N), device=DEV)
    lsa.score(torch.from_numpy(keys[None]).to(DEV), torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s)
    got = s.cpu().numpy()[0].astype(np.float64)
    want = oracle.score(keys, "f32", q[0], w[0], "max").astype(np.float64)
    absum = oracle.score(np.abs(keys), "f32", np.abs(q[0]), np.abs(w[0]), "max").astype(np.float64)
    assert np.all(np.abs(got - want) <= 2 * dk * 2.0 ** -24 * absum + 1e-30)
    if mix == "some":
        grid_rows = np.setdiff1d(np.arange(N), rows)
        assert np.array_equal(bits(got.astype(np.float32)[grid_rows]), bits(want.astype(np.float32)[grid_rows]))


@pytest.mark.parametrize("kd", ["bf16", "fp8"])
def test_general_fp32_query_split_is_exact_per_product(kd):
    """bf16 and fp8 keys meet a query of arbitrary fp32 values (not grid values),
    which the kernel splits into three bf16 parts: every product is exact, so the
    result differs from the exact score only by fp32 accumulation rounding."""
    rng = np.random.default_rng(8)
    B, N, dk, n_idx, H = 1, 1000, 128, 3, 8
    keys = L.grid_uniform(rng, (B, N, dk))
    q = rng.standard_normal((B, n_idx, H, dk)).astype(np.float32)
    w = rng.random((B, n_idx, H)).astype(np.float32)
    enc = L.encode(keys[0], kd)
    kt = to_device(enc[None], kd, DEV)
    s = torch.zeros((B, N), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, "max")
    got = s.cpu().numpy()[0].astype(np.float64)
    want = oracle.score(enc, kd, q[0], w[0], "max").astype(np.float64)
    # bound: 2 * dk ulps of the absolute-value score, per indexer
    absum = oracle.score(np.abs(keys[0]), "f32", np.abs(q[0]), w[0], "max").astype(np.float64)
    assert np.all(np.abs(got - want) <= 2 * dk * 2.0 ** -24 * absum + 1e-30)
    # and grid queries and weights (exact split: mid = lo = 0; exact sums) are bit-exact
    qg = L.grid_uniform(rng, (B, n_idx, H, dk))
    wg = L.grid_uniform(rng, (B, n_idx, H))
    lsa.score(kt, torch.from_numpy(qg).to(DEV), torch.from_numpy(wg).to(DEV), s, "max")
    assert np.array_equal(bits(s.cpu().numpy()[0]), bits(oracle.score(enc, kd, qg[0], wg[0], "max")))


def test_mean_ensemble_rounds_the_indexer_sum_once():
    """Indexer scores 1, 2^-24 and 2^-24 (one head each, exact products): the
    float sum taken once is 1 + 2^-23, while two float adds in a row would give
    1; the mean is that sum divided once by 3, exactly as the oracle computes
    it (and not fl(fl(1 + 2^-24) + 2^-24) / 3)."""
    dk, N = 128, 64
    keys = np.zeros((1, N, dk), np.float32)
    keys[0, :, 0] = 1.0
    keys[0, 1::2, 0] = 0.5
    q = np.zeros((1, 3, 1, dk), np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 1, 0, 0] = 2.0 ** -24
    q[0, 2, 0, 0] = 2.0 ** -24
    w = np.ones((1, 3, 1), np.float32)
    s = torch.zeros((1, N), device=DEV)
    lsa.score(torch.from_numpy(keys).to(DEV), torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, "mean")
    got = s.cpu().numpy()[0]
    want = oracle.score(keys[0], "f32", q[0], w[0], "mean")
    assert np.array_equal(bits(got), bits(want))
    assert got[0] == np.float32(np.float32(1 + 2.0 ** -23) / np.float32(3))
    assert got[0] != np.float32(np.float32(np.float32(1 + 2.0 ** -24) + np.float32(2.0 ** -24)) / np.float32(3))


@pytest.mark.parametrize("kd", ["f32", "bf16"])
def test_mean_ensemble_off_grid(kd):
    """Mean ensemble with arbitrary fp32 queries and weights (and full-precision
    fp32 keys): within the fp32 accumulation bound of the oracle's score, per
    indexer, with the sum of the indexer scores rounded once."""
    rng = np.random.default_rng(21 if kd == "f32" else 22)
    B, N, dk, n_idx, H = 1, 2000, 128, 3, 8
    if kd == "f32":
        keys = rng.standard_normal((N, dk)).astype(np.float32)
        enc = keys
    else:
        keys = L.grid_uniform(rng, (N, dk))
        enc = L.encode(keys, "bf16")
    q = rng.standard_normal((B, n_idx, H, dk)).astype(np.float32)
    w = rng.random((B, n_idx, H)).astype(np.float32)
    kt = to_device(enc[None], kd, DEV)
    s = torch.zeros((B, N), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, "mean")
    got = s.cpu().numpy()[0].astype(np.float64)
    want = oracle.score(enc, kd, q[0], w[0], "mean").astype(np.float64)
    # each indexer score is within 2*dk ulps of its absolute-value score; the mean
    # of three such errors plus the two roundings of the mean itself
    absum = oracle.score(np.abs(keys), "f32", np.abs(q[0]), np.abs(w[0]), "max").astype(np.float64)
    bound = 2 * dk * 2.0 ** -24 * absum + 2 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= bound + 1e-30)
    assert np.mean(got == want) > 0.05     # not a vacuous bound: many agree exactly


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


def run_mx(keys, dtype, q, w, ens, n_valid=None):
    """keys: per-sequence MXKeys; compares every sequence with the oracle, bit for bit."""
    B = len(keys)
    N = keys[0].codes.shape[0]
    codes, scales = to_device(L.stack_keys(keys, dtype), dtype, DEV)
    out = torch.full((B, N), float("nan"), device=DEV)
    lsa.score(codes, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), out, ens, n_valid, key_scales=scales)
    got = out.cpu().numpy()
    for b in range(B):
        nv = N if n_valid is None else n_valid[b]
        want = oracle.score(keys[b], dtype, q[b], w[b], ens, n_valid=nv)
        assert np.array_equal(bits(got[b, :nv]), bits(want)), f"seq {b}: first diff at {np.argmax(bits(got[b,:nv]) != bits(want))}"
        assert np.all(np.isnan(got[b, nv:]))


MX_CASES = [
    # (B, N, dk, n_idx, H, dtype, ensemble)
    (2, 4133, 128, 3, 8, "mxfp4", "max"),
    (3, 300, 64, 2, 5, "mxfp4", "mean"),
    (2, 4133, 128, 3, 8, "mxint8", "max"),
    (1, 777, 32, 4, 8, "mxint8", "mean"),
    (3, 300, 64, 1, 1, "mxint8", "max"),
    (1, 1, 128, 1, 1, "mxfp4", "max"),
]


@pytest.mark.parametrize("case", MX_CASES, ids=[str(c) for c in MX_CASES])
def test_mx_score_matches_oracle(case):
    B, N, dk, n_idx, H, kd, ens = case
    say(f"mx score case {case}")
    rng = np.random.default_rng(zlib.crc32(str(case).encode()))
    keys = [L.mx_keys(rng, N, dk, kd) for _ in range(B)]
    q = L.grid_uniform(rng, (B, n_idx, H, dk))
    w = L.grid_uniform(rng, (B, n_idx, H))
    run_mx(keys, kd, q, w, ens)
    if B > 1:
        run_mx(keys, kd, q, w, ens, n_valid=[N - 1] + [max(0, N // (b + 2)) for b in range(1, B)])


@pytest.mark.parametrize("dk", [64, 128])
def test_mxfp4_every_code_in_every_nibble_and_block(dk):
    """Each E2M1 code alone in each element position, with its block's scale
    varied, decoded through the kernel (score = the element, +0 for zeros)."""
    n = 16 * dk
    codes = np.zeros((n, dk // 2), np.uint8)
    scales = np.full((n, dk // 32), 127, np.uint8)
    idx = np.arange(n)
    pos, code = idx % dk, idx // dk
    codes[idx, pos // 2] = (code << (4 * (pos % 2))).astype(np.uint8)
    scales[idx, pos // 32] = (120 + (idx % 9)).astype(np.uint8)
    q = np.stack([np.ones(dk, np.float32), -np.ones(dk, np.float32)])[None, None]
    w = np.array([[[1.0, -1.0]]], np.float32)
    run_mx([L.MXKeys(codes, scales)], "mxfp4", q, w, "max")


def test_mxint8_every_code_in_every_column():
    dk = 128
    c = np.arange(-128, 128)
    n = c.size * dk
    idx = np.arange(n)
    codes = np.zeros((n, dk), np.int8)
    codes[idx, idx % dk] = c[idx // dk].astype(np.int8)
    scales = (124 + (idx % 5)).astype(np.uint8)[:, None].repeat(dk // 32, axis=1)
    q = np.stack([np.ones(dk, np.float32), -np.ones(dk, np.float32)])[None, None]
    w = np.array([[[1.0, -1.0]]], np.float32)
    run_mx([L.MXKeys(codes, scales)], "mxint8", q, w, "max")


@pytest.mark.parametrize("name", ["thresh_256k", "swap_1m", "swap_1m_fp8", "swap_1m_mxfp4", "swap_1m_mxint8"])
def test_full_size_workload_scores(name):
    wl = L.WORKLOADS[name]
    say(f"full-size score {name}: B={wl.batch} N={wl.n_src}")
    B = wl.batch
    keys = [L.indexer_keys(wl, b) for b in range(B)]
    qw = [L.indexer_query(wl, b, 0) for b in range(B)]
    q = np.stack([x[0] for x in qw])
    w = np.stack([x[1] for x in qw])
    kt = to_device(L.stack_keys(keys, wl.key_dtype), wl.key_dtype, DEV)
    ks = None
    if wl.key_dtype in L.MX_DTYPES:
        kt, ks = kt
    s = torch.zeros((B, wl.n_src), device=DEV)
    lsa.score(kt, torch.from_numpy(q).to(DEV), torch.from_numpy(w).to(DEV), s, wl.ensemble, key_scales=ks)
    got = s.cpu().numpy()
    for b in range(B):
        want = oracle.score(keys[b], wl.key_dtype, q[b], w[b], wl.ensemble)
        assert np.array_equal(bits(got[b]), bits(want)), f"seq {b}"
