"""Pins of oracle.score (indexer scoring + ensemble) against a hand-worked
example, exact rational brute force, and special cases with closed forms."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import lsa_inputs as L
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "score_hand.json")))


def round_f32(x: Fraction) -> np.float32:
    """Round a rational to the nearest float32 (ties to even), exactly."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def brute_score(keys, q, w, ens):
    """Exact rational score of every key; the mean is the float sum divided once."""
    n_idx, H, dk = q.shape
    out = []
    for k in keys:
        s = []
        for i in range(n_idx):
            acc = Fraction(0)
            for h in range(H):
                d = sum(Fraction(float(q[i, h, t])) * Fraction(float(k[t])) for t in range(dk))
                acc += Fraction(float(w[i, h])) * max(d, Fraction(0))
            s.append(round_f32(acc))
        if ens == "max":
            out.append(max(s))
        else:
            tot = round_f32(sum(Fraction(float(v)) for v in s))
            out.append(round_f32(Fraction(float(tot)) / n_idx))
    return np.array(out, np.float32)


def test_hand_example():
    keys = np.array(GOLD["keys"], np.float32)
    q = np.array(GOLD["q"], np.float32)
    w = np.array(GOLD["w"], np.float32)
    for ens in ("max", "mean"):
        e = oracle.score(keys, "f32", q, w, ens)
        assert e.tolist() == GOLD[ens], ens


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_grid(seed):
    rng = np.random.default_rng(seed)
    n_idx, H, dk, N = rng.integers(1, 4), rng.integers(1, 4), rng.integers(1, 9), rng.integers(1, 25)
    keys = L.grid_uniform(rng, (N, dk))
    q = L.grid_uniform(rng, (n_idx, H, dk))
    w = L.grid_uniform(rng, (n_idx, H))
    for ens in ("max", "mean"):
        got = oracle.score(keys, "f32", q, w, ens)
        want = brute_score(keys, q, w, ens)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), ens


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_general_floats(seed):
    # arbitrary fp32 inputs: the double-accumulated oracle is within one float ulp
    # of the exact rational result
    rng = np.random.default_rng(100 + seed)
    n_idx, H, dk, N = 3, 3, 7, 16
    keys = rng.standard_normal((N, dk)).astype(np.float32)
    q = rng.standard_normal((n_idx, H, dk)).astype(np.float32)
    w = rng.standard_normal((n_idx, H)).astype(np.float32)
    for ens in ("max", "mean"):
        got = oracle.score(keys, "f32", q, w, ens)
        want = brute_score(keys, q, w, ens)
        ulp = np.spacing(np.abs(want)).astype(np.float64)
        assert np.all(np.abs(got.astype(np.float64) - want) <= ulp + 1e-30)


def test_single_positive_head_is_matmul():
    # one indexer, one head, weight 1, all-positive operands: the score is q.k,
    # i.e. a matrix-vector product
    rng = np.random.default_rng(7)
    keys = L.grid_uniform(rng, (300, 64), lo=0.125, hi=1.0)
    q = L.grid_uniform(rng, (1, 1, 64), lo=0.125, hi=1.0)
    w = np.ones((1, 1), np.float32)
    got = oracle.score(keys, "f32", q, w)
    want = (keys.astype(np.float64) @ q[0, 0].astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, want)


def test_relu_clips_negative_dots():
    # all dots negative -> every head contributes 0 -> score +0 (sign bit clear)
    rng = np.random.default_rng(8)
    keys = L.grid_uniform(rng, (50, 16), lo=0.125, hi=1.0)
    q = -L.grid_uniform(rng, (2, 3, 16), lo=0.125, hi=1.0)
    w = -np.ones((2, 3), np.float32)  # negative weights times 0 give -0
    for ens in ("max", "mean"):
        e = oracle.score(keys, "f32", q, w, ens)
        assert np.all(e.view(np.uint32) == 0), ens


def test_identical_indexers_ensemble_agree():
    rng = np.random.default_rng(9)
    keys = L.grid_uniform(rng, (200, 32))
    q1 = L.grid_uniform(rng, (1, 4, 32))
    w1 = L.grid_uniform(rng, (1, 4))
    one = oracle.score(keys, "f32", q1, w1)
    q3, w3 = np.repeat(q1, 3, 0), np.repeat(w1, 3, 0)
    assert np.array_equal(oracle.score(keys, "f32", q3, w3, "max"), one)
    assert np.array_equal(oracle.score(keys, "f32", q3, w3, "mean"), one)


def test_max_ensemble_is_max_of_single_indexers():
    rng = np.random.default_rng(10)
    keys = L.grid_uniform(rng, (200, 32))
    q = L.grid_uniform(rng, (3, 4, 32))
    w = L.grid_uniform(rng, (3, 4))
    singles = np.stack([oracle.score(keys, "f32", q[i:i + 1], w[i:i + 1]) for i in range(3)])
    assert np.array_equal(oracle.score(keys, "f32", q, w, "max"), singles.max(0) + np.float32(0))
    mean = ((singles[0] + singles[1]) + singles[2]) / np.float32(3)  # exact sums on the grid
    assert np.array_equal(oracle.score(keys, "f32", q, w, "mean"), mean.astype(np.float32))


def test_weights_scale_linearly():
    rng = np.random.default_rng(11)
    keys = L.grid_uniform(rng, (100, 16))
    q = L.grid_uniform(rng, (2, 3, 16))
    w = L.grid_uniform(rng, (2, 3))
    assert np.array_equal(oracle.score(keys, "f32", q, 2 * w), 2 * oracle.score(keys, "f32", q, w))


def test_key_permutation_permutes_scores():
    rng = np.random.default_rng(12)
    keys = L.grid_uniform(rng, (120, 16))
    q = L.grid_uniform(rng, (3, 2, 16))
    w = L.grid_uniform(rng, (3, 2))
    perm = rng.permutation(120)
    assert np.array_equal(oracle.score(keys[perm], "f32", q, w), oracle.score(keys, "f32", q, w)[perm])


def test_bf16_and_f16_storage_decode():
    rng = np.random.default_rng(13)
    keys = L.grid_uniform(rng, (64, 16))
    q = L.grid_uniform(rng, (3, 8, 16))
    w = L.grid_uniform(rng, (3, 8))
    ref = oracle.score(keys, "f32", q, w)
    assert np.array_equal(oracle.score(L.f32_to_bf16_bits(keys), "bf16", q, w), ref)
    assert np.array_equal(oracle.score(L.f32_to_f16_bits(keys), "f16", q, w), ref)
    # f16 decode incl. subnormals: one positive key element, q = w = 1 -> the value itself
    vals = np.array([6.1e-5, 5.96e-8, 1.0, 0.333, 65504.0, 2.0 ** -20], np.float16)
    e = oracle.score(vals.view(np.uint16).reshape(-1, 1), "f16", np.ones((1, 1, 1), np.float32),
                     np.ones((1, 1), np.float32))
    assert np.array_equal(e, vals.astype(np.float32))


def test_fp8_e4m3_storage_decode():
    """Every finite OCP E4M3 code decodes to torch's float8_e4m3fn value and to
    the format's defining values; grid keys stored as fp8 score as in fp32."""
    import torch
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    one = np.ones((1, 1), np.float32)
    pos = oracle.score(codes.reshape(-1, 1), "fp8", np.ones((1, 1, 1), np.float32), one)
    neg = oracle.score(codes.reshape(-1, 1), "fp8", -np.ones((1, 1, 1), np.float32), one)
    dec = (pos - neg).astype(np.float64)          # ReLU(k) - ReLU(-k) = k
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(dec, want)
    by_code = dict(zip(codes.tolist(), dec.tolist()))
    # subnormals m * 2^-9, smallest normal 2^-6, 1.0, the largest finite 448
    assert by_code[0x01] == 2.0 ** -9 and by_code[0x07] == 7 * 2.0 ** -9
    assert by_code[0x08] == 2.0 ** -6 and by_code[0x38] == 1.0 and by_code[0xB8] == -1.0
    assert by_code[0x7E] == 448.0 and by_code[0x33] == 0.6875
    rng = np.random.default_rng(15)
    keys = L.grid_uniform(rng, (64, 16))
    q = L.grid_uniform(rng, (3, 8, 16))
    w = L.grid_uniform(rng, (3, 8))
    assert np.array_equal(oracle.score(L.f32_to_fp8_e4m3_bits(keys), "fp8", q, w), oracle.score(keys, "f32", q, w))


# OCP MX specification: the E2M1 magnitudes of codes 0..7 (code 8..15: the negatives)
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _element_values(keys, dtype, dk):
    """Every key holds one nonzero element: with two heads (q = +1 and -1 everywhere,
    w = +1 and -1) the score is ReLU(x) - ReLU(-x) = x, the decoded element."""
    q = np.stack([np.ones(dk, np.float32), -np.ones(dk, np.float32)])[None]
    w = np.array([[1.0, -1.0]], np.float32)
    return oracle.score(keys, dtype, q, w).astype(np.float64)


def test_mxfp4_decode_every_code_nibble_and_block():
    dk = 64
    codes, scales, want = [], [], []
    for code in range(16):
        for pos in (0, 1, 33, 63):             # low and high nibble; first and second block
            for s in (1, 120, 127, 131, 250):
                row = np.zeros(dk // 2, np.uint8)
                row[pos // 2] = code << (4 * (pos % 2))
                sc = np.full(dk // 32, 127, np.uint8)
                sc[pos // 32] = s
                codes.append(row)
                scales.append(sc)
                want.append((-1.0 if code & 8 else 1.0) * E2M1[code & 7] * 2.0 ** (s - 127))
    got = _element_values((np.array(codes), np.array(scales)), "mxfp4", dk)
    assert np.array_equal(got, np.array(want, np.float32).astype(np.float64))


def test_e8m0_scale_decode_against_torch():
    import torch
    s = np.arange(0, 255, dtype=np.uint8)
    codes = np.zeros((s.size, 16), np.uint8)
    codes[:, 0] = 2                            # E2M1 code 2 is 1.0
    got = _element_values((codes, s.reshape(-1, 1)), "mxfp4", 32)
    want = torch.from_numpy(s.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(got, want.astype(np.float32).astype(np.float64))


def test_mxint8_decode_every_code():
    dk = 32
    c = np.arange(-128, 128, dtype=np.int64)
    codes = np.zeros((c.size * 2, dk), np.int8)
    codes[:c.size, 5] = c
    codes[c.size:, 31] = c
    scales = np.concatenate([np.full((c.size, 1), 127), np.full((c.size, 1), 124)]).astype(np.uint8)
    got = _element_values((codes, scales), "mxint8", dk)
    want = np.concatenate([c / 64.0, c / 64.0 * 2.0 ** -3])
    assert np.array_equal(got, want)


def test_mx_encodings_of_grid_values_score_as_f32():
    rng = np.random.default_rng(16)
    dk = 128
    q = L.grid_uniform(rng, (3, 8, dk))
    w = L.grid_uniform(rng, (3, 8))
    # MX INT8 with scale 1: code = 64 * value for every 1/8-grid value in [-1, 1]
    v = L.grid_uniform(rng, (50, dk))
    i8 = (v * 64).astype(np.int8)
    ref = oracle.score(v, "f32", q, w)
    assert np.array_equal(oracle.score((i8, np.full((50, dk // 32), 127, np.uint8)), "mxint8", q, w), ref)
    # MX FP4 with scale 1/4: the grid values 4 * E2M1 covers
    mags = np.array([0.0, 0.125, 0.25, 0.375, 0.5, 0.75, 1.0])
    v = (mags[rng.integers(0, mags.size, (50, dk))] * rng.choice([-1.0, 1.0], (50, dk))).astype(np.float32)
    nib = np.array([E2M1.index(abs(x) * 4) | (8 if x < 0 else 0) for x in v.ravel()], np.uint8).reshape(50, dk)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    ref = oracle.score(v, "f32", q, w)
    assert np.array_equal(oracle.score((packed, np.full((50, dk // 32), 125, np.uint8)), "mxfp4", q, w), ref)


def test_n_valid_prefix():
    rng = np.random.default_rng(14)
    keys = L.grid_uniform(rng, (100, 16))
    q = L.grid_uniform(rng, (1, 2, 16))
    w = L.grid_uniform(rng, (1, 2))
    assert np.array_equal(oracle.score(keys, "f32", q, w, n_valid=37), oracle.score(keys[:37], "f32", q, w))
