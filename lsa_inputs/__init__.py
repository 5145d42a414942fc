"""Seeded synthetic inputs for the LSA decode hot path.

This module only draws numbers and lays them out in memory.  It holds none of
the method's arithmetic: no score, no selection, no LRU, no attention.  Both
the CPU oracle (``oracle/``) and the HIP library (``learned_sparse_kv_amd``)
are fed from here, so that the two sides see bit-identical inputs.

Values are drawn on the 1/8 grid (multiples of 2**-3) so that every dot
product and weighted head sum the scorer forms is exactly representable in
fp32 whatever the summation order.  The shapes follow the pages'
configuration: a 128-token sliding window plus compressed entries of width
512 (FlashMemory 1M context doc, "Memory Layout" in the technical-details
section), compressed capacity ceil(ctx / ratio) for ratios 4 and 128 (same
doc, pinned-memory formula), three memory indexers combined by max or mean
(same doc, FlashMemory configuration), and KVSwap's grouped low-rank keys
(KVSwap article, sections 2.2 and 2.3).
"""
from __future__ import annotations

import dataclasses
import zlib
from typing import NamedTuple, Optional, Tuple

import numpy as np

GRID = 0.125  # 1/8


# --------------------------------------------------------------------------
# random streams
# --------------------------------------------------------------------------
def rng_for(base_seed: int, tag: str, *idx: int) -> np.random.Generator:
    """A PCG64 stream keyed by (base seed, tensor tag, indices...)."""
    key = [int(base_seed) & 0xFFFFFFFF, zlib.crc32(tag.encode())]
    key += [int(i) & 0xFFFFFFFF for i in idx]
    return np.random.default_rng(np.random.SeedSequence(key))


def _fill_chunks(out: np.ndarray, draw, chunk: int = 1 << 23) -> np.ndarray:
    flat = out.reshape(-1)
    for s in range(0, flat.size, chunk):
        e = min(flat.size, s + chunk)
        flat[s:e] = draw(e - s)
    return out


def grid_uniform(rng: np.random.Generator, shape, lo: float = -1.0, hi: float = 1.0,
                 step: float = GRID, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Uniform over the points lo, lo+step, ..., hi (inclusive), float32."""
    n_lo = int(round(lo / step))
    n_hi = int(round(hi / step))
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    st = np.float32(step)

    def draw(n):
        return rng.integers(n_lo, n_hi + 1, size=n, dtype=np.int16).astype(np.float32) * st

    return _fill_chunks(out, draw)


def grid_gauss(rng: np.random.Generator, shape, sigma: float, lo: float = -1.0,
               hi: float = 1.0, step: float = GRID) -> np.ndarray:
    """Gaussian N(0, sigma^2) rounded to the grid and clamped to [lo, hi]."""
    z = rng.standard_normal(size=shape) * sigma
    v = np.clip(np.round(z / step) * step, lo, hi)
    return v.astype(np.float32)


# --------------------------------------------------------------------------
# dtype encodings (exact for grid values; they refuse anything else)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not exactly representable in bfloat16")
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    h = np.asarray(x, dtype=np.float32).astype(np.float16)
    if not np.array_equal(h.astype(np.float32), np.asarray(x, dtype=np.float32)):
        raise ValueError("value not exactly representable in float16")
    return h.view(np.uint16)


def f32_to_fp8_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 byte codes (sign, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 is subnormal, m * 2^-9) of values that the format holds
    exactly: every grid value here does.  Refuses anything else."""
    x = np.asarray(x, dtype=np.float32)
    sign = np.signbit(x).astype(np.uint8) << 7
    a = np.abs(x).astype(np.float64)
    m, e = np.frexp(a)                 # a = m * 2^e, 0.5 <= m < 1 (m = e = 0 for a = 0)
    biased = e + 6                     # a = (2m) * 2^(e - 1), exponent field e - 1 + 7
    normal = a >= 2.0 ** -6            # below: the subnormal range, zero included
    frac = np.where(normal, (2.0 * m - 1.0) * 8.0, a * 512.0)
    field = np.where(normal, biased, 0)
    ok = (frac == np.round(frac)) & (frac >= 0) & (frac < 8) & (field <= 15) & np.isfinite(a)
    ok &= ~((field == 15) & (frac == 7))          # 0x7F / 0xFF are NaN
    if not np.all(ok):
        raise ValueError("value not exactly representable in fp8 e4m3")
    return (sign | (field.astype(np.uint8) << 3) | frac.astype(np.uint8)).astype(np.uint8)


DTYPE_CODES = {"f32": 0, "bf16": 1, "f16": 2, "fp8": 3, "mxfp4": 4, "mxint8": 5}
DTYPE_BYTES = {"f32": 4, "bf16": 2, "f16": 2, "fp8": 1, "mxfp4": 0.5, "mxint8": 1}
MX_DTYPES = ("mxfp4", "mxint8")


class MXKeys(NamedTuple):
    """Keys in an OCP MX format: codes ([N][dk/2] bytes of two E2M1 codes, or
    [N][dk] int8) and one E8M0 scale byte per 32 elements ([N][dk/32])."""
    codes: np.ndarray
    scales: np.ndarray


def mx_keys(rng: np.random.Generator, n: int, dk: int, dtype: str) -> MXKeys:
    """Random MX keys whose every dot product with 1/8-grid queries and weights
    stays exact in fp32: fp4 codes uniform over all 16, scales 2^-3..2^-1 (values
    up to 3 on a 1/16 grid); int8 codes uniform in [-64, 64] (values c/64), scales
    2^-2..1 (values up to 1 on a 1/256 grid)."""
    if dtype == "mxfp4":
        codes = rng.integers(0, 256, size=(n, dk // 2), dtype=np.uint8)
        scales = (127 + rng.integers(-3, 0, size=(n, dk // 32))).astype(np.uint8)
    elif dtype == "mxint8":
        codes = rng.integers(-64, 65, size=(n, dk), dtype=np.int8)
        scales = (127 + rng.integers(-2, 1, size=(n, dk // 32))).astype(np.uint8)
    else:
        raise ValueError(dtype)
    return MXKeys(codes, scales)


def stack_keys(keys: list, dtype: str):
    """Per-sequence keys -> one batch array (an MXKeys of stacked codes and scales)."""
    if dtype in MX_DTYPES:
        return MXKeys(np.stack([k.codes for k in keys]), np.stack([k.scales for k in keys]))
    return np.stack(keys)


def encode(x: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 grid values in the named storage dtype (f32 / bf16 / f16 bits /
    fp8 E4M3 bytes)."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "fp8":
        return f32_to_fp8_e4m3_bits(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
def compressed_cap(ctx: int, ratio: int) -> int:
    return (ctx + ratio - 1) // ratio


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode-step workload: a shared ratio-``src_ratio`` source layer that
    is scored, and ``layer_ratios`` sparse layers that stage and attend."""
    name: str
    base_seed: int
    ctx: int
    batch: int
    src_ratio: int
    layer_ratios: Tuple[int, ...]
    gpu_chunks: int
    cold: str            # "hbm" or "host"
    dk: int
    n_idx: int
    heads: int
    key_dtype: str
    kv_dtype: str
    mode: str            # "topk" or "threshold"
    k: int               # top-k, or the cap in threshold mode
    ensemble: str = "max"
    tau: Optional[float] = None
    steps: int = 16
    window: int = 128
    kv_dim: int = 512
    hq: int = 16
    dist: str = "uniform"     # "uniform" or "planted"
    drift: Optional[float] = None  # fraction of indexer-query coordinates redrawn per step
    # replacement of the swapping pools (KVSwap article §3.2 reading): recency
    # weight in percent for the layers whose ratio is the source ratio (100 =
    # plain LRU), and the high-water mark in percent of the capacity (100 = off)
    recency_w: int = 100
    high_water: int = 100

    @property
    def n_src(self) -> int:
        return compressed_cap(self.ctx, self.src_ratio)

    def layer_cap(self, layer: int) -> int:
        return compressed_cap(self.ctx, self.layer_ratios[layer])

    @property
    def n_layers(self) -> int:
        return len(self.layer_ratios)

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.kv_dim))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# Threshold for the 256K workload: sigmoid of the midpoint between the 1311th and
# 1312th distinct largest step-0 scores pooled over the batch (0.5% of 4 x 65536),
# and the per-step redraw fraction of the 1M workload, chosen so that consecutive
# top-512 sets overlap by about 80%.  Both written by oracle/calibrate_workloads.py.
THRESH_256K_TAU = 0.9999999942439965
SWAP_1M_DRIFT = 0.01875

WORKLOADS = {
    # tiny single-layer step: 8K ctx, ratio 4, 1 indexer x 4 heads x 64, top-64
    "tiny_8k": Workload(
        name="tiny_8k", base_seed=1001, ctx=8192, batch=1, src_ratio=4, layer_ratios=(4,),
        gpu_chunks=2048, cold="hbm", dk=64, n_idx=1, heads=4, key_dtype="f32", kv_dtype="f32",
        mode="topk", k=64, steps=16),
    # 8K ctx, 3-indexer ensemble, ratio-4 + ratio-128 layers, 512-slot LRU pool
    "ens_8k": Workload(
        name="ens_8k", base_seed=1002, ctx=8192, batch=1, src_ratio=4, layer_ratios=(4, 128),
        gpu_chunks=512, cold="hbm", dk=128, n_idx=3, heads=8, key_dtype="f32", kv_dtype="f32",
        mode="topk", k=512, ensemble="max", steps=64),
    # 256K ctx, threshold mode, bf16, batch 4, planted high-score clusters, fully resident
    "thresh_256k": Workload(
        name="thresh_256k", base_seed=1003, ctx=262144, batch=4, src_ratio=4, layer_ratios=(4, 128),
        gpu_chunks=65536, cold="hbm", dk=128, n_idx=3, heads=8, key_dtype="bf16", kv_dtype="bf16",
        mode="threshold", k=512, ensemble="max", tau=THRESH_256K_TAU, steps=64, dist="planted"),
    # 1M ctx, 4 x (ratio-4 + ratio-128) layers, pinned-host cold pools, 1024-slot LRU
    "swap_1m": Workload(
        name="swap_1m", base_seed=1004, ctx=1048576, batch=1, src_ratio=4,
        layer_ratios=(4, 128, 4, 128, 4, 128, 4, 128),
        gpu_chunks=1024, cold="host", dk=128, n_idx=3, heads=8, key_dtype="f32", kv_dtype="f32",
        mode="topk", k=512, ensemble="max", steps=256, drift=SWAP_1M_DRIFT),
}
# the 1M swap workload with its indexer keys stored as OCP fp8 E4M3 bytes: the
# same grid values (exact in E4M3), so the same selections, at a quarter of the
# key bytes
WORKLOADS["swap_1m_fp8"] = WORKLOADS["swap_1m"].replace(name="swap_1m_fp8", key_dtype="fp8")
# ... and in the OCP MX formats (codes and block scales drawn in the format:
# 17.8 and 34.6 MB of keys)
WORKLOADS["swap_1m_mxfp4"] = WORKLOADS["swap_1m"].replace(name="swap_1m_mxfp4", key_dtype="mxfp4")
WORKLOADS["swap_1m_mxint8"] = WORKLOADS["swap_1m"].replace(name="swap_1m_mxint8", key_dtype="mxint8")
# the pages' whole sparse-layer stack (FlashMemory 1M doc, PINNED_MIB worked
# examples and the expected log sparse_layers=41): 20 ratio-4 and 21 ratio-128
# layers, alternating, all served by one selection per step; at 64K context for
# parity (the ratio-4 layers swap from HBM, the ratio-128 ones are resident) and
# at 1M with pinned-host cold pools (11.1 GB)
STACK_41 = tuple([128, 4] * 20 + [128])
WORKLOADS["stack_64k_41"] = WORKLOADS["ens_8k"].replace(name="stack_64k_41", base_seed=1007, ctx=65536,
                                                       layer_ratios=STACK_41, gpu_chunks=1024, drift=0.05)
WORKLOADS["stack_1m_41"] = WORKLOADS["swap_1m"].replace(name="stack_1m_41", layer_ratios=STACK_41)
# the 1M workload with the rolling-buffer replacement: recency and importance
# weighed equally, and at most 70 % of the 1024 slots kept in use after a step
WORKLOADS["swap_1m_wr"] = WORKLOADS["swap_1m"].replace(name="swap_1m_wr", recency_w=50, high_water=70)
# a small one for parity: 8K context, 1024 slots for top-512 (the ratio-4 layer swaps)
WORKLOADS["ens_8k_wr"] = WORKLOADS["ens_8k"].replace(name="ens_8k_wr", gpu_chunks=1024, recency_w=50,
                                                    high_water=70, drift=0.05)


# --------------------------------------------------------------------------
# per-tensor generators
# --------------------------------------------------------------------------
PLANT_RUN = 32        # planted clusters are runs of 32 consecutive entries
PLANT_FRACTION = 0.02  # ... covering 2% of the source entries


def _topic(wl: Workload, b: int) -> np.ndarray:
    return grid_uniform(rng_for(wl.base_seed, "topic", b), (wl.dk,))


def planted_runs(wl: Workload, b: int) -> np.ndarray:
    """Start indices (ascending) of the planted runs of sequence b."""
    n_blocks = wl.n_src // PLANT_RUN
    n_runs = int(round(PLANT_FRACTION * wl.n_src / PLANT_RUN))
    rng = rng_for(wl.base_seed, "runs", b)
    blocks = np.sort(rng.choice(n_blocks, size=n_runs, replace=False))
    return blocks * PLANT_RUN


def indexer_keys_f32(wl: Workload, b: int) -> np.ndarray:
    """Compressed indexer keys of the source layer, [n_src][dk], float32 grid values."""
    rng = rng_for(wl.base_seed, "keys", b)
    if wl.dist == "uniform":
        return grid_uniform(rng, (wl.n_src, wl.dk))
    keys = grid_gauss(rng, (wl.n_src, wl.dk), sigma=0.35)
    topic = _topic(wl, b)
    rng_p = rng_for(wl.base_seed, "plant", b)
    for s in planted_runs(wl, b):
        half = rng_p.random((PLANT_RUN, wl.dk)) < 0.5
        blk = keys[s:s + PLANT_RUN]
        blk[half] = np.broadcast_to(topic, blk.shape)[half]
    return keys


def indexer_keys(wl: Workload, b: int):
    """Keys of sequence b in the workload's key dtype (an MXKeys for the MX dtypes,
    drawn in that format; every other dtype encodes the grid values exactly)."""
    if wl.key_dtype in MX_DTYPES:
        if wl.dist != "uniform":
            raise ValueError("MX keys are drawn for the uniform workloads only")
        return mx_keys(rng_for(wl.base_seed, "keys", b), wl.n_src, wl.dk, wl.key_dtype)
    return encode(indexer_keys_f32(wl, b), wl.key_dtype)


def indexer_query(wl: Workload, b: int, step: int, prev: Optional[np.ndarray] = None):
    """Indexer queries q [n_idx][H][dk] and head weights w [n_idx][H] for one step.

    With ``wl.drift`` set, step t > 0 keeps q of step t-1 and redraws a fraction
    ``drift`` of its coordinates (pass the previous q as ``prev``); w is drawn
    once per sequence."""
    shape_q = (wl.n_idx, wl.heads, wl.dk)
    shape_w = (wl.n_idx, wl.heads)
    if wl.dist == "planted":
        topic = _topic(wl, b)
        noise = grid_gauss(rng_for(wl.base_seed, "qnoise", b, step), shape_q, sigma=0.25)
        q = np.clip(topic[None, None, :] + noise, -1.0, 1.0).astype(np.float32)
        w = grid_uniform(rng_for(wl.base_seed, "w", b, step), shape_w,
                         lo=1.0 / 64, hi=1.0 / 8, step=1.0 / 64)
        return q, w
    if wl.drift is None:
        q = grid_uniform(rng_for(wl.base_seed, "q", b, step), shape_q)
        w = grid_uniform(rng_for(wl.base_seed, "w", b, step), shape_w)
        return q, w
    w = grid_uniform(rng_for(wl.base_seed, "w", b, 0), shape_w)
    if step == 0:
        return grid_uniform(rng_for(wl.base_seed, "q", b, 0), shape_q), w
    if prev is None:
        raise ValueError("a drifting query needs the previous step's q")
    rng = rng_for(wl.base_seed, "q", b, step)
    redraw = rng.random(shape_q) < wl.drift
    fresh = grid_uniform(rng, shape_q)
    return np.where(redraw, fresh, prev).astype(np.float32), w


def window_rows(wl: Workload, layer: int, b: int) -> np.ndarray:
    """Sliding-window KV rows [W][D] (float32 grid values)."""
    return grid_uniform(rng_for(wl.base_seed, "window", layer, b), (wl.window, wl.kv_dim))


def cold_rows(wl: Workload, layer: int, b: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """All compressed KV entries of one sparse layer [cap][D] (float32 grid values).
    ``out`` may be any float32 buffer of that shape (e.g. pinned host memory)."""
    cap = wl.layer_cap(layer)
    return grid_uniform(rng_for(wl.base_seed, "cold", layer, b), (cap, wl.kv_dim), out=out)


def attn_query(wl: Workload, layer: int, b: int, step: int) -> np.ndarray:
    """Attention queries [Hq][D] of one sparse layer for one step."""
    return grid_uniform(rng_for(wl.base_seed, "aq", layer, b, step), (wl.hq, wl.kv_dim))


# the decode token's hidden state and the indexers' projection weights: the
# hidden width of the pages' model (hidden[4096]); weights on a 1/512 grid in
# [-1/64, 1/64], so every product is a multiple of 2^-12 and every partial sum
# of a projected value (at most 64 in magnitude) is exact in fp32
D_MODEL = 4096
PROJ_STEP = 1.0 / 512
PROJ_MAX = 1.0 / 64


def projection_weights(wl: Workload, d_model: int = D_MODEL):
    """wq [n_idx][H][dk][d_model] and ww [n_idx][H][d_model], float32 grid values."""
    wq = grid_uniform(rng_for(wl.base_seed, "wq"), (wl.n_idx, wl.heads, wl.dk, d_model),
                      lo=-PROJ_MAX, hi=PROJ_MAX, step=PROJ_STEP)
    ww = grid_uniform(rng_for(wl.base_seed, "ww"), (wl.n_idx, wl.heads, d_model),
                      lo=-PROJ_MAX, hi=PROJ_MAX, step=PROJ_STEP)
    return wq, ww


def hidden_state(wl: Workload, b: int, step: int, d_model: int = D_MODEL) -> np.ndarray:
    """The decode token's hidden state [d_model] of sequence b at a step, on the 1/8 grid."""
    return grid_uniform(rng_for(wl.base_seed, "hidden", b, step), (d_model,))


def indexer_query_steps(wl: Workload, b: int, steps: int):
    """Indexer queries of steps 0..steps-1, as (q [steps][n_idx][H][dk], w [steps][n_idx][H])."""
    qs, ws = [], []
    prev = None
    for t in range(steps):
        q, w = indexer_query(wl, b, t, prev)
        qs.append(q)
        ws.append(w)
        prev = q
    return np.stack(qs), np.stack(ws)


# --------------------------------------------------------------------------
# KVSwap grouped low-rank keys (KVSwap article, sections 2.2-2.3 and 3.2)
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class KVSwapWorkload:
    """Grouped low-rank key prediction: ``layers`` x ``groups`` groups of
    ``group_heads`` KV heads of width ``head_dim`` per sequence; a group's keys
    over ``ctx`` positions are given as factors U [ctx][rank], S [rank],
    V [C][rank] (C = group_heads * head_dim); top ``k`` positions per group are
    staged into a ``slots``-slot LRU pool and attended per head over full K/V.

    Segment s = (layer * groups + group) * batch + b.  The cold K/V rows of a
    (group, sequence) are shared by all layers (one synthetic store; see the
    design notes), each row being [K of the group's heads | V of the group's
    heads] in f16."""
    name: str
    base_seed: int
    ctx: int
    batch: int
    layers: int
    groups: int
    k: int
    slots: int
    group_heads: int = 4
    head_dim: int = 128
    rank: int = 32
    kv_dtype: str = "f16"
    steps: int = 8
    drift: Optional[float] = None
    recency_w: int = 100      # replacement weighting, percent (100 = plain LRU)
    high_water: int = 100     # slots kept in use after a step, percent of the 400 (100 = off)

    @property
    def C(self) -> int:
        return self.group_heads * self.head_dim

    @property
    def n_pools(self) -> int:
        return self.layers * self.groups

    @property
    def n_seg(self) -> int:
        return self.n_pools * self.batch

    @property
    def row_elems(self) -> int:
        return 2 * self.C

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    def seg(self, layer: int, group: int, b: int) -> int:
        return (layer * self.groups + group) * self.batch + b

    def replace(self, **kw) -> "KVSwapWorkload":
        return dataclasses.replace(self, **kw)


KVSWAP_WORKLOADS = {
    # small case the oracle finishes in seconds: 2 sequences x 2 layers x 2 groups
    "kvswap_small": KVSwapWorkload(name="kvswap_small", base_seed=1005, ctx=2048, batch=2, layers=2, groups=2,
                                   k=400, slots=400, steps=6, drift=0.05),
    # the article's shape: 32K ctx, batch 16, 32 layers x 8 groups of 4 heads x 128, rank 32, top-400
    "kvswap_32k": KVSwapWorkload(name="kvswap_32k", base_seed=1006, ctx=32768, batch=16, layers=32, groups=8,
                                 k=400, slots=400, steps=16, drift=0.05),
}
# the rolling buffer of the article's section 3.2: 400 slots per group, the
# replacement weighing recency and importance equally, at most 70 % of the
# slots in use after a step; each step keeps its top 200, so the buffer holds
# earlier entries too and the weighting decides which of them stay
KVSWAP_WORKLOADS["kvswap_small_wr"] = dataclasses.replace(KVSWAP_WORKLOADS["kvswap_small"], name="kvswap_small_wr",
                                                          k=200, recency_w=50, high_water=70)
KVSWAP_WORKLOADS["kvswap_32k_wr"] = dataclasses.replace(KVSWAP_WORKLOADS["kvswap_32k"], name="kvswap_32k_wr",
                                                        k=200, recency_w=50, high_water=70)

HALF = 0.5


def grid_codes(rng: np.random.Generator, shape, n_points: int) -> np.ndarray:
    """uint8 codes uniform on 0..n_points-1 (n_points a power of two <= 256),
    taken from the low bits of raw random bytes; much cheaper than
    ``grid_uniform`` for the multi-GiB KVSwap tensors."""
    assert n_points & (n_points - 1) == 0 and 2 <= n_points <= 256
    n = int(np.prod(shape))
    return (np.frombuffer(rng.bytes(n), dtype=np.uint8) & np.uint8(n_points - 1)).reshape(shape)


# KVSwap tensors are stored as codes: value = (code - offset) / 8
U_POINTS, U_OFFSET = 8, 4          # U, V on {-1/2, ..., 3/8}
KV_POINTS, KV_OFFSET = 16, 8       # cold K/V on {-1, ..., 7/8}


def codes_to_f32(codes: np.ndarray, offset: int) -> np.ndarray:
    return (codes.astype(np.float32) - np.float32(offset)) * np.float32(GRID)


def code_table_f16(n_points: int, offset: int) -> np.ndarray:
    """f16 bit patterns of the code values, indexed by code."""
    return f32_to_f16_bits((np.arange(n_points, dtype=np.float32) - offset) * np.float32(GRID))


def lowrank_U_codes(wl: KVSwapWorkload, layer: int, group: int, b: int) -> np.ndarray:
    return grid_codes(rng_for(wl.base_seed, "U", layer, group, b), (wl.ctx, wl.rank), U_POINTS)


def lowrank_U(wl: KVSwapWorkload, layer: int, group: int, b: int) -> np.ndarray:
    """U [ctx][rank], 1/8 grid on [-1/2, 3/8] (float32 values)."""
    return codes_to_f32(lowrank_U_codes(wl, layer, group, b), U_OFFSET)


def lowrank_S(wl: KVSwapWorkload, layer: int, group: int, b: int) -> np.ndarray:
    """Singular values S [rank] on the 1/8 grid in [0, 1/2], float32."""
    return grid_uniform(rng_for(wl.base_seed, "S", layer, group, b), (wl.rank,), lo=0.0, hi=HALF)


def lowrank_V_codes(wl: KVSwapWorkload, layer: int, group: int, b: int) -> np.ndarray:
    return grid_codes(rng_for(wl.base_seed, "V", layer, group, b), (wl.C, wl.rank), U_POINTS)


def lowrank_V(wl: KVSwapWorkload, layer: int, group: int, b: int) -> np.ndarray:
    """V [C][rank], 1/8 grid on [-1/2, 3/8] (float32 values)."""
    return codes_to_f32(lowrank_V_codes(wl, layer, group, b), U_OFFSET)


def kvswap_query(wl: KVSwapWorkload, layer: int, group: int, b: int, step: int,
                 prev: Optional[np.ndarray] = None) -> np.ndarray:
    """The group's query [C] (its heads' queries concatenated), 1/8 grid in
    [-1/2, 1/2].  With ``wl.drift`` set, step t > 0 redraws that fraction of the
    previous step's coordinates."""
    rng = rng_for(wl.base_seed, "kq", layer, group, b, step)
    fresh = grid_uniform(rng, (wl.C,), lo=-HALF, hi=HALF)
    if wl.drift is None or step == 0:
        return fresh
    if prev is None:
        raise ValueError("a drifting query needs the previous step's q")
    redraw = rng.random(wl.C) < wl.drift
    return np.where(redraw, fresh, prev).astype(np.float32)


def kvswap_query_steps(wl: KVSwapWorkload, layer: int, group: int, b: int, steps: int) -> np.ndarray:
    out, prev = [], None
    for t in range(steps):
        prev = kvswap_query(wl, layer, group, b, t, prev)
        out.append(prev)
    return np.stack(out)


def kvswap_cold_codes(wl: KVSwapWorkload, group: int, b: int) -> np.ndarray:
    return grid_codes(rng_for(wl.base_seed, "kvcold", group, b), (wl.ctx, wl.row_elems), KV_POINTS)


def kvswap_cold(wl: KVSwapWorkload, group: int, b: int) -> np.ndarray:
    """Full-precision K/V rows of one (group, sequence) [ctx][2*C] (float32 values
    on the 1/8 grid in [-1, 7/8]): the group's heads' keys, then their values."""
    return codes_to_f32(kvswap_cold_codes(wl, group, b), KV_OFFSET)
